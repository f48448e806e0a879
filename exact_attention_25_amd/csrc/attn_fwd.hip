// Forward attention kernels for gfx950.
//
// O = softmax(Q K^T * scale + mask) V, computed tile by tile with an online
// softmax, and LSE per row -- the tiled double loop and running (m, l) of
// "FlashAttention技术解析：优化Transformer注意力计算效率"
// (jsqmd.com/news/722897) §2.2, with the single final normalisation of its
// §4.1 and fp32 statistics / 16-bit matrix products of its §6.3.
//
// Work decomposition: one work-group per (batch, q-head, block of
// NW*QB*32 query rows); the block's query tile stays in registers while
// K/V tiles of BC keys stream through LDS (double-buffered, filled by
// direct global->LDS loads).  Each wave owns QB*32 query rows.
//
// Per KV tile and wave:
//   S^T = K_j Q^T        32x32x16 MFMA, A = K from LDS, B = Q from registers;
//                        each lane ends up holding 16 keys of one query, so
//                        the row maximum is a per-lane max plus one swap
//                        between the two lane halves.
//   online softmax       in base 2: t = s * scale * log2(e) (+ mask*log2(e));
//                        p = exp2(t - m).  The reference point m is moved
//                        only when a tile's maximum exceeds it by more than
//                        TH (then O and l are rescaled); otherwise p <= 2^TH.
//                        In exact arithmetic the result does not depend on
//                        m; it only bounds the range of p.
//   O^T += V_j^T P^T     32x32x16 MFMA, A = V^T read transposed from the
//                        row-major LDS tile, B = P^T straight from the S^T
//                        registers (keys are matched slot by slot).
// Epilogue: O /= l (one reciprocal per row), round to the output type,
// LSE = ln2 * (m + log2 l).
#include "attn_kernels.h"
#include "device_common.h"

namespace attn {

constexpr float kRescaleThreshold = 8.0f;  // log2 units: p stays <= 256

template <class E, int D, int QB, int NW, int BC, bool CAUSAL, bool MASK>
struct FwdKernel {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE_BYTES = BC * D * 2;     // one K or V tile
  static constexpr int ROWS = NW * QB * 32;         // query rows per block
  static constexpr int SLOTS_PER_WAVE = BC * CPR / (NW * 64);  // dma per tensor
  static constexpr int KB = BC / 32;                // 32-key blocks per tile
  static constexpr int KS = D / 16;                 // k-steps of QK^T
  static constexpr int DT = D / 32;                 // 32-wide d tiles of O
  static constexpr int PT = BC / 16;                // k-steps of PV
  static_assert(BC * CPR % (NW * 64) == 0, "tile must split evenly into DMA slots");

  using T = typename E::T;
  using V8 = typename E::V8;
  using V4 = typename E::V4;

  // Issue the direct loads of one K tile and one V tile (keys j0..j0+BC-1).
  // Rows beyond the last key and chunks beyond the head dimension are
  // clamped onto valid memory: the extra keys are masked to -inf and the
  // extra K columns meet zero Q columns, so their (finite) values never
  // reach the result.
  static __device__ __forceinline__ void issue_tile(const T* kp, const T* vp, int64_t k_sn,
                                                    int64_t v_sn, int j0, int nk, int dchunks,
                                                    char* kbuf, char* vbuf, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < SLOTS_PER_WAVE; ++i) {
      const int slot0 = (i * NW + wave) * 64;
      const int s = slot0 + lane;
      const int row = s / CPR;
      const int p = s % CPR;
      const int grow = min(j0 + row, nk - 1);
      const int ck = min(p ^ swz_k<CPR>(row), dchunks - 1);
      const int cv = min(p ^ swz_v<CPR>(row), dchunks - 1);
      dma16(kp + grow * k_sn + ck * 8, kbuf + slot0 * 16);
      dma16(vp + grow * v_sn + cv * 8, vbuf + slot0 * 16);
    }
  }

  static __device__ __forceinline__ void run(const FwdArgs& a, char* k0, char* v0, char* k1,
                                             char* v1) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5;   // lane half
    const int l32 = lane & 31;

    int wid = xcd_remap(blockIdx.x, a.total_blocks);
    int qblk = wid % a.nqb;
    const int bh = wid / a.nqb;
    const int h = bh % a.Hq;
    const int b = bh / a.Hq;
    if (CAUSAL) qblk = a.nqb - 1 - qblk;  // longest rows first
    const int g = h / a.group;
    const int q_blk0 = qblk * ROWS;
    const int q_w0 = q_blk0 + wave * QB * 32;

    int kv_limit = a.Nk;
    if (a.kv_lens) kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
    int kv_end = kv_limit;
    if (CAUSAL) kv_end = min(kv_end, min(q_blk0 + ROWS, a.Nq));
    const int n_tiles = (kv_end + BC - 1) / BC;
    const int dchunks = a.d / 8;

    const T* qp = (const T*)a.q + b * a.q_sb + h * a.q_sh;
    const T* kp = (const T*)a.k + b * a.k_sb + g * a.k_sh;
    const T* vp = (const T*)a.v + b * a.v_sb + g * a.v_sh;

    // Query fragments (B operand of S^T = K Q^T), zero beyond d.
    V8 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = min(q_w0 + qb * 32 + l32, a.Nq - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + hl * 8;
        if (d0 < a.d)
          qf[qb][ks] = *(const V8*)(qp + row * a.q_sn + d0);
        else
          qf[qb][ks] = V8{};
      }
    }

    f32x16 acc[QB][DT];
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_run[qb] = -INFINITY;
      l_run[qb] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[qb][dt] = f32x16{};
    }

    if (n_tiles > 0)
      issue_tile(kp, vp, a.k_sn, a.v_sn, 0, a.Nk, dchunks, k0, v0, wave, lane);

    for (int j = 0; j < n_tiles; j += 2) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (j + 1 < n_tiles)
        issue_tile(kp, vp, a.k_sn, a.v_sn, (j + 1) * BC, a.Nk, dchunks, k1, v1, wave, lane);
      tile(a, k0, v0, j * BC, kv_limit, q_w0, b, h, qf, acc, m_run, l_run);
      if (j + 1 >= n_tiles) break;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (j + 2 < n_tiles)
        issue_tile(kp, vp, a.k_sn, a.v_sn, (j + 2) * BC, a.Nk, dchunks, k0, v0, wave, lane);
      tile(a, k1, v1, (j + 1) * BC, kv_limit, q_w0, b, h, qf, acc, m_run, l_run);
    }

    // Epilogue.
    T* op = (T*)a.o + b * a.o_sb + h * a.o_sh;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = add_with_other_half(l_run[qb]);
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      const int row = q_w0 + qb * 32 + l32;
      if (row < a.Nq) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int col = dt * 32 + gq * 8 + hl * 4;
            if (col < a.d) {
              auto lo = E::cvt2(acc[qb][dt][gq * 4 + 0] * inv, acc[qb][dt][gq * 4 + 1] * inv);
              auto hi = E::cvt2(acc[qb][dt][gq * 4 + 2] * inv, acc[qb][dt][gq * 4 + 3] * inv);
              V4 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
              *(V4*)(op + row * a.o_sn + col) = w;
            }
          }
        }
        if (hl == 0)
          a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] =
              l_tot > 0.f ? (m_run[qb] + fast_log2(l_tot)) * kLn2 : -INFINITY;
      }
    }
  }

  static __device__ __forceinline__ void tile(const FwdArgs& a, const char* kbuf, const char* vbuf,
                                              int j0, int kv_limit, int q_w0, int b, int h,
                                              const V8 (&qf)[QB][KS], f32x16 (&acc)[QB][DT],
                                              float (&m_run)[QB], float (&l_run)[QB]) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;

    // S^T = K_j Q^T
    f32x16 s[QB][KB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int row = kb * 32 + l32;
        const int c = (ks * 2 + hl) ^ swz_k<CPR>(row);
        const V8 kf = lds_read16<V8>(kbuf + row * (D * 2) + c * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = E::mfma(kf, qf[qb][ks], s[qb][kb]);
      }
    }

    const bool edge = (j0 + BC > kv_limit) || (CAUSAL && j0 + BC - 1 > q_w0);
    V8 pf[QB][PT];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = q_w0 + qb * 32 + l32;
      if constexpr (MASK) {
        const int mrow = min(qrow, a.Nq - 1);
        const float* mp = a.mask + b * a.m_sb + h * a.m_sh + (int64_t)mrow * a.m_sq;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + kb * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
            const float mv = mp[min(key, a.Nk - 1)];
            s[qb][kb][r] = s[qb][kb][r] * a.c + mv * kLog2e;
          }
      }
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + kb * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
            const bool dead = key >= kv_limit || (CAUSAL && key > qrow);
            if (dead) s[qb][kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      mx = max_with_other_half(mx);
      const float cand = MASK ? mx : mx * a.c;
      const bool need = cand > m_run[qb] + kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = fmaxf(m_run[qb], cand);
        const float alpha = (m_run[qb] == -INFINITY) ? 0.f : fast_exp2(m_run[qb] - m_new);
        if (m_new != -INFINITY) {
          l_run[qb] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[qb][dt] *= alpha;
          m_run[qb] = m_new;
        }
      }
      const float mref = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float t = MASK ? (s[qb][kb][r] - mref) : __builtin_fmaf(s[qb][kb][r], a.c, -mref);
          const float p = fast_exp2(t);
          s[qb][kb][r] = p;
          lsum += p;
        }
      l_run[qb] += lsum;
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        const int kb = t >> 1, r0 = (t & 1) * 8;
        auto p01 = E::cvt2(s[qb][kb][r0 + 0], s[qb][kb][r0 + 1]);
        auto p23 = E::cvt2(s[qb][kb][r0 + 2], s[qb][kb][r0 + 3]);
        auto p45 = E::cvt2(s[qb][kb][r0 + 4], s[qb][kb][r0 + 5]);
        auto p67 = E::cvt2(s[qb][kb][r0 + 6], s[qb][kb][r0 + 7]);
        V4 lo = __builtin_shufflevector(p01, p23, 0, 1, 2, 3);
        V4 hi = __builtin_shufflevector(p45, p67, 0, 1, 2, 3);
        pf[qb][t] = concat4<V8, V4>(lo, hi);
      }
    }

    // O^T += V_j^T P^T
    const int grp = lane >> 4, gi = lane & 15;
#pragma unroll
    for (int t = 0; t < PT; ++t) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int row = t * 16 + 4 * (grp >> 1) + (gi >> 2);
        const int col = dt * 32 + 16 * (grp & 1) + 4 * (gi & 3);
        const int chunk = col >> 3, within = (col & 7) * 2;
        const V4 lo = lds_read_tr4<V4>(vbuf + row * (D * 2) + ((chunk ^ swz_v<CPR>(row)) << 4) + within);
        const int row2 = row + 8;
        const V4 hi = lds_read_tr4<V4>(vbuf + row2 * (D * 2) + ((chunk ^ swz_v<CPR>(row2)) << 4) + within);
        const V8 vf = concat4<V8, V4>(lo, hi);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][dt] = E::mfma(vf, pf[qb][t], acc[qb][dt]);
      }
    }
  }
};

template <class E, int D, int QB, int NW, int BC, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(FwdArgs a) {
  using K = FwdKernel<E, D, QB, NW, BC, CAUSAL, MASK>;
  __shared__ __attribute__((aligned(1024))) char k0[K::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[K::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[K::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[K::TILE_BYTES];
  K::run(a, k0, v0, k1, v1);
}

template <class E, int D, int QB, int NW, int BC>
static hipError_t launch_fwd_t(const FwdArgs& a0, bool causal, bool mask, hipStream_t st) {
  FwdArgs a = a0;
  constexpr int ROWS = NW * QB * 32;
  a.nqb = (a.Nq + ROWS - 1) / ROWS;
  a.total_blocks = a.B * a.Hq * a.nqb;
  dim3 grid(a.total_blocks), block(NW * 64);
  if (causal) {
    if (mask) hipLaunchKernelGGL((fwd_kernel<E, D, QB, NW, BC, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<E, D, QB, NW, BC, true, false>), grid, block, 0, st, a);
  } else {
    if (mask) hipLaunchKernelGGL((fwd_kernel<E, D, QB, NW, BC, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<E, D, QB, NW, BC, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <class E>
static hipError_t launch_fwd_e(const FwdArgs& a, bool causal, bool mask, hipStream_t st) {
  if (a.d > 64) return launch_fwd_t<E, 128, 1, 4, 64>(a, causal, mask, st);
  return launch_fwd_t<E, 64, 1, 4, 64>(a, causal, mask, st);
}

hipError_t launch_fwd16(const FwdArgs& a, bool is_bf16, bool causal, bool mask, hipStream_t st) {
  if (a.total_blocks < 0) return hipErrorInvalidValue;
  return is_bf16 ? launch_fwd_e<BF16>(a, causal, mask, st) : launch_fwd_e<FP16>(a, causal, mask, st);
}

}  // namespace attn
