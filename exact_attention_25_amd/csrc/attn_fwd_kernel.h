// Forward attention kernel for gfx950 (16-bit inputs).
//
// O = softmax(Q K^T * scale + mask) V, computed tile by tile with an online
// softmax, and LSE per row -- the tiled double loop and running (m, l) of
// "FlashAttention技术解析：优化Transformer注意力计算效率"
// (jsqmd.com/news/722897) §2.2, with the single final normalisation of its
// §4.1 and fp32 statistics / 16-bit matrix products of its §6.3.
//
// Work decomposition: one work-group of NW waves per (batch, q-head, block of
// NW*32 query rows); each wave owns 32 rows, whose Q fragments stay in
// registers.  K/V tiles of BC keys stream through LDS, double-buffered and
// filled by direct global->LDS loads: the load of tile j+1 runs while tile j
// is in use.  With NW = 8 (two waves per SIMD) the waves of a SIMD overlap
// each other's LDS and VALU latency.
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
#pragma once

#include "attn_kernels.h"
#include "device_common.h"

namespace attn {

constexpr float kRescaleThreshold = 8.0f;  // log2 units: p stays <= 256

template <class E, int D, int NW, int BC, bool CAUSAL, bool MASK>
struct FwdKernel {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE_BYTES = BC * D * 2;     // one K or V tile
  static constexpr int ROWS = NW * 32;              // query rows per block
  static constexpr int SPW = BC * CPR / (NW * 64);  // DMA slots per wave per tensor
  static constexpr int KB = BC / 32;                // 32-key blocks per tile
  static constexpr int KS = D / 16;                 // k-steps of QK^T
  static constexpr int DT = D / 32;                 // 32-wide d tiles of O
  static constexpr int PT = BC / 16;                // k-steps of PV
  static_assert(BC * CPR % (NW * 64) == 0, "tile must split evenly into DMA slots");

  using T = typename E::T;
  using V8 = typename E::V8;
  using V4 = typename E::V4;

  struct State {
    int lane, wave, hl, l32;
    int b, h;                   // batch and q-head of this block
    int q_w0;                   // first query row of this wave
    int kv_limit;               // keys >= kv_limit are excluded
    int nk;                     // keys in memory
    int n_act;                  // tiles this wave has to visit (causal)
    int dchunks;                // 16-byte chunks per row in memory (d / 8)
    const T* kp;
    const T* vp;
    int64_t k_sn, v_sn;
    int koff[SPW], voff[SPW];   // element offset of this lane's DMA chunks in a tile
    float c;                    // scale * log2(e)
    V8 qf[KS];                  // Q fragments (B operand of S^T = K Q^T)
    f32x16 acc[DT];             // O^T accumulators
    float m_run, l_run;
  };

  // DMA slot s of a tile (16 bytes): its row and the element offsets of the
  // K and V chunks that land there (swizzled, clamped to the head dim).
  static __device__ __forceinline__ void slot_chunks(int s, int dchunks, int& row, int& kc,
                                                     int& vc) {
    row = s / CPR;
    const int p = s % CPR;
    kc = min(p ^ swz_k<CPR>(row), dchunks - 1) * 8;
    vc = min(p ^ swz_v<CPR>(row), dchunks - 1) * 8;
  }

  // Direct loads of one K tile and one V tile (keys j0..j0+BC-1).  In the
  // last, partial tile the rows beyond the last key are clamped onto valid
  // memory; chunks beyond the head dimension are clamped likewise.  Those
  // extra keys are masked to -inf and the extra K columns meet zero Q
  // columns, so their (finite) values never reach the result.
  static __device__ __forceinline__ void issue(const State& st, int j0, char* kb, char* vb) {
    if (j0 + BC <= st.nk) {
      const T* kbase = st.kp + (int64_t)j0 * st.k_sn;
      const T* vbase = st.vp + (int64_t)j0 * st.v_sn;
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int slot0 = (i * NW + st.wave) * 64;
        dma16(kbase + st.koff[i], kb + slot0 * 16);
        dma16(vbase + st.voff[i], vb + slot0 * 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int slot0 = (i * NW + st.wave) * 64;
        int row, kc, vc;
        slot_chunks(slot0 + st.lane, st.dchunks, row, kc, vc);
        const int64_t grow = min(j0 + row, st.nk - 1);
        dma16(st.kp + grow * st.k_sn + kc, kb + slot0 * 16);
        dma16(st.vp + grow * st.v_sn + vc, vb + slot0 * 16);
      }
    }
  }

  // One KV tile: S^T, masking, online softmax, PV.
  static __device__ __forceinline__ void tile(const FwdArgs& a, State& st, const char* kbuf,
                                              const char* vbuf, int j0) {
    // S^T = K_j Q^T
    f32x16 s[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) s[k] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int row = k * 32 + st.l32;
        const int c = (ks * 2 + st.hl) ^ swz_k<CPR>(row);
        const V8 kf = lds_read16<V8>(kbuf + row * (D * 2) + c * 16);
        s[k] = E::mfma(kf, st.qf[ks], s[k]);
      }
    }

    const int qrow = st.q_w0 + st.l32;
    if constexpr (MASK) {
      const int mrow = min(qrow, a.Nq - 1);
      const float* mp = a.mask + st.b * a.m_sb + st.h * a.m_sh + (int64_t)mrow * a.m_sq;
#pragma unroll
      for (int k = 0; k < KB; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + k * 32 + (r >> 2) * 8 + st.hl * 4 + (r & 3);
          s[k][r] = s[k][r] * st.c + mp[min(key, a.Nk - 1)] * kLog2e;
        }
    }
    const bool edge = (j0 + BC > st.kv_limit) || (CAUSAL && j0 + BC - 1 > st.q_w0);
    if (edge) {
#pragma unroll
      for (int k = 0; k < KB; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + k * 32 + (r >> 2) * 8 + st.hl * 4 + (r & 3);
          if (key >= st.kv_limit || (CAUSAL && key > qrow)) s[k][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < KB; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[k][r]);
    mx = max_with_other_half(mx);
    const float cand = MASK ? mx : mx * st.c;
    if (__builtin_amdgcn_ballot_w64(cand > st.m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(st.m_run, cand);
      if (m_new > st.m_run) {
        const float alpha = (st.m_run == -INFINITY) ? 0.f : fast_exp2(st.m_run - m_new);
        st.l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) st.acc[dt] *= alpha;
        st.m_run = m_new;
      }
    }
    const float mref = st.m_run == -INFINITY ? 0.f : st.m_run;
    float lsum = 0.f;
    V8 pf[PT];
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      const int k = t >> 1, r0 = (t & 1) * 8;
      typename E::V2 pp[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x0 = s[k][r0 + 2 * q], x1 = s[k][r0 + 2 * q + 1];
        x0 = fast_exp2(MASK ? x0 - mref : __builtin_fmaf(x0, st.c, -mref));
        x1 = fast_exp2(MASK ? x1 - mref : __builtin_fmaf(x1, st.c, -mref));
        lsum += x0 + x1;
        pp[q] = E::cvt2(x0, x1);
      }
      V4 lo = __builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3);
      V4 hi = __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3);
      pf[t] = concat4<V8, V4>(lo, hi);
    }
    st.l_run += lsum;

    // O^T += V_j^T P^T
    const int grp = st.lane >> 4, gi = st.lane & 15;
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
        st.acc[dt] = E::mfma(concat4<V8, V4>(lo, hi), pf[t], st.acc[dt]);
      }
    }
  }

  static __device__ __forceinline__ void step(const FwdArgs& a, State& st, int j, int n_tiles,
                                              const char* kc, const char* vc, char* kn, char* vn) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's share of tile j has landed
    __syncthreads();
    if (j + 1 < n_tiles) issue(st, (j + 1) * BC, kn, vn);
    if (j < st.n_act) tile(a, st, kc, vc, j * BC);
  }

  static __device__ __forceinline__ void run(const FwdArgs& a, char* k0, char* v0, char* k1,
                                             char* v1) {
    State st;
    st.lane = threadIdx.x & 63;
    st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    st.hl = st.lane >> 5;
    st.l32 = st.lane & 31;

    const int wid = xcd_remap(blockIdx.x, a.total_blocks);
    int qblk = wid % a.nqb;
    const int bh = wid / a.nqb;
    const int h = bh % a.Hq;
    const int b = bh / a.Hq;
    st.b = b;
    st.h = h;
    if (CAUSAL) qblk = a.nqb - 1 - qblk;  // longest rows first
    const int g = h / a.group;
    const int q_blk0 = qblk * ROWS;
    st.q_w0 = q_blk0 + st.wave * 32;

    st.kv_limit = a.Nk;
    if (a.kv_lens) st.kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
    int kv_end = st.kv_limit;
    if (CAUSAL) kv_end = min(kv_end, min(q_blk0 + ROWS, a.Nq));
    const int n_tiles = (kv_end + BC - 1) / BC;
    // causal: a wave sees no key beyond its last row
    st.n_act = CAUSAL ? min(n_tiles, (st.q_w0 + 31) / BC + 1) : n_tiles;
    st.dchunks = a.d / 8;
    st.nk = a.Nk;
    st.c = a.c;
    st.k_sn = a.k_sn;
    st.v_sn = a.v_sn;
    st.kp = (const T*)a.k + b * a.k_sb + g * a.k_sh;
    st.vp = (const T*)a.v + b * a.v_sb + g * a.v_sh;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      int row, kc, vc;
      slot_chunks((i * NW + st.wave) * 64 + st.lane, st.dchunks, row, kc, vc);
      st.koff[i] = row * (int)st.k_sn + kc;
      st.voff[i] = row * (int)st.v_sn + vc;
    }

    const T* qp = (const T*)a.q + b * a.q_sb + h * a.q_sh;
    {
      const int row = min(st.q_w0 + st.l32, a.Nq - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + st.hl * 8;
        st.qf[ks] = d0 < a.d ? *(const V8*)(qp + row * a.q_sn + d0) : V8{};
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc[dt] = f32x16{};
    st.m_run = -INFINITY;
    st.l_run = 0.f;

    if (n_tiles > 0) issue(st, 0, k0, v0);
    for (int j = 0; j < n_tiles; j += 2) {
      step(a, st, j, n_tiles, k0, v0, k1, v1);
      if (j + 1 >= n_tiles) break;
      step(a, st, j + 1, n_tiles, k1, v1, k0, v0);
    }

    // Epilogue.
    T* op = (T*)a.o + b * a.o_sb + h * a.o_sh;
    const float l_tot = add_with_other_half(st.l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const int row = st.q_w0 + st.l32;
    if (row < a.Nq) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int col = dt * 32 + gq * 8 + st.hl * 4;
          if (col < a.d) {
            auto lo = E::cvt2(st.acc[dt][gq * 4 + 0] * inv, st.acc[dt][gq * 4 + 1] * inv);
            auto hi = E::cvt2(st.acc[dt][gq * 4 + 2] * inv, st.acc[dt][gq * 4 + 3] * inv);
            V4 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
            *(V4*)(op + row * a.o_sn + col) = w;
          }
        }
      }
      if (st.hl == 0)
        a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] =
            l_tot > 0.f ? (st.m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
  }
};

template <class E, int D, int NW, int BC, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4)))
void fwd_kernel(FwdArgs a) {
  using K = FwdKernel<E, D, NW, BC, CAUSAL, MASK>;
  __shared__ __attribute__((aligned(1024))) char k0[K::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[K::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[K::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[K::TILE_BYTES];
  K::run(a, k0, v0, k1, v1);
}

}  // namespace attn
