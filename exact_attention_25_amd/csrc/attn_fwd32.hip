// fp32 forward attention for gfx950: the same tiled online softmax as the
// 16-bit kernels ("FlashAttention技术解析" §2.2), with both matrix products
// on the fp32 MFMA (v_mfma_f32_32x32x2_f32) and P kept in fp32, so the
// result carries no 16-bit rounding.
//
// One work-group of 4 waves per (batch, q-head, 128 query rows); each wave
// owns 32 rows.  K/V tiles of 32 keys go through LDS (row stride D+1 floats,
// so a column read by 32 lanes hits 32 different banks).
//
// LOCAL / SOFTCAP as in the 16-bit FwdKernel: only the key tiles that may be
// visible to the work-group's rows are loaded, a wave skips tiles without a
// visible key for any of its lanes, and elements are masked through the
// visibility bits of local_mask.h; the soft cap transforms S right after
// QK^T.
#include "attn_kernels.h"
#include "device_common.h"
#include "local_mask.h"

namespace attn {

template <int D, bool CAUSAL, bool MASK, bool LOCAL, bool SOFTCAP>
__global__ __launch_bounds__(256) void fwd32_kernel(FwdArgs a) {
  constexpr int BC = 32, NW = 4, ROWS = NW * 32, DT = D / 32, KS = D / 2, LD = D + 1;
  constexpr float TH = 8.0f;
  constexpr bool PRE = MASK || SOFTCAP;   // S already in log2 units
  __shared__ float ks_[BC * LD];
  __shared__ float vs_[BC * LD];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane >> 5, l32 = lane & 31;

  int qblk, bh;
  block_coords(CAUSAL, blockIdx.x, a.B * a.Hq, a.nqb, qblk, bh);
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int g = h / a.group;
  const int q_blk0 = qblk * ROWS;
  const int q_w0 = q_blk0 + wave * 32;
  const int qrow = q_w0 + l32;

  int kv_limit = a.Nk;
  if (a.kv_lens) kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
  int kv_end = kv_limit;
  if (CAUSAL) kv_end = min(kv_end, min(q_blk0 + ROWS, a.Nq));
  int t_begin = 0, t_end = (kv_end + BC - 1) / BC;
  int w_lo = 0, w_hi = t_end;   // this wave's tiles
  LocalVis::Row lrow{};
  if constexpr (LOCAL) {
    int lo, hi;
    a.loc.key_range(q_blk0, min(q_blk0 + ROWS, a.Nq) - 1, kv_limit, lo, hi);
    t_begin = lo / BC;
    t_end = hi >= lo ? hi / BC + 1 : t_begin;
    w_lo = w_hi = 0;
    if (q_w0 < a.Nq) {
      a.loc.key_range(q_w0, min(q_w0 + 31, a.Nq - 1), kv_limit, lo, hi);
      w_lo = lo / BC;
      w_hi = hi >= lo ? hi / BC + 1 : w_lo;
    }
    lrow = a.loc.row(min(qrow, a.Nq - 1));
  }

  const float* qp = (const float*)a.q + b * a.q_sb + h * a.q_sh;
  const float* kp = (const float*)a.k + b * a.k_sb + g * a.k_sh;
  const float* vp = (const float*)a.v + b * a.v_sb + g * a.v_sh;

  float qf[KS];
  {
    const int row = min(qrow, a.Nq - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int col = 2 * ks + hl;
      qf[ks] = col < a.d ? qp[row * a.q_sn + col] : 0.f;
    }
  }
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // K/V tiles are read 16 bytes at a time into registers one tile ahead (the
  // next tile's loads are in flight while the current one is computed), then
  // written to LDS; rows past kv_lens are zero, whatever the tensors hold.
  constexpr int NL = BC * D / 4 / (NW * 64);   // float4 per thread per tensor
  f32x4 kr[NL], vr[NL];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = (threadIdx.x + i * NW * 64) * 4;
      const int r = e / D, c = e % D;
      const bool ok = c < a.d && j0 + r < kv_limit;
      const int64_t grow = ok ? j0 + r : 0;
      kr[i] = ok ? *(const f32x4*)(kp + grow * a.k_sn + c) : f32x4{};
      vr[i] = ok ? *(const f32x4*)(vp + grow * a.v_sn + c) : f32x4{};
    }
  };
  if (t_begin < t_end) load_tile(t_begin * BC);
  for (int j = t_begin; j < t_end; ++j) {
    const int j0 = j * BC;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = (threadIdx.x + i * NW * 64) * 4;
      const int r = e / D, c = e % D;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ks_[r * LD + c + u] = kr[i][u];
        vs_[r * LD + c + u] = vr[i][u];
      }
    }
    __syncthreads();
    if (j + 1 < t_end) load_tile(j0 + BC);
    uint32_t bits = 0;   // LOCAL: bit i set iff key j0 + i is visible to this lane's row
    if constexpr (LOCAL) {
      if (j < w_lo || j >= w_hi) continue;
      bits = (uint32_t)a.loc.bits(lrow, j0, kv_limit);
      if (!__builtin_amdgcn_ballot_w64(bits != 0)) continue;
    }

    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks_[l32 * LD + 2 * ks + hl], qf[ks], s, 0, 0, 0);

    if constexpr (SOFTCAP) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = softcap_log2(s[r], a.cap_a, a.cap_c2);
    }
    if constexpr (MASK) {
      const int mrow = min(qrow, a.Nq - 1);
      const float* mp = a.mask + b * a.m_sb + h * a.m_sh + (int64_t)mrow * a.m_sq;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + (r >> 2) * 8 + hl * 4 + (r & 3);
        s[r] = (SOFTCAP ? s[r] : s[r] * a.c) + mp[min(key, a.Nk - 1)] * kLog2e;
      }
    }
    if constexpr (LOCAL) {
      const uint32_t w = bits >> (hl * 4);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = keep_if_bit(s[r], w, (r >> 2) * 8 + (r & 3));
    } else {
      const bool edge = (j0 + BC > kv_limit) || (CAUSAL && j0 + BC - 1 > q_w0);
      if (edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (key >= kv_limit || (CAUSAL && key > qrow)) s[r] = -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_with_other_half(mx);
    const float cand = PRE ? mx : mx * a.c;
    if (__builtin_amdgcn_ballot_w64(cand > m_run + TH)) {
      const float m_new = fmaxf(m_run, cand);
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      if (m_new != -INFINITY) {
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
        m_run = m_new;
      }
    }
    const float mref = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float t = PRE ? (s[r] - mref) : __builtin_fmaf(s[r], a.c, -mref);
      s[r] = fast_exp2(t);
      l_run += s[r];
    }
    // O^T += V^T P^T, two keys per step: lane half hl supplies key
    // (r/4)*8 + 4*hl + r%4 through register r.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = (r >> 2) * 8 + hl * 4 + (r & 3);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs_[key * LD + dt * 32 + l32], s[r], acc[dt], 0, 0, 0);
    }
  }

  const float l_tot = add_with_other_half(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qrow < a.Nq) {
    float* op = (float*)a.o + b * a.o_sb + h * a.o_sh + qrow * a.o_sn;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = dt * 32 + gq * 8 + hl * 4;
        if (col < a.d) {
          f32x4 w = {acc[dt][gq * 4 + 0] * inv, acc[dt][gq * 4 + 1] * inv,
                     acc[dt][gq * 4 + 2] * inv, acc[dt][gq * 4 + 3] * inv};
          *(f32x4*)(op + col) = w;
        }
      }
    if (hl == 0)
      a.lse[((int64_t)b * a.Hq + h) * a.Nq + qrow] =
          l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool MASK, bool LOCAL, bool SOFTCAP>
static void launch32_c(const FwdArgs& a, bool causal, hipStream_t st) {
  dim3 grid(a.total_blocks), block(256);
  if (causal && !LOCAL)
    hipLaunchKernelGGL((fwd32_kernel<D, !LOCAL, MASK, LOCAL, SOFTCAP>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((fwd32_kernel<D, false, MASK, LOCAL, SOFTCAP>), grid, block, 0, st, a);
}

template <int D, bool MASK>
static void launch32_m(const FwdArgs& a, FwdMode m, hipStream_t st) {
  if (m.local) {
    if (m.softcap) launch32_c<D, MASK, true, true>(a, false, st);
    else launch32_c<D, MASK, true, false>(a, false, st);
  } else {
    if (m.softcap) launch32_c<D, MASK, false, true>(a, m.causal, st);
    else launch32_c<D, MASK, false, false>(a, m.causal, st);
  }
}

template <int D>
static void launch32_d(const FwdArgs& a, FwdMode m, hipStream_t st) {
  if (m.mask) launch32_m<D, true>(a, m, st);
  else launch32_m<D, false>(a, m, st);
}

hipError_t launch_fwd32(const FwdArgs& a0, FwdMode m, hipStream_t st) {
  FwdArgs a = a0;
  a.nqb = (a.Nq + 127) / 128;
  a.total_blocks = a.B * a.Hq * a.nqb;
  if (a.d > 64) launch32_d<128>(a, m, st);
  else launch32_d<64>(a, m, st);
  return hipGetLastError();
}

}  // namespace attn
