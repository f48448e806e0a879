// fp32 forward attention for gfx950: the same tiled online softmax as the
// 16-bit kernels ("FlashAttention技术解析" §2.2), with both matrix products
// on the fp32 MFMA (v_mfma_f32_32x32x2_f32) and P kept in fp32, so the
// result carries no 16-bit rounding.
//
// One work-group of 4 waves per (batch, q-head, 128 query rows); each wave
// owns 32 rows.  K/V tiles of 32 keys go through LDS (row stride D+1 floats,
// so a column read by 32 lanes hits 32 different banks).
#include "attn_kernels.h"
#include "device_common.h"

namespace attn {

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256) void fwd32_kernel(FwdArgs a) {
  constexpr int BC = 32, NW = 4, ROWS = NW * 32, DT = D / 32, KS = D / 2, LD = D + 1;
  constexpr float TH = 8.0f;
  __shared__ float ks_[BC * LD];
  __shared__ float vs_[BC * LD];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane >> 5, l32 = lane & 31;

  const int wid = xcd_remap(blockIdx.x, a.total_blocks);
  int qblk = wid % a.nqb;
  const int bh = wid / a.nqb;
  const int h = bh % a.Hq, b = bh / a.Hq;
  if (CAUSAL) qblk = a.nqb - 1 - qblk;
  const int g = h / a.group;
  const int q_blk0 = qblk * ROWS;
  const int q_w0 = q_blk0 + wave * 32;
  const int qrow = q_w0 + l32;

  int kv_limit = a.Nk;
  if (a.kv_lens) kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
  int kv_end = kv_limit;
  if (CAUSAL) kv_end = min(kv_end, min(q_blk0 + ROWS, a.Nq));
  const int n_tiles = (kv_end + BC - 1) / BC;

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

  for (int j = 0; j < n_tiles; ++j) {
    const int j0 = j * BC;
    __syncthreads();
    for (int idx = threadIdx.x; idx < BC * D; idx += NW * 64) {
      const int r = idx / D, c = idx % D;
      const int grow = min(j0 + r, a.Nk - 1);
      ks_[r * LD + c] = c < a.d ? kp[grow * a.k_sn + c] : 0.f;
      vs_[r * LD + c] = c < a.d ? vp[grow * a.v_sn + c] : 0.f;
    }
    __syncthreads();

    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks_[l32 * LD + 2 * ks + hl], qf[ks], s, 0, 0, 0);

    if constexpr (MASK) {
      const int mrow = min(qrow, a.Nq - 1);
      const float* mp = a.mask + b * a.m_sb + h * a.m_sh + (int64_t)mrow * a.m_sq;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + (r >> 2) * 8 + hl * 4 + (r & 3);
        s[r] = s[r] * a.c + mp[min(key, a.Nk - 1)] * kLog2e;
      }
    }
    const bool edge = (j0 + BC > kv_limit) || (CAUSAL && j0 + BC - 1 > q_w0);
    if (edge) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + (r >> 2) * 8 + hl * 4 + (r & 3);
        if (key >= kv_limit || (CAUSAL && key > qrow)) s[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_with_other_half(mx);
    const float cand = MASK ? mx : mx * a.c;
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
      const float t = MASK ? (s[r] - mref) : __builtin_fmaf(s[r], a.c, -mref);
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

template <int D>
static hipError_t launch32_d(const FwdArgs& a, bool causal, bool mask, hipStream_t st) {
  dim3 grid(a.total_blocks), block(256);
  if (causal) {
    if (mask) hipLaunchKernelGGL((fwd32_kernel<D, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd32_kernel<D, true, false>), grid, block, 0, st, a);
  } else {
    if (mask) hipLaunchKernelGGL((fwd32_kernel<D, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd32_kernel<D, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd32(const FwdArgs& a0, bool causal, bool mask, hipStream_t st) {
  FwdArgs a = a0;
  a.nqb = (a.Nq + 127) / 128;
  a.total_blocks = a.B * a.Hq * a.nqb;
  if (a.d > 64) return launch32_d<128>(a, causal, mask, st);
  return launch32_d<64>(a, causal, mask, st);
}

}  // namespace attn
