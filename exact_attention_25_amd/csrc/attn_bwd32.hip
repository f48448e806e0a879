// fp32 backward attention for gfx950: the gradients of <dO, O> for
// O = softmax(S) V with P formed again from the forward's LSE
// ("FlashAttention技术解析：优化Transformer注意力计算效率" §3.3), every
// product on the fp32 MFMA (v_mfma_f32_32x32x2_f32) and every intermediate in
// fp32, so the result carries no 16-bit rounding:
//     P = exp(S - LSE), dP = dO V^T, D_i = sum_c dO_ic O_ic,
//     dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
// With fp32 O, D comes straight from dO and O (its rounding is that of fp32).
//
//  1. bwd32_prep_kernel: D and nl2 = -LSE log2(e) per row (0 / -inf on the
//     padding rows past Nq and nl2 = -inf on fully masked rows).
//  2. bwd32_q_kernel: 4 waves per (batch, q-head, 128 rows), lanes own query
//     rows; K/V tiles of 32 keys through LDS.
//  3. bwd32_kv_kernel: 4 waves per (batch, kv-head, 128 keys), lanes own
//     keys; it loops over every q-head of the kv-head and over Q/dO tiles of
//     32 rows, so grouped-query sums need neither atomics nor partials.
//
// LDS tiles use a row stride of D+1 floats.  MFMA operand layouts (32x32x2):
// lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32]; register r of the
// result holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
//
// LOCAL (window / 2-D neighbourhood, causal folded in) and SOFTCAP as in the
// 16-bit kernels (attn_bwd_kernel.h): tiles outside a block's reach are
// skipped, excluded elements get P = 0 from the visibility words of
// local_mask.h, and the soft cap's logit and derivative come from
// softcap_grad.
#include "attn_kernels.h"
#include "device_common.h"
#include "local_mask.h"

namespace attn {

__global__ __launch_bounds__(256) void bwd32_prep_kernel(BwdArgs a) {
  const int64_t n = (int64_t)a.B * a.Hq * a.ld_rows;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int row = (int)(i % a.ld_rows);
    const int64_t bh = i / a.ld_rows;
    const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
    float dsum = 0.f, nl = -INFINITY;
    if (row < a.Nq) {
      const int64_t off = b * a.q_sb + h * a.q_sh + (int64_t)row * a.q_sn;
      const float* op = (const float*)a.o + off;
      const float* dp = (const float*)a.dout + off;
      for (int c = 0; c < a.d; ++c) dsum = __builtin_fmaf(dp[c], op[c], dsum);
      const float lse = a.lse[bh * a.Nq + row];
      nl = lse == -INFINITY ? -INFINITY : -lse * kLog2e;
    }
    a.delta[i] = dsum;
    a.nl2[i] = nl;
  }
}

template <int D, bool CAUSAL, bool MASK, bool LOCAL, bool SOFTCAP>
__global__ __launch_bounds__(256) void bwd32_q_kernel(BwdArgs a) {
  constexpr int BC = 32, NW = 4, ROWS = NW * 32, DT = D / 32, KS = D / 2, LD = D + 1;
  __shared__ float ks_[BC * LD];
  __shared__ float vs_[BC * LD];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane >> 5, l32 = lane & 31;

  const int nqb = (a.Nq + ROWS - 1) / ROWS;
  int qblk, bh;
  block_coords(CAUSAL, blockIdx.x, a.B * a.Hq, nqb, qblk, bh);
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int g = h / a.group;
  const int q_blk0 = qblk * ROWS;
  const int q_w0 = q_blk0 + wave * 32;
  const int qrow = q_w0 + l32;
  const int crow = min(qrow, a.Nq - 1);

  int kv_limit = a.Nk;
  if (a.kv_lens) kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
  int kv_end = kv_limit;
  if (CAUSAL) kv_end = min(kv_end, min(q_blk0 + ROWS, a.Nq));
  int t_begin = 0, t_end = (kv_end + BC - 1) / BC;
  int w_lo = 0, w_hi = t_end;   // this wave's key tiles
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
    lrow = a.loc.row(crow);
  }

  const float* qp = (const float*)a.q + b * a.q_sb + h * a.q_sh + (int64_t)crow * a.q_sn;
  const float* dop = (const float*)a.dout + b * a.q_sb + h * a.q_sh + (int64_t)crow * a.q_sn;
  const float* kp = (const float*)a.k + b * a.k_sb + g * a.k_sh;
  const float* vp = (const float*)a.v + b * a.k_sb + g * a.k_sh;
  const float* mrow = MASK ? a.mask + b * a.m_sb + h * a.m_sh + (int64_t)crow * a.m_sq : nullptr;

  float qf[KS], df[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int col = 2 * ks + hl;
    qf[ks] = col < a.d ? qp[col] : 0.f;
    df[ks] = col < a.d ? dop[col] : 0.f;
  }
  // rows past Nq read D = 0 and nl2 = -inf (the padded workspace rows)
  const int64_t wrow = ((int64_t)b * a.Hq + h) * a.ld_rows + qrow;
  const float nl2 = a.nl2[wrow];
  const float dd = a.delta[wrow];

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  for (int j = t_begin; j < t_end; ++j) {
    const int j0 = j * BC;
    __syncthreads();
    for (int idx = threadIdx.x; idx < BC * D; idx += NW * 64) {
      const int r = idx / D, c = idx % D;
      // rows past kv_lens are zero, whatever the tensors hold there
      const int64_t grow = min(j0 + r, a.Nk - 1);
      const bool ok = c < a.d && j0 + r < kv_limit;
      ks_[r * LD + c] = ok ? kp[grow * a.k_sn + c] : 0.f;
      vs_[r * LD + c] = ok ? vp[grow * a.k_sn + c] : 0.f;
    }
    __syncthreads();
    uint32_t w = 0;   // LOCAL: bit 8 (r / 4) + r % 4 set iff register r's key is visible
    if constexpr (LOCAL) {
      if (j < w_lo || j >= w_hi) continue;
      const uint32_t bits = (uint32_t)a.loc.bits(lrow, j0, kv_limit);
      if (!__builtin_amdgcn_ballot_w64(bits != 0)) continue;
      w = bits >> (4 * hl);
    }

    // S^T = K Q^T and dP^T = V dO^T: lane holds row qrow, register r key
    // j0 + 8 (r / 4) + 4 hl + r % 4
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks_[l32 * LD + 2 * ks + hl], qf[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vs_[l32 * LD + 2 * ks + hl], df[ks], dp, 0, 0, 0);
    }
    f32x16 ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + (r >> 2) * 8 + hl * 4 + (r & 3);
      const float ml = MASK ? __builtin_fmaf(mrow[min(key, a.Nk - 1)], kLog2e, nl2) : nl2;
      float g = 1.f;
      const float t = SOFTCAP ? softcap_grad(s[r], a.cap_a, a.cap_c2, g) + ml
                              : __builtin_fmaf(s[r], a.c, ml);
      float p = fast_exp2(t);
      if constexpr (LOCAL) {
        if (!((w >> ((r >> 2) * 8 + (r & 3))) & 1u)) p = 0.f;
      } else {
        if (key >= kv_limit || (CAUSAL && key > qrow)) p = 0.f;
      }
      ds[r] = SOFTCAP ? p * g * (dp[r] - dd) : p * (dp[r] - dd);
    }
    // dQ^T += K^T dS^T, two keys per step (lane half hl supplies key
    // 8 (r / 4) + 4 hl + r % 4 of the tile through register r)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = (r >> 2) * 8 + hl * 4 + (r & 3);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks_[kk * LD + dt * 32 + l32], ds[r], acc[dt],
                                                       0, 0, 0);
    }
  }

  if (qrow >= a.Nq) return;
  const int64_t base = b * a.q_sb + h * a.q_sh + (int64_t)qrow * a.q_sn;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int col = dt * 32 + gq * 8 + hl * 4;
      if (col < a.d) {
        f32x4 w = {a.scale * acc[dt][gq * 4 + 0], a.scale * acc[dt][gq * 4 + 1],
                   a.scale * acc[dt][gq * 4 + 2], a.scale * acc[dt][gq * 4 + 3]};
        *(f32x4*)((float*)a.dq + base + col) = w;
      }
    }
}

template <int D, bool CAUSAL, bool MASK, bool LOCAL, bool SOFTCAP>
__global__ __launch_bounds__(256) void bwd32_kv_kernel(BwdArgs a) {
  constexpr int BR = 32, NW = 4, KEYS = NW * 32, DT = D / 32, KS = D / 2, LD = D + 1;
  __shared__ float qs_[BR * LD];
  __shared__ float os_[BR * LD];     // dO tile
  __shared__ float nls_[BR];
  __shared__ float dds_[BR];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane >> 5, l32 = lane & 31;

  const int nkb = (a.Nk + KEYS - 1) / KEYS;
  const int kblk = blockIdx.x % nkb;
  const int rest = blockIdx.x / nkb;
  const int g = rest % a.Hkv, b = rest / a.Hkv;
  const int key0 = kblk * KEYS;
  const int kw0 = key0 + wave * 32;
  const int key = kw0 + l32;
  const int ckey = min(key, a.Nk - 1);

  int kv_limit = a.Nk;
  if (a.kv_lens) kv_limit = min(max(a.kv_lens[b], 0), a.Nk);

  // K^T / V^T operands of this lane's key
  float kf[KS], vf[KS];
  {
    const float* kp = (const float*)a.k + b * a.k_sb + g * a.k_sh + (int64_t)ckey * a.k_sn;
    const float* vp = (const float*)a.v + b * a.k_sb + g * a.k_sh + (int64_t)ckey * a.k_sn;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int col = 2 * ks + hl;
      kf[ks] = col < a.d ? kp[col] : 0.f;
      vf[ks] = col < a.d ? vp[col] : 0.f;
    }
  }
  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  // rows before key0 see none of this block's keys (causal)
  int q_start = CAUSAL ? (key0 / BR) * BR : 0;
  int q_end = a.Nq;
  int wq_lo = 0, wq_hi = a.Nq - 1;   // rows that may see one of this wave's keys
  LocalVis lvt{};
  LocalVis::Row lrow{};
  if constexpr (LOCAL) {
    // the rows that see key j are those the exchanged relation gives for j
    lvt = a.loc.transposed();
    int lo, hi;
    lvt.key_range(key0, min(key0 + KEYS, kv_limit) - 1, a.Nq, lo, hi);
    q_start = (lo / BR) * BR;
    q_end = hi >= lo ? hi + 1 : q_start;
    wq_lo = 1;
    wq_hi = 0;
    if (kw0 < kv_limit) lvt.key_range(kw0, min(kw0 + 31, kv_limit - 1), a.Nq, wq_lo, wq_hi);
    lrow = lvt.row(ckey);
  }
  const bool any = key0 < kv_limit;
  for (int hh = 0; hh < a.group && any; ++hh) {
    const int h = g * a.group + hh;
    const float* qp = (const float*)a.q + b * a.q_sb + h * a.q_sh;
    const float* dop = (const float*)a.dout + b * a.q_sb + h * a.q_sh;
    const float* mcol = MASK ? a.mask + b * a.m_sb + h * a.m_sh + ckey : nullptr;
    const int64_t wbase = ((int64_t)b * a.Hq + h) * a.ld_rows;
    for (int q0 = q_start; q0 < q_end; q0 += BR) {
      __syncthreads();
      for (int idx = threadIdx.x; idx < BR * D; idx += NW * 64) {
        const int r = idx / D, c = idx % D;
        const int64_t grow = min(q0 + r, a.Nq - 1);
        qs_[r * LD + c] = c < a.d ? qp[grow * a.q_sn + c] : 0.f;
        os_[r * LD + c] = c < a.d ? dop[grow * a.q_sn + c] : 0.f;
      }
      // q0 + BR <= Nq rounded up to 32 <= ld_rows
      if (threadIdx.x < BR) {
        nls_[threadIdx.x] = a.nl2[wbase + q0 + threadIdx.x];
        dds_[threadIdx.x] = a.delta[wbase + q0 + threadIdx.x];
      }
      __syncthreads();
      uint32_t w = 0;   // LOCAL: bit 8 (r / 4) + r % 4 set iff register r's row sees the key
      if constexpr (LOCAL) {
        if (q0 + BR - 1 < wq_lo || q0 > wq_hi) continue;
        const uint32_t bits = (uint32_t)lvt.bits(lrow, q0, a.Nq);
        if (!__builtin_amdgcn_ballot_w64(bits != 0)) continue;
        w = bits >> (4 * hl);
      }

      // S = Q K^T and dP = dO V^T: lane holds key `key`, register r row
      // q0 + 8 (r / 4) + 4 hl + r % 4
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(qs_[l32 * LD + 2 * ks + hl], kf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x2f32(os_[l32 * LD + 2 * ks + hl], vf[ks], dp, 0, 0, 0);
      }
      f32x16 pv, dsv;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = (r >> 2) * 8 + hl * 4 + (r & 3);
        const int row = q0 + lr;
        const float ml = MASK ? __builtin_fmaf(mcol[(int64_t)min(row, a.Nq - 1) * a.m_sq], kLog2e,
                                               nls_[lr])
                              : nls_[lr];
        float g = 1.f;
        const float t = SOFTCAP ? softcap_grad(s[r], a.cap_a, a.cap_c2, g) + ml
                                : __builtin_fmaf(s[r], a.c, ml);
        float p = fast_exp2(t);
        if constexpr (LOCAL) {
          if (!((w >> ((r >> 2) * 8 + (r & 3))) & 1u)) p = 0.f;
        } else {
          if (CAUSAL && key > row) p = 0.f;
        }
        pv[r] = p;
        dsv[r] = SOFTCAP ? p * g * (dp[r] - dds_[lr]) : p * (dp[r] - dds_[lr]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS, two rows per step
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = (r >> 2) * 8 + hl * 4 + (r & 3);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          dv[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(os_[lr * LD + dt * 32 + l32], pv[r], dv[dt],
                                                        0, 0, 0);
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(qs_[lr * LD + dt * 32 + l32], dsv[r], dk[dt],
                                                        0, 0, 0);
        }
      }
    }
  }

  // lane holds key `key`; register r of block dt holds d = 32 dt + 8 (r / 4) + 4 hl + r % 4.
  // Keys at or past kv_limit get zero (their P was not masked above).
  if (key >= a.Nk) return;
  const bool kv_ok = key < kv_limit;
  const int64_t base = b * a.k_sb + g * a.k_sh + (int64_t)key * a.k_sn;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int col = dt * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
      if (col < a.d) {
        ((float*)a.dk)[base + col] = kv_ok ? a.scale * dk[dt][r] : 0.f;
        ((float*)a.dv)[base + col] = kv_ok ? dv[dt][r] : 0.f;
      }
    }
}

template <int D, bool CAUSAL, bool MASK, bool LOCAL, bool SOFTCAP>
static void launch_bwd32_t(const BwdArgs& a, hipStream_t st) {
  if (a.Nq > 0) {
    const int nqb = (a.Nq + 127) / 128;
    hipLaunchKernelGGL((bwd32_q_kernel<D, CAUSAL, MASK, LOCAL, SOFTCAP>),
                       dim3((unsigned)(a.B * a.Hq * nqb)), dim3(256), 0, st, a);
  }
  if (a.Nk > 0) {
    const int nkb = (a.Nk + 127) / 128;
    hipLaunchKernelGGL((bwd32_kv_kernel<D, CAUSAL, MASK, LOCAL, SOFTCAP>),
                       dim3((unsigned)(a.B * a.Hkv * nkb)), dim3(256), 0, st, a);
  }
}

// causal is folded into a.loc under LOCAL
template <int D, bool MASK, bool LOCAL, bool SOFTCAP>
static void launch_bwd32_c(const BwdArgs& a, bool causal, hipStream_t st) {
  if (causal && !LOCAL) launch_bwd32_t<D, !LOCAL, MASK, LOCAL, SOFTCAP>(a, st);
  else launch_bwd32_t<D, false, MASK, LOCAL, SOFTCAP>(a, st);
}

template <int D, bool MASK>
static void launch_bwd32_m(const BwdArgs& a, FwdMode m, hipStream_t st) {
  if (m.local) {
    if (m.softcap) launch_bwd32_c<D, MASK, true, true>(a, false, st);
    else launch_bwd32_c<D, MASK, true, false>(a, false, st);
  } else {
    if (m.softcap) launch_bwd32_c<D, MASK, false, true>(a, m.causal, st);
    else launch_bwd32_c<D, MASK, false, false>(a, m.causal, st);
  }
}

template <int D>
static void launch_bwd32_d(const BwdArgs& a, FwdMode m, hipStream_t st) {
  if (m.mask) launch_bwd32_m<D, true>(a, m, st);
  else launch_bwd32_m<D, false>(a, m, st);
}

hipError_t launch_bwd32(const BwdArgs& a, FwdMode m, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.Hq * a.ld_rows;
  if (n > 0) {
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(bwd32_prep_kernel, dim3(blocks), dim3(256), 0, st, a);
  }
  if (a.d > 64) launch_bwd32_d<128>(a, m, st);
  else launch_bwd32_d<64>(a, m, st);
  return hipGetLastError();
}

}  // namespace attn
