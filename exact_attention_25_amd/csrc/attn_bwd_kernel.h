// Backward attention kernels for gfx950 (16-bit inputs, fp32 accumulation).
//
// The gradients of <dO, O> for O = softmax(S) V, S = scale * Q K^T, with P
// formed again from the forward's LSE instead of being stored
// ("FlashAttention技术解析：优化Transformer注意力计算效率"
// (jsqmd.com/news/722897) §3.3):
//     P  = exp(S - LSE),  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
//     dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// D_i equals sum_c dO_ic O_ic in exact arithmetic; it is accumulated here
// from P and dP (exact to fp32 rounding) rather than from the 16-bit stored
// O, whose rounding would otherwise dominate the error of dK and dQ.
//
// Loop order (the same page, §4.1 item 3): the dQ kernel keeps a block of
// query rows in registers and loops over key blocks; it finishes D on the
// way, using  dQ_i = scale (sum_j P_ij dP_ij k_j - D_i sum_j P_ij k_j),  and
// writes D for the dK/dV kernel, which keeps a block of keys in registers and
// loops over query blocks and over the q-heads that share the kv-head (so
// grouped-query sums need no atomics).
//
// Precision: the matrix products that take P or dS as an operand use fp16
// (11-bit significand) rather than bf16; bf16 inputs are converted to fp16
// for those products (exact for |x| in [2^-14, 65504]).  Exponentials are
// exp2 with the scale and log2(e) folded in: P = exp2(s * c + nl2), with
// nl2 = -LSE * log2(e) (-inf for a fully masked row, so that P = 0).
#pragma once

#include <type_traits>

#include "attn_kernels.h"
#include "device_common.h"

namespace attn {

// 8 x 16-bit input values -> 8 x fp16 (identity for fp16 inputs).
template <class E>
__device__ __forceinline__ f16x8 to_f16x8(typename E::V8 x) {
  if constexpr (std::is_same<E, FP16>::value) {
    return x;
  } else {
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    return __builtin_convertvector(__builtin_convertvector(x, f32x8), f16x8);
  }
}

// In-place bf16 -> fp16 conversion of the 16-byte LDS slots this lane filled
// (after its own direct loads have landed; identity for fp16 inputs).
template <class E, int SPW, int NW>
__device__ __forceinline__ void convert_own_slots(char* buf, int wave, int lane) {
  if constexpr (!std::is_same<E, FP16>::value) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      char* p = buf + ((i * NW + wave) * 64 + lane) * 16;
      const typename E::V8 x = lds_read16<typename E::V8>(p);
      *(LDS_AS f16x8*)(LDS_AS void*)(p) = to_f16x8<E>(x);
    }
  }
}

// --------------------------------------------------------------- dQ kernel
// One work-group of NW waves per (batch, q-head, block of NW*32 rows); each
// wave owns 32 rows, whose Q (as fp16) and dO fragments stay in registers.
// K and V tiles of BC keys stream through LDS (K converted to fp16 there).
// Per tile and wave:
//   S^T = K Q^T, dP^T = V dO^T        32x32x16 MFMA; each lane holds 16 keys
//                                     of one row
//   P^T, X^T = P^T * dP^T, D += X     per element
//   A^T += K^T X^T, B^T += K^T P^T    32x32x16 fp16 MFMA, K^T read transposed
//                                     from LDS, X^T / P^T from registers
// Epilogue: dQ = scale (A - D B); D and nl2 to the workspace.
template <class E, int D, int NW, int BC, bool CAUSAL>
struct BwdQ {
  static constexpr int ROWS = NW * 32;
  static constexpr int CPR = D / 8;
  static constexpr int TILE_BYTES = BC * D * 2;
  static constexpr int SPW = BC * CPR / (NW * 64);
  static constexpr int KB = BC / 32;
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int PT = BC / 16;
  static_assert(BC * CPR % (NW * 64) == 0, "tile must split evenly into DMA slots");

  using T = typename E::T;
  using V8 = typename E::V8;
  using H8 = f16x8;
  using H4 = f16x4;

  static __device__ __forceinline__ void issue(const BwdArgs& a, const T* kp, const T* vp, int j0,
                                               char* kb, char* vb, int wave, int lane) {
    const int dch = a.d / 8;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int slot0 = (i * NW + wave) * 64;
      const int s = slot0 + lane;
      const int row = s / CPR, p = s % CPR;
      const int64_t grow = min(j0 + row, a.Nk - 1);
      const int c = min(p ^ swz_k<CPR>(row), dch - 1) * 8;
      dma16(kp + grow * a.k_sn + c, kb + slot0 * 16);
      dma16(vp + grow * a.k_sn + c, vb + slot0 * 16);
    }
  }

  static __device__ void run(const BwdArgs& a, char* k0, char* v0, char* k1, char* v1) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, l32 = lane & 31;

    const int nqb = (a.Nq + ROWS - 1) / ROWS;
    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    int qblk = wid % nqb;
    const int bh = wid / nqb;
    const int h = bh % a.Hq, b = bh / a.Hq;
    if (CAUSAL) qblk = nqb - 1 - qblk;
    const int g = h / a.group;
    const int q_blk0 = qblk * ROWS;
    const int q_w0 = q_blk0 + wave * 32;
    const int qrow = q_w0 + l32;

    int kv_limit = a.Nk;
    if (a.kv_lens) kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
    int kv_end = kv_limit;
    if (CAUSAL) kv_end = min(kv_end, min(q_blk0 + ROWS, a.Nq));
    const int n_tiles = (kv_end + BC - 1) / BC;
    const int n_act = CAUSAL ? min(n_tiles, (q_w0 + 31) / BC + 1) : n_tiles;

    H8 qf[KS];
    V8 df[KS];
    const int crow = min(qrow, a.Nq - 1);
    {
      const T* qp = (const T*)a.q + b * a.q_sb + h * a.q_sh + crow * a.q_sn;
      const T* dp = (const T*)a.dout + b * a.q_sb + h * a.q_sh + crow * a.q_sn;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + hl * 8;
        qf[ks] = d0 < a.d ? to_f16x8<E>(*(const V8*)(qp + d0)) : H8{};
        df[ks] = d0 < a.d ? *(const V8*)(dp + d0) : V8{};
      }
    }
    const int64_t rid = ((int64_t)b * a.Hq + h) * a.Nq + crow;
    const float lse = a.lse[rid];
    const float nl2 = (qrow < a.Nq && lse != -INFINITY) ? -lse * kLog2e : -INFINITY;
    f32x16 acc_a[DT], acc_b[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc_a[dt] = f32x16{};
      acc_b[dt] = f32x16{};
    }
    float dsum = 0.f;

    const T* kp = (const T*)a.k + b * a.k_sb + g * a.k_sh;
    const T* vp = (const T*)a.v + b * a.k_sb + g * a.k_sh;
    if (n_tiles > 0) issue(a, kp, vp, 0, k0, v0, wave, lane);
    for (int j = 0; j < n_tiles; ++j) {
      char* kc = (j & 1) ? k1 : k0;
      const char* vc = (j & 1) ? v1 : v0;
      __builtin_amdgcn_s_waitcnt(0);
      convert_own_slots<E, SPW, NW>(kc, wave, lane);
      __syncthreads();
      if (j + 1 < n_tiles) issue(a, kp, vp, (j + 1) * BC, (j & 1) ? k0 : k1, (j & 1) ? v0 : v1, wave, lane);
      if (j >= n_act) continue;
      const int j0 = j * BC;
      f32x16 s[KB], dp[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        s[k] = f32x16{};
        dp[k] = f32x16{};
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          const int row = k * 32 + l32;
          const int c = ((ks * 2 + hl) ^ swz_k<CPR>(row)) << 4;
          s[k] = FP16::mfma(lds_read16<H8>(kc + row * (D * 2) + c), qf[ks], s[k]);
          dp[k] = E::mfma(lds_read16<V8>(vc + row * (D * 2) + c), df[ks], dp[k]);
        }
      H8 pf[PT], xf[PT];
#pragma unroll
      for (int t = 0; t < PT; ++t) {
        const int k = t >> 1, r0 = (t & 1) * 8;
        float pv[8], xv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = r0 + e;
          const int key = j0 + k * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          const bool vis = key < kv_limit && (!CAUSAL || key <= qrow);
          pv[e] = vis ? fast_exp2(__builtin_fmaf(s[k][r], a.c, nl2)) : 0.f;
          xv[e] = pv[e] * dp[k][r];
          dsum += xv[e];
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f16x2 p2 = FP16::cvt2(pv[e], pv[e + 1]);
          const f16x2 x2 = FP16::cvt2(xv[e], xv[e + 1]);
          pf[t][e] = p2[0];
          pf[t][e + 1] = p2[1];
          xf[t][e] = x2[0];
          xf[t][e + 1] = x2[1];
        }
      }
      // A^T += K^T X^T, B^T += K^T P^T (K^T read transposed from the tile)
      const int grp = lane >> 4, gi = lane & 15;
#pragma unroll
      for (int t = 0; t < PT; ++t)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int row = t * 16 + 4 * (grp >> 1) + (gi >> 2);
          const int col = dt * 32 + 16 * (grp & 1) + 4 * (gi & 3);
          const int chunk = col >> 3, within = (col & 7) * 2;
          const H4 lo = lds_read_tr4<H4>(kc + row * (D * 2) + ((chunk ^ swz_k<CPR>(row)) << 4) + within);
          const int row2 = row + 8;
          const H4 hi = lds_read_tr4<H4>(kc + row2 * (D * 2) + ((chunk ^ swz_k<CPR>(row2)) << 4) + within);
          const H8 kt = concat4<H8, H4>(lo, hi);
          acc_a[dt] = FP16::mfma(kt, xf[t], acc_a[dt]);
          acc_b[dt] = FP16::mfma(kt, pf[t], acc_b[dt]);
        }
    }

    const float dtot = add_with_other_half(dsum);
    if (qrow >= a.Nq) return;
    if (hl == 0) {
      const int64_t wid_row = ((int64_t)b * a.Hq + h) * a.ld_rows + qrow;
      a.delta[wid_row] = dtot;
      a.nl2[wid_row] = nl2;
    }
    const int64_t base = b * a.q_sb + h * a.q_sh + qrow * a.q_sn;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = dt * 32 + gq * 8 + hl * 4;
        if (col >= a.d) continue;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = a.scale * (acc_a[dt][gq * 4 + e] - dtot * acc_b[dt][gq * 4 + e]);
        if (a.grad_f32) {
          f32x4 w = {x[0], x[1], x[2], x[3]};
          *(f32x4*)((float*)a.dq + base + col) = w;
        } else {
          auto lo = E::cvt2(x[0], x[1]), hi = E::cvt2(x[2], x[3]);
          *(typename E::V4*)((T*)a.dq + base + col) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
        }
      }
  }
};

template <class E, int D, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void bwd_q_kernel(BwdArgs a) {
  using K = BwdQ<E, D, NW, BC, CAUSAL>;
  __shared__ __attribute__((aligned(1024))) char k0[K::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[K::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[K::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[K::TILE_BYTES];
  K::run(a, k0, v0, k1, v1);
}

// ---------------------------------------------------------- dK / dV kernel
// One work-group of NW waves per (batch, kv-head, block of NW*32 keys,
// chunk of q-heads); each wave owns 32 keys, whose K and V fragments (fp16)
// stay in registers.  Q and dO tiles of BR rows stream through LDS (converted
// to fp16 there).  Per 32-row sub-block and wave:
//   S  = Q K^T, dP = dO V^T      32x32x16 MFMA, A = Q / dO rows from LDS,
//                                B = K^T / V^T from registers; each lane holds
//                                16 query rows of one key
//   P, dS = P (dP - D)           per element, D and nl2 from the dQ kernel
//   dV += P^T dO, dK += dS^T Q   32x32x16 MFMA, A = P^T / dS^T from the same
//                                registers (query slots matched), B = dO / Q
//                                read transposed from LDS
template <class E, int D, int NW, int BR, bool CAUSAL>
struct BwdKV {
  static constexpr int KEYS = NW * 32;
  static constexpr int CPR = D / 8;
  static constexpr int TILE_BYTES = BR * D * 2;
  static constexpr int SPW = BR * CPR / (NW * 64);
  static constexpr int QB = BR / 32;
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static_assert(BR * CPR % (NW * 64) == 0, "tile must split evenly into DMA slots");

  using T = typename E::T;
  using V8 = typename E::V8;
  using H8 = f16x8;
  using H4 = f16x4;

  // Q and dO tile rows q0..q0+BR-1 of head h, rows clamped onto valid memory
  // (rows >= Nq get P = 0 below), and the tile's nl2 and D rows (16 bytes =
  // 4 rows per lane: lanes 0..BR/4-1 nl2, the next BR/4 lanes D) into sb.
  static __device__ __forceinline__ void issue(const BwdArgs& a, int b, int h, int q0, char* qb,
                                               char* db, char* sb, int wave, int lane) {
    if (wave == 0 && lane < BR / 2) {
      // rows q0 .. q0+BR-1 lie inside the head's ld_rows-long block
      const float* src = (lane < BR / 4 ? a.nl2 : a.delta) + ((int64_t)b * a.Hq + h) * a.ld_rows +
                         q0 + (lane % (BR / 4)) * 4;
      dma16(src, sb);
    }
    const T* qp = (const T*)a.q + b * a.q_sb + h * a.q_sh;
    const T* dp = (const T*)a.dout + b * a.q_sb + h * a.q_sh;
    const int dch = a.d / 8;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int slot0 = (i * NW + wave) * 64;
      const int s = slot0 + lane;
      const int row = s / CPR, p = s % CPR;
      const int64_t grow = min(q0 + row, a.Nq - 1);
      const int c = min(p ^ swz_k<CPR>(row), dch - 1) * 8;
      dma16(qp + grow * a.q_sn + c, qb + slot0 * 16);
      dma16(dp + grow * a.q_sn + c, db + slot0 * 16);
    }
  }

  // A operand: row `row` of the tile, chunk 2 ks + hl (row pattern).
  static __device__ __forceinline__ H8 rowfrag(const char* buf, int row, int ks, int hl) {
    return lds_read16<H8>(buf + row * (D * 2) + (((ks * 2 + hl) ^ swz_k<CPR>(row)) << 4));
  }
  // B operand read transposed: query slots of k-step t, d-tile dt.
  static __device__ __forceinline__ H8 trfrag(const char* buf, int qbase, int t, int dt, int lane) {
    const int grp = lane >> 4, gi = lane & 15;
    const int row = qbase + t * 16 + 4 * (grp >> 1) + (gi >> 2);
    const int col = dt * 32 + 16 * (grp & 1) + 4 * (gi & 3);
    const int chunk = col >> 3, within = (col & 7) * 2;
    const H4 lo = lds_read_tr4<H4>(buf + row * (D * 2) + ((chunk ^ swz_k<CPR>(row)) << 4) + within);
    const int row2 = row + 8;
    const H4 hi = lds_read_tr4<H4>(buf + row2 * (D * 2) + ((chunk ^ swz_k<CPR>(row2)) << 4) + within);
    return concat4<H8, H4>(lo, hi);
  }

  static __device__ void run(const BwdArgs& a, char* q0b, char* q1b) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, l32 = lane & 31;

    // block -> (key block, chunk, kv-head, batch)
    const int nkb = (a.Nk + KEYS - 1) / KEYS;
    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    const int kblk = wid % nkb;
    int rest = wid / nkb;
    const int chunk = rest % a.kv_chunks;
    rest /= a.kv_chunks;
    const int g = rest % a.Hkv;
    const int b = rest / a.Hkv;
    const int key0 = kblk * KEYS;
    const int kw0 = key0 + wave * 32;
    const int key = kw0 + l32;

    int kv_limit = a.Nk;
    if (a.kv_lens) kv_limit = min(max(a.kv_lens[b], 0), a.Nk);

    // K^T and V^T fragments of this lane's key, fp16 (zero beyond d)
    H8 kf[KS], vf[KS];
    {
      const int krow = min(key, a.Nk - 1);
      const T* kp = (const T*)a.k + b * a.k_sb + g * a.k_sh + krow * a.k_sn;
      const T* vp = (const T*)a.v + b * a.k_sb + g * a.k_sh + krow * a.k_sn;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + hl * 8;
        kf[ks] = d0 < a.d ? to_f16x8<E>(*(const V8*)(kp + d0)) : H8{};
        vf[ks] = d0 < a.d ? to_f16x8<E>(*(const V8*)(vp + d0)) : H8{};
      }
    }
    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dk[dt] = f32x16{};
      dv[dt] = f32x16{};
    }

    // query rows that can see some key of this block
    const int q_start = CAUSAL ? (key0 / BR) * BR : 0;
    const int n_qt = (key0 < kv_limit && q_start < a.Nq) ? (a.Nq - q_start + BR - 1) / BR : 0;
    const int HS = a.group / a.kv_chunks;
    const int h0 = g * a.group + chunk * HS;
    const int n_t = n_qt * HS;   // (head, q-tile) pairs, head-major

    // stage buffers: [Q tile | dO tile | nl2, D] each
    char* const sbuf[2] = {q0b + 2 * TILE_BYTES, q1b + 2 * TILE_BYTES};
    if (n_t > 0) issue(a, b, h0, q_start, q0b, q0b + TILE_BYTES, sbuf[0], wave, lane);
    int q0 = q_start;              // tile t (its head needs no tracking here)
    int hn = h0, qn = q_start;     // tile t + 1
    for (int t = 0; t < n_t; ++t) {
      char* qc = (t & 1) ? q1b : q0b;
      char* dc = qc + TILE_BYTES;
      const char* sc = sbuf[t & 1];
      __builtin_amdgcn_s_waitcnt(0);
      convert_own_slots<E, SPW, NW>(qc, wave, lane);
      convert_own_slots<E, SPW, NW>(dc, wave, lane);
      __syncthreads();
      qn += BR;
      if (qn >= a.Nq) {
        qn = q_start;
        ++hn;
      }
      if (t + 1 < n_t) {
        char* qx = (t & 1) ? q0b : q1b;
        issue(a, b, hn, qn, qx, qx + TILE_BYTES, sbuf[(t + 1) & 1], wave, lane);
      }
      const int qt0 = q0;
      q0 = qn;
      if (CAUSAL && qt0 + BR - 1 < kw0) continue;  // no row of the tile sees this wave's keys
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = FP16::mfma(rowfrag(qc, qb * 32 + l32, ks, hl), kf[ks], s);
          dp = FP16::mfma(rowfrag(dc, qb * 32 + l32, ks, hl), vf[ks], dp);
        }
        // rows of register r: qt0 + qb*32 + (r/4)*8 + 4 hl + r%4
        H8 pp[2], dsp[2];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int lr = qb * 32 + gq * 8 + hl * 4;   // local row of e = 0
          const f32x4 nl = *(const LDS_AS f32x4*)(const LDS_AS void*)(sc + lr * 4);
          const f32x4 dd = *(const LDS_AS f32x4*)(const LDS_AS void*)(sc + BR * 4 + lr * 4);
          float pv[4], dsv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = gq * 4 + e;
            const int qr = qt0 + lr + e;
            const bool vis = key < kv_limit && qr < a.Nq && (!CAUSAL || key <= qr);
            const float p = fast_exp2(__builtin_fmaf(s[r], a.c, nl[e]));
            pv[e] = vis ? p : 0.f;
            dsv[e] = vis ? p * (dp[r] - dd[e]) : 0.f;
          }
          const int t2 = gq >> 1, half = (gq & 1) * 4;
          const f16x2 p01 = FP16::cvt2(pv[0], pv[1]), p23 = FP16::cvt2(pv[2], pv[3]);
          const f16x2 s01 = FP16::cvt2(dsv[0], dsv[1]), s23 = FP16::cvt2(dsv[2], dsv[3]);
          pp[t2][half + 0] = p01[0];
          pp[t2][half + 1] = p01[1];
          pp[t2][half + 2] = p23[0];
          pp[t2][half + 3] = p23[1];
          dsp[t2][half + 0] = s01[0];
          dsp[t2][half + 1] = s01[1];
          dsp[t2][half + 2] = s23[0];
          dsp[t2][half + 3] = s23[1];
        }
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            dv[dt] = FP16::mfma(pp[t2], trfrag(dc, qb * 32, t2, dt, lane), dv[dt]);
            dk[dt] = FP16::mfma(dsp[t2], trfrag(qc, qb * 32, t2, dt, lane), dk[dt]);
          }
      }
    }

    // Store: lane holds d column dt*32 + l32, keys kw0 + (r/4)*8 + 4 hl + r%4.
    if (kw0 >= a.Nk) return;
    const bool direct = a.kv_chunks == 1;
    const int64_t part = (int64_t)a.B * a.Hkv * a.Nk * a.d;  // one partial tensor
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int col = dt * 32 + l32;
      if (col >= a.d) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = kw0 + (r >> 2) * 8 + hl * 4 + (r & 3);
        if (kr >= a.Nk) continue;
        const int64_t off = b * a.k_sb + g * a.k_sh + kr * a.k_sn + col;
        const float kval = dk[dt][r] * a.scale, vval = dv[dt][r];
        if (!direct) {
          a.part_dk[chunk * part + off] = kval;
          a.part_dv[chunk * part + off] = vval;
        } else if (a.grad_f32) {
          ((float*)a.dk)[off] = kval;
          ((float*)a.dv)[off] = vval;
        } else {
          ((T*)a.dk)[off] = (T)kval;
          ((T*)a.dv)[off] = (T)vval;
        }
      }
    }
  }
};

template <class E, int D, int NW, int BR, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void bwd_kv_kernel(BwdArgs a) {
  using K = BwdKV<E, D, NW, BR, CAUSAL>;
  // per stage: Q tile | dO tile | nl2 and D of the tile's rows
  __shared__ __attribute__((aligned(1024))) char s0[2 * K::TILE_BYTES + 2 * BR * 4];
  __shared__ __attribute__((aligned(1024))) char s1[2 * K::TILE_BYTES + 2 * BR * 4];
  K::run(a, s0, s1);
}

// Sum of the per-chunk partial dK / dV in a fixed order (deterministic).
template <class T>
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(BwdArgs a) {
  const int64_t n = (int64_t)a.B * a.Hkv * a.Nk * a.d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float sk = 0.f, sv = 0.f;
    for (int c = 0; c < a.kv_chunks; ++c) {
      sk += a.part_dk[c * n + i];
      sv += a.part_dv[c * n + i];
    }
    if (a.grad_f32) {
      ((float*)a.dk)[i] = sk;
      ((float*)a.dv)[i] = sv;
    } else {
      ((T*)a.dk)[i] = (T)sk;
      ((T*)a.dv)[i] = (T)sv;
    }
  }
}

}  // namespace attn
