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
// (11-bit significand) rather than bf16.  For bf16 inputs a first pass
// (bwd_prep_kernel) writes fp16 copies of Q, dO and K (exact for |x| in
// [2^-14, 65504]); the tiles of those copies then go to LDS unchanged.
// Exponentials are exp2 with the scale and log2(e) folded in:
// P = exp2(s * c + nl2), with nl2 = -LSE * log2(e) (-inf for a fully masked
// row and for the padding rows past Nq, so that P = 0 there).
//
// Tiles of 128 rows (dK/dV) or keys (dQ) stream through LDS, double-
// buffered, filled by direct buffer->LDS loads (rows or columns past the
// tensor read as zero).  At D = 128 the 16-byte chunks of a row are XOR-
// swizzled (SwzTile), which keeps both the row-fragment reads and the
// transposed reads free of bank conflicts; at D = 64 rows are padded to
// D/8 + 1 slots (PadTile: row reads conflict-free, transposed reads sharing
// banks pairwise).  Every read address is a per-lane base plus a
// compile-time offset.
//
// Both kernels run a tile as a fixed software pipeline over its four 32-row
// (32-key) sub-blocks, one wave per SIMD: the S/dP products of sub-block i
// are issued while the dV/dK (A/B) products of sub-block i-1 run beside the
// exponentials of sub-block i, and each LDS operand is read PF products
// ahead.  Masking costs no per-element work in the loop: on a tile with
// excluded keys (causal, and in the dQ kernel also keys past kv_lens) the S
// accumulator of a sub-block starts at -inf where a key is excluded and 0
// elsewhere, so P = 0 and dS = 0 there; other tiles start from the MFMA's
// zero operand.  The dK/dV kernel leaves keys past kv_lens unmasked: their
// P and dS reach only their own rows of dK and dV, which it stores as zero.
//
// Local attention (LOCAL: window and/or 2-D neighbourhood, causal folded into
// the window; local_mask.h) uses the same start pattern, taken from the
// 64-bit visibility words of the lane's row (dQ kernel) or, with queries and
// keys exchanged, of its key (dK/dV kernel); tiles outside a block's reach
// are skipped whole.  SOFTCAP recomputes the capped logit
// t = cap tanh(scale s / cap) (in log2 units) for P and multiplies dS by the
// cap's derivative 1 - tanh^2 = 4 r (1 - r), r = 1 / (1 + e^(2 scale s / cap));
// a masked score (-inf) is kept at -inf, since the cap would map it to -cap.
#pragma once

#include <type_traits>
#include <utility>

#include "attn_kernels.h"
#include "device_common.h"
#include "local_mask.h"


namespace attn {


// Register placement.  These kernels need more than the 256 VGPRs of a
// wave, so part of their state lives in AGPRs, which only the matrix cores
// read and write directly.  The fragments a kernel keeps for its whole
// life (K and V in the dK/dV kernel, Q and dO in the dQ kernel) are only
// ever MFMA A/B operands, which may come from AGPRs; pin_agpr places them
// there.  The sources are compiled with the MFMA results in VGPRs
// (-amdgpu-mfma-vgpr-form, set by build.py), so S, dP and the gradient
// accumulators, which the vector code reads, stay in VGPRs and no
// AGPR->VGPR copy is issued per element.
template <class V, int N>
__device__ __forceinline__ void pin_agpr(V (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(x[i]));
}

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

// Power-of-two scales of the fp16 operands of a bf16 backward.  The fp16
// copies hold sq Q, sk K, sdo dO and (in registers) sv V, each scale chosen
// from the tensor's largest magnitude so that the copy is exact and the
// products that are rounded to fp16 stay in its range:
//   S' = sq sk S          -> the exponent takes c / (sq sk);
//   dP' = sdo sv dP       -> X = P dP' and dS' = P (dP' - D') stay below
//                            128 * 8 * 8 = 8192 for d <= 128;
//   dQ = scale / (sk sdo sv) (A' - D' B'),  dK = scale / (sdo sv sq) dK',
//   dV = dV' / sdo.
// Scaling by powers of two is exact, so inputs already in range (scale 1)
// give the unscaled results bit for bit.  fp16 inputs use every scale = 1.
struct BwdScales {
  float q, k, v, dout;
};
__device__ __forceinline__ BwdScales bwd_scales(const BwdArgs& a) {
  if (!a.escale) return {1.f, 1.f, 1.f, 1.f};
  return {a.escale[0], a.escale[1], a.escale[2], a.escale[3]};
}

// 2^(target - t) for a tensor whose largest magnitude amax has binary
// exponent t outside [lo, hi] (1 inside it, or for a zero / non-finite
// amax); the exponent shift is clamped to +-40 so that products of three
// scales stay normal fp32 numbers.
__device__ __forceinline__ float pow2_scale(float amax, int lo, int hi, int target) {
  if (!(amax > 0.f) || !(amax < INFINITY)) return 1.f;
  const int t = __builtin_amdgcn_frexp_expf(amax) - 1;   // amax in [2^t, 2^(t+1))
  if (t >= lo && t <= hi) return 1.f;
  return __builtin_amdgcn_ldexpf(1.f, max(-40, min(40, target - t)));
}
// Q and K: largest magnitude kept in [2^-6, 2^14), else moved to [2^13, 2^14);
// dO and V: kept in [2^-6, 8), else moved to [4, 8).
constexpr int kQkLo = -6, kQkHi = 13, kQkTarget = 13;
constexpr int kDvLo = -6, kDvHi = 2, kDvTarget = 2;

// 8 x 16-bit input values times a power of two -> 8 x fp16.
template <class E>
__device__ __forceinline__ f16x8 to_f16x8_scaled(typename E::V8 x, float s) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  if constexpr (std::is_same<E, FP16>::value) {
    return x;
  } else {
    return __builtin_convertvector(__builtin_convertvector(x, f32x8) * s, f16x8);
  }
}
// 8 x bf16 values times a power of two, still bf16 (exact); fp16 unchanged.
template <class E>
__device__ __forceinline__ typename E::V8 scale_v8(typename E::V8 x, float s) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  if constexpr (std::is_same<E, FP16>::value) {
    return x;
  } else {
    return __builtin_convertvector(__builtin_convertvector(x, f32x8) * s, typename E::V8);
  }
}

// A tile of R rows x D columns (16-bit) in LDS, loaded by NW waves.
template <int R, int D, int NW>
struct PadTile {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int PS = CPR + 1;                // LDS slots per row (one pad)
  static constexpr int P = PS * 16;                 // pitch in bytes
  static constexpr int BYTES = R * P;
  static constexpr int INS = (R * PS + 63) / 64;    // load instructions per tile
  static constexpr int IPW = (INS + NW - 1) / NW;   // ... per wave

  // Byte offset in a tile of row stride sn elements of the chunk lane `lane`
  // copies in load instruction `ins`; pad slots and columns past d get an
  // out-of-range offset (they load zero).
  static __device__ __forceinline__ uint32_t offset(int ins, int lane, int dchunks, int64_t sn) {
    const int s = ins * 64 + lane;
    const int r = s / PS, ch = s % PS;
    if (r >= R || ch >= dchunks) return kBufOutOfRange;
    return (uint32_t)((r * sn + ch * 8) * 2);
  }
  static __device__ __forceinline__ void load(BufRsrc rs, const uint32_t (&off)[IPW], char* buf,
                                              int wave) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int ins = i * NW + wave;
      if (ins < INS) dma16_buf(rs, off[i], buf + ins * 1024);
    }
  }
  // Lane bases: row fragment (row l32, chunk hl) and transposed read (row
  // 4 (group / 2) + i / 4, column 16 (group % 2) + 4 (i % 4) for lane i of
  // 16-lane group `group`).
  struct Bases {
    int rb, tb;
  };
  static __device__ __forceinline__ Bases bases(int lane) {
    const int l32 = lane & 31, hl = lane >> 5, grp = lane >> 4, gi = lane & 15;
    return {l32 * P + hl * 16,
            (4 * (grp >> 1) + (gi >> 2)) * P + (16 * (grp & 1) + 4 * (gi & 3)) * 2};
  }
  // MFMA operand from rows r0 + (lane % 32), k-step ks (d = 16 ks + 8 hl ..).
  template <class V8>
  static __device__ __forceinline__ V8 row(const char* buf, const Bases& b, int r0, int ks) {
    return lds_read16<V8>(buf + b.rb + r0 * P + ks * 32);
  }
  // MFMA operand read transposed: column dt*32 + lane%32, rows r0 + slot
  // order 8 (s / 4) + 4 hl + s % 4 for slot s.
  template <class V8, class V4>
  static __device__ __forceinline__ V8 tr(const char* buf, const Bases& b, int r0, int dt) {
    const char* p = buf + b.tb + r0 * P + dt * 64;
    const V4 lo = lds_read_tr4<V4>(p);
    const V4 hi = lds_read_tr4<V4>(p + 8 * P);
    return concat4<V8, V4>(lo, hi);
  }
};

// The same tile for D = 128 without padding: rows of 16 chunks of 16 bytes,
// chunk c of row r stored at position c ^ f(r), f(r) = 4 (r % 4) + (r / 4) % 4.
// The 16 rows of a row-fragment read land on 16 distinct chunk positions, and
// so do the 4 rows x 4 chunks of a transposed read by 32 lanes: both are
// free of bank conflicts.  The XOR is folded into per-lane bases (one per
// k-step, and per 32-column block and half of a transposed read), since
// r0 is a multiple of 16 in every read.
template <int R, int NW>
struct SwzTile {
  static constexpr int D = 128;
  static constexpr int CPR = 16;
  static constexpr int P = 256;                     // pitch in bytes
  static constexpr int BYTES = R * P;
  static constexpr int INS = R * CPR / 64;          // load instructions per tile
  static constexpr int IPW = (INS + NW - 1) / NW;
  static __host__ __device__ constexpr int f(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

  static __device__ __forceinline__ uint32_t offset(int ins, int lane, int dchunks, int64_t sn) {
    const int s = ins * 64 + lane;
    const int r = s >> 4, lc = (s & 15) ^ f(r & 15);
    if (r >= R || lc >= dchunks) return kBufOutOfRange;
    return (uint32_t)((r * sn + lc * 8) * 2);
  }
  static __device__ __forceinline__ void load(BufRsrc rs, const uint32_t (&off)[IPW], char* buf,
                                              int wave) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int ins = i * NW + wave;
      if (ins < INS) dma16_buf(rs, off[i], buf + ins * 1024);
    }
  }
  struct Bases {
    int rb[8];        // row fragment, k-step ks
    int tb[4][2];     // transposed read, 32-column block dt, rows +0 / +8
  };
  static __device__ __forceinline__ Bases bases(int lane) {
    const int l32 = lane & 31, hl = lane >> 5, grp = lane >> 4, gi = lane & 15;
    Bases b;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) b.rb[ks] = l32 * P + (((2 * ks + hl) ^ f(l32 & 15)) << 4);
    const int rr = 4 * (grp >> 1) + (gi >> 2);           // row within 16
    const int lc = 2 * (grp & 1) + ((gi & 3) >> 1);      // chunk within a 64-byte block
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        b.tb[dt][h] = (rr + 8 * h) * P + (((dt * 4 + lc) ^ f(rr + 8 * h)) << 4) + (gi & 1) * 8;
    return b;
  }
  template <class V8>
  static __device__ __forceinline__ V8 row(const char* buf, const Bases& b, int r0, int ks) {
    return lds_read16<V8>(buf + b.rb[ks] + r0 * P);
  }
  template <class V8, class V4>
  static __device__ __forceinline__ V8 tr(const char* buf, const Bases& b, int r0, int dt) {
    const V4 lo = lds_read_tr4<V4>(buf + b.tb[dt][0] + r0 * P);
    const V4 hi = lds_read_tr4<V4>(buf + b.tb[dt][1] + r0 * P);
    return concat4<V8, V4>(lo, hi);
  }
};

template <int R, int D, int NW>
using BwdTile = typename std::conditional<D == 128, SwzTile<R, NW>, PadTile<R, D, NW>>::type;

// --------------------------------------------------------------- dQ kernel
// One work-group of NW waves per (batch, q-head, block of NW*32 rows); each
// wave owns 32 rows, whose Q (as fp16) and dO fragments stay in registers.
// Tiles of BC keys of K (its fp16 copy) and V stream through LDS.  Per
// 32-key block of a tile and wave:
//   S^T = K Q^T, dP^T = V dO^T        32x32x16 MFMA; each lane holds 16 keys
//                                     of one row
//   P^T, X^T = P^T * dP^T, D += X     per element
//   A^T += K^T X^T, B^T += K^T P^T    32x32x16 fp16 MFMA, K^T read transposed
//                                     from LDS, X^T / P^T from registers
// Epilogue: dQ = scale (A - D B); D and nl2 to the workspace.
template <class E, int D, int NW, int BC, bool CAUSAL, bool MASK, bool LOCAL = false,
          bool SOFTCAP = false>
struct BwdQ {
  static_assert(!(LOCAL && CAUSAL), "causal masking is part of the window under LOCAL");
  static_assert(!LOCAL || BC == 128, "LOCAL masks a tile through two 64-bit words");
  using TL = BwdTile<BC, D, NW>;
  static constexpr int ROWS = NW * 32;
  static constexpr int KB = BC / 32;
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int PF = 3;                // LDS operand read-ahead, in MFMAs

  using T = typename E::T;
  using V8 = typename E::V8;
  using H8 = f16x8;
  using H4 = f16x4;

  struct State {
    int lane, wave, hl, l32;
    int q_w0, qrow, kv_limit;
    typename TL::Bases lb;      // LDS lane bases
    const char* kp;             // K / V of this (batch, kv-head), key 0
    const char* vp;
    int64_t tile_bytes, end_bytes;
    uint32_t off[TL::IPW];
    float c, nl2;
    const float* mrow;          // additive mask row of this lane's query (MASK)
    int nk1;                    // Nk - 1
    int t_lo, t_hi;             // LOCAL: this wave's key tiles [t_lo, t_hi)
    LocalVis::Row lrow;         // LOCAL: this lane's query position
    float cap_a, cap_c2;        // SOFTCAP constants
    float dq_scale;             // scale / (sk sdo sv)
    H8 qf[KS];
    V8 df[KS];
    f32x16 acc_a[DT], acc_b[DT];
    float dsum[4];
  };

  static __device__ __forceinline__ void issue(const State& st, int j, char* kb, char* vb) {
    const int64_t o = (int64_t)j * st.tile_bytes;
    const uint32_t n = (uint32_t)min(st.end_bytes - o, (int64_t)kBufLimit);
    TL::load(make_rsrc(st.kp + o, n), st.off, kb, st.wave);
    TL::load(make_rsrc(st.vp + o, n), st.off, vb, st.wave);
  }

  // ---- software-pipelined tile: blocks of MFMAs per 32-key block k ----
  //   SD(0) | p/x(0) | SD(1) | GR(0)+p/x(1) | ... | SD(KB-1) | GR(KB-2)+p/x(KB-1) | GR(KB-1)
  // SD(k): the 2 KS S^T / dP^T MFMAs of key block k; GR(k): its 4 DT A^T /
  // B^T MFMAs (each transposed K^T fragment feeds one A^T and one B^T MFMA);
  // 16 each at d = 128.
  static constexpr int NBLK = 2 * KB + 1;
  static constexpr int SDN = 2 * KS;   // MFMAs of an SD block
  static constexpr int GRN = 4 * DT;   // MFMAs of a GR block
  static __host__ __device__ constexpr int blk_len(int b) {
    return (b % 2 == 0) ? (b / 2 < KB ? SDN : GRN) : (b == 1 ? 0 : GRN);
  }
  static __host__ __device__ constexpr int blk_start(int b) {
    int s = 0;
    for (int q = 0; q < b; ++q) s += blk_len(q);
    return s;
  }
  static constexpr int NSLOT = KB * (SDN + GRN);
  static __host__ __device__ constexpr int slot_blk(int s) {
    int b = 0;
    for (int q = 0; q < NBLK; ++q)
      if (blk_len(q) > 0 && blk_start(q) <= s) b = q;
    return b;
  }
  static __host__ __device__ constexpr int slot_kind(int s) {
    const int b = slot_blk(s);
    return (b % 2 == 0 && b / 2 < KB) ? 0 : 1;
  }
  static __host__ __device__ constexpr int slot_sub(int s) {
    const int b = slot_blk(s);
    return slot_kind(s) == 0 ? b / 2 : (b % 2 == 1 ? (b - 1) / 2 - 1 : KB - 1);
  }
  static __host__ __device__ constexpr int slot_m(int s) { return s - blk_start(slot_blk(s)); }
  static __host__ __device__ constexpr int group_slot(int k, int g) {
    return k == 0 ? blk_start(2) : blk_start(2 * k + 1) + g * (GRN / 4);
  }
  // does slot s read an LDS operand (transposed K^T fragments are read once
  // for a pair of MFMAs)
  static __host__ __device__ constexpr bool slot_reads(int s) {
    return slot_kind(s) == 0 || (slot_m(s) & 1) == 0;
  }

  struct Pipe {
    const char* kc;
    const char* vc;
    int lim;                    // keys with offset > lim are masked (see pipe_slot)
    bool msk;                   // the tile has masked keys for this wave
    int j0;                     // first key of the tile
    uint32_t lw[KB];            // LOCAL: visibility words per key block (bit 8 (r/4) + r%4)
    float mv[KB][16];           // additive mask values per key block (MASK)
    f32x16 s, dp;
    H8 pf[2][2], xf[2][2];
    H8 opd[NSLOT];
    V8 opv[NSLOT];
  };
  template <int SL>
  static __device__ __forceinline__ void pipe_load(const State& st, Pipe& c) {
    if constexpr (SL < NSLOT && slot_reads(SL)) {
      constexpr int k = slot_sub(SL), m = slot_m(SL);
      if constexpr (slot_kind(SL) == 0) {
        if constexpr (m & 1) c.opv[SL] = TL::template row<V8>(c.vc, st.lb, k * 32, m >> 1);
        else c.opd[SL] = TL::template row<H8>(c.kc, st.lb, k * 32, m >> 1);
      } else {
        c.opd[SL] = TL::template tr<H8, H4>(c.kc, st.lb, k * 32 + (m / (2 * DT)) * 16, (m >> 1) % DT);
      }
    }
  }
  // Additive mask values of key block K for this lane's row: register r
  // holds key j0 + 32 K + 8 (r / 4) + 4 hl + r % 4 (clamped to the last key;
  // keys past Nk are excluded through S anyway).
  template <int K>
  static __device__ __forceinline__ void pipe_mask(const State& st, Pipe& c) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      c.mv[K][r] = st.mrow[min(c.j0 + K * 32 + (r >> 2) * 8 + st.hl * 4 + (r & 3), st.nk1)];
  }
  template <int K, int GQ>
  static __device__ __forceinline__ void pipe_group(State& st, Pipe& c) {
    constexpr int par = K & 1;
    float pv[4], xv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // P = exp2(s c + mask log2(e) - LSE log2(e))
      const float ml = MASK ? __builtin_fmaf(c.mv[K][GQ * 4 + e], kLog2e, st.nl2) : st.nl2;
      if constexpr (SOFTCAP) {
        // D sums P dP; the products take P g and P g dP (dS = P g (dP - D))
        float g;
        const float t = softcap_grad(c.s[GQ * 4 + e], st.cap_a, st.cap_c2, g);
        const float p = fast_exp2(t + ml);
        const float x = p * c.dp[GQ * 4 + e];
        st.dsum[e] += x;
        pv[e] = p * g;
        xv[e] = x * g;
      } else {
        const float p = fast_exp2(__builtin_fmaf(c.s[GQ * 4 + e], st.c, ml));
        pv[e] = p;
        xv[e] = p * c.dp[GQ * 4 + e];
        st.dsum[e] += xv[e];
      }
    }
    constexpr int t2 = GQ >> 1, half = (GQ & 1) * 4;
    const f16x2 p01 = FP16::cvt2(pv[0], pv[1]), p23 = FP16::cvt2(pv[2], pv[3]);
    const f16x2 x01 = FP16::cvt2(xv[0], xv[1]), x23 = FP16::cvt2(xv[2], xv[3]);
    c.pf[par][t2][half + 0] = p01[0];
    c.pf[par][t2][half + 1] = p01[1];
    c.pf[par][t2][half + 2] = p23[0];
    c.pf[par][t2][half + 3] = p23[1];
    c.xf[par][t2][half + 0] = x01[0];
    c.xf[par][t2][half + 1] = x01[1];
    c.xf[par][t2][half + 2] = x23[0];
    c.xf[par][t2][half + 3] = x23[1];
  }
  template <int SL, int K>
  static __device__ __forceinline__ void pipe_groups_of(State& st, Pipe& c) {
    if constexpr (group_slot(K, 0) == SL) pipe_group<K, 0>(st, c);
    if constexpr (group_slot(K, 1) == SL) pipe_group<K, 1>(st, c);
    if constexpr (group_slot(K, 2) == SL) pipe_group<K, 2>(st, c);
    if constexpr (group_slot(K, 3) == SL) pipe_group<K, 3>(st, c);
  }
  template <int PF, int SL>
  static __device__ __forceinline__ void pipe_slot(State& st, Pipe& c) {
    pipe_load<SL + PF>(st, c);
    constexpr int k = slot_sub(SL), m = slot_m(SL), par = k & 1;
    if constexpr (SL == blk_start(2)) {
      pipe_groups_of<SL, 0>(st, c);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MASK && slot_kind(SL) == 0 && m == 0) pipe_mask<k>(st, c);
    if constexpr (slot_kind(SL) == 0) {
      if constexpr (m == 0) {
        // On a tile with masked keys, S^T starts at -inf for keys past the
        // row (causal) or past kv_limit: register r holds key
        // j0 + 32 k + 4 hl + 8 (r / 4) + r % 4, visible iff
        // 32 k + 8 (r / 4) + r % 4 <= lim; 0 elsewhere.  Other tiles start
        // from the MFMA's zero operand.  LOCAL: the same from the
        // visibility word of key block k.
        if (c.msk) {
          f32x16 init;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if constexpr (LOCAL)
              init[r] = keep_if_bit(0.f, c.lw[k], (r >> 2) * 8 + (r & 3));
            else
              init[r] = (k * 32 + (r >> 2) * 8 + (r & 3) <= c.lim) ? 0.f : -INFINITY;
          }
          c.s = FP16::mfma(c.opd[SL], st.qf[0], init);
        } else {
          c.s = FP16::mfma(c.opd[SL], st.qf[0], f32x16{});
        }
      } else if constexpr (m == 1) {
        c.dp = E::mfma(c.opv[SL], st.df[0], f32x16{});
      } else if constexpr (m & 1) {
        c.dp = E::mfma(c.opv[SL], st.df[m >> 1], c.dp);
      } else {
        c.s = FP16::mfma(c.opd[SL], st.qf[m >> 1], c.s);
      }
    } else {
      constexpr int t2 = m / (2 * DT), dt = (m >> 1) % DT;
      if constexpr (m & 1) st.acc_b[dt] = FP16::mfma(c.opd[SL - 1], c.pf[par][t2], st.acc_b[dt]);
      else st.acc_a[dt] = FP16::mfma(c.opd[SL], c.xf[par][t2], st.acc_a[dt]);
    }
    if constexpr (slot_kind(SL) == 1 && slot_blk(SL) % 2 == 1)
      pipe_groups_of<SL, (slot_blk(SL) - 1) / 2>(st, c);
    __builtin_amdgcn_sched_barrier(0);
  }
  template <int PF, int... SL>
  static __device__ __forceinline__ void pipe_slots(State& st, Pipe& c,
                                                    std::integer_sequence<int, SL...>) {
    (pipe_slot<PF, SL>(st, c), ...);
  }
  template <int... SL>
  static __device__ __forceinline__ void pipe_prologue(State& st, Pipe& c,
                                                       std::integer_sequence<int, SL...>) {
    (pipe_load<SL>(st, c), ...);
  }
  // bits: LOCAL visibility of keys j0..j0+63 and j0+64..j0+127 for this
  // lane's row
  template <int PF>
  static __device__ __forceinline__ void pipe_tile(State& st, const char* kc, const char* vc,
                                                   int j0, uint64_t b0, uint64_t b1) {
    Pipe c;
    c.kc = kc;
    c.vc = vc;
    if constexpr (LOCAL) {
#pragma unroll
      for (int k = 0; k < KB; ++k)
        c.lw[k] = (uint32_t)(((k < 2) ? b0 : b1) >> ((k & 1) * 32 + 4 * st.hl));
      c.msk = __builtin_amdgcn_ballot_w64((b0 & b1) != ~0ull) != 0;
    } else {
      const int base = j0 + 4 * st.hl;
      c.lim = st.kv_limit - 1 - base;
      if (CAUSAL) c.lim = min(c.lim, st.qrow - base);
      c.msk = (j0 + BC > st.kv_limit) || (CAUSAL && j0 + BC - 1 > st.q_w0);
    }
    c.j0 = j0;
    pipe_prologue(st, c, std::make_integer_sequence<int, PF>{});
    pipe_slots<PF>(st, c, std::make_integer_sequence<int, NSLOT>{});
  }

  // Iteration j: tile j is in (kc, vc); tile j+1 goes into (kn, vn).
  static __device__ __forceinline__ void step(const BwdArgs& a, State& st, int j, int n,
                                              int n_act, char* kc, const char* vc, char* kn,
                                              char* vn) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < n) issue(st, j + 1, kn, vn);
    if constexpr (LOCAL) {
      if (j < st.t_lo || j >= st.t_hi) return;
      const uint64_t b0 = a.loc.bits(st.lrow, j * BC, st.kv_limit);
      const uint64_t b1 = a.loc.bits(st.lrow, j * BC + 64, st.kv_limit);
      if (!__builtin_amdgcn_ballot_w64((b0 | b1) != 0)) return;   // no visible key
      pipe_tile<PF>(st, kc, vc, j * BC, b0, b1);
    } else {
      if (j >= n_act) return;
      pipe_tile<PF>(st, kc, vc, j * BC, 0, 0);
    }
  }

  static __device__ void run(const BwdArgs& a, char* k0, char* v0, char* k1, char* v1) {
    State st;
    st.lane = threadIdx.x & 63;
    st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    st.hl = st.lane >> 5;
    st.l32 = st.lane & 31;

    const int nqb = (a.Nq + ROWS - 1) / ROWS;
    int qblk, bh;
    block_coords(CAUSAL, blockIdx.x, a.B * a.Hq, nqb, qblk, bh);
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int g = h / a.group;
    const int q_blk0 = qblk * ROWS;
    st.q_w0 = q_blk0 + st.wave * 32;
    st.qrow = st.q_w0 + st.l32;

    st.kv_limit = a.Nk;
    if (a.kv_lens) st.kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
    int kv_end = st.kv_limit;
    if (CAUSAL) kv_end = min(kv_end, min(q_blk0 + ROWS, a.Nq));
    const int n_tiles = (kv_end + BC - 1) / BC;
    const int n_act = CAUSAL ? min(n_tiles, (st.q_w0 + 31) / BC + 1) : n_tiles;

    const int crow = min(st.qrow, a.Nq - 1);
    const BwdScales sc = bwd_scales(a);
    {
      const T* qp = (const T*)a.q + b * a.q_sb + h * a.q_sh + crow * a.q_sn;
      const T* dp = (const T*)a.dout + b * a.q_sb + h * a.q_sh + crow * a.q_sn;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + st.hl * 8;
        st.qf[ks] = d0 < a.d ? to_f16x8_scaled<E>(*(const V8*)(qp + d0), sc.q) : H8{};
        st.df[ks] = d0 < a.d ? scale_v8<E>(*(const V8*)(dp + d0), sc.dout * sc.v) : V8{};
      }
      pin_agpr(st.qf);
      pin_agpr(st.df);
    }
    const float lse = a.lse[((int64_t)b * a.Hq + h) * a.Nq + crow];
    st.nl2 = (st.qrow < a.Nq && lse != -INFINITY) ? -lse * kLog2e : -INFINITY;
    st.nk1 = a.Nk - 1;
    if (MASK) st.mrow = a.mask + b * a.m_sb + h * a.m_sh + (int64_t)crow * a.m_sq;
    st.c = a.c / (sc.q * sc.k);
    st.cap_a = a.cap_a;
    st.cap_c2 = a.cap_c2 / (sc.q * sc.k);
    st.dq_scale = a.scale / (sc.k * sc.dout * sc.v);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      st.acc_a[dt] = f32x16{};
      st.acc_b[dt] = f32x16{};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) st.dsum[i] = 0.f;

    st.kp = (const char*)((const _Float16*)a.k16 + b * a.k_sb + g * a.k_sh);
    st.vp = (const char*)((const T*)a.v + b * a.k_sb + g * a.k_sh);
    st.tile_bytes = (int64_t)BC * a.k_sn * 2;
    // rows past kv_lens read as zero: S = -inf there and dP = 0, whatever
    // those rows hold
    st.end_bytes = max(((int64_t)(st.kv_limit - 1) * a.k_sn + a.d) * 2, (int64_t)0);
    const int dchunks = a.d / 8;
#pragma unroll
    for (int i = 0; i < TL::IPW; ++i)
      st.off[i] = TL::offset(i * NW + st.wave, st.lane, dchunks, a.k_sn);
    st.lb = TL::bases(st.lane);

    // key tiles [t_begin, t_end) pass through LDS
    int t_begin = 0, t_end = n_tiles;
    if constexpr (LOCAL) {
      int lo, hi;
      a.loc.key_range(q_blk0, min(q_blk0 + ROWS, a.Nq) - 1, st.kv_limit, lo, hi);
      t_begin = lo / BC;
      t_end = hi >= lo ? hi / BC + 1 : t_begin;
      st.t_lo = st.t_hi = 0;
      if (st.q_w0 < a.Nq) {
        a.loc.key_range(st.q_w0, min(st.q_w0 + 31, a.Nq - 1), st.kv_limit, lo, hi);
        st.t_lo = lo / BC;
        st.t_hi = hi >= lo ? hi / BC + 1 : st.t_lo;
      }
      st.lrow = a.loc.row(crow);
    }
    if (t_begin < t_end) issue(st, t_begin, k0, v0);
    for (int j = t_begin; j < t_end; j += 2) {
      step(a, st, j, t_end, n_act, k0, v0, k1, v1);
      if (j + 1 >= t_end) break;
      step(a, st, j + 1, t_end, n_act, k1, v1, k0, v0);
    }

    const float dtot = add_with_other_half((st.dsum[0] + st.dsum[1]) + (st.dsum[2] + st.dsum[3]));
    // D and nl2 for every row of the padded workspace (D = 0 and nl2 = -inf
    // past Nq, so the dK/dV pass gets P = 0 there)
    if (st.qrow < a.ld_rows && st.hl == 0) {
      const int64_t wrow = ((int64_t)b * a.Hq + h) * a.ld_rows + st.qrow;
      a.delta[wrow] = st.qrow < a.Nq ? dtot : 0.f;
      a.nl2[wrow] = st.nl2;
    }
    if (st.qrow >= a.Nq) return;
    const int64_t base = b * a.q_sb + h * a.q_sh + st.qrow * a.q_sn;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = dt * 32 + gq * 8 + st.hl * 4;
        if (col >= a.d) continue;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = st.dq_scale * (st.acc_a[dt][gq * 4 + e] - dtot * st.acc_b[dt][gq * 4 + e]);
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

template <class E, int D, int NW, int BC, bool CAUSAL, bool MASK, bool LOCAL = false,
          bool SOFTCAP = false>
__global__ __launch_bounds__(NW * 64) void bwd_q_kernel(BwdArgs a) {
  using K = BwdQ<E, D, NW, BC, CAUSAL, MASK, LOCAL, SOFTCAP>;
  __shared__ __attribute__((aligned(1024))) char k0[K::TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[K::TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[K::TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[K::TL::BYTES];
  K::run(a, k0, v0, k1, v1);
}

// ---------------------------------------------------------- dK / dV kernel
// One work-group of NW waves per (batch, kv-head, block of NW*32 keys,
// chunk of q-heads); each wave owns 32 keys, whose K and V fragments (fp16)
// stay in registers.  Tiles of BR rows of Q and dO (their fp16 copies)
// stream through LDS.  Per 32-row sub-block and wave:
//   S  = Q K^T, dP = dO V^T      32x32x16 MFMA, A = Q / dO rows from LDS,
//                                B = K^T / V^T from registers; each lane holds
//                                16 query rows of one key
//   P, dS = P (dP - D)           per element, D and nl2 from the dQ kernel
//   dV += P^T dO, dK += dS^T Q   32x32x16 MFMA, A = P^T / dS^T from the same
//                                registers (query slots matched), B = dO / Q
//                                read transposed from LDS
template <class E, int D, int NW, int BR, bool CAUSAL, bool MASK, bool LOCAL = false,
          bool SOFTCAP = false>
struct BwdKV {
  static_assert(!(LOCAL && CAUSAL), "causal masking is part of the window under LOCAL");
  static_assert(!LOCAL || BR == 128, "LOCAL masks a tile through two 64-bit words");
  using TL = BwdTile<BR, D, NW>;
  static constexpr int KEYS = NW * 32;
  static constexpr int QB = BR / 32;
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int PF = 3;                // LDS operand read-ahead, in MFMAs
  // per stage: Q tile | dO tile | nl2[BR] | D[BR]
  static constexpr int STAGE_BYTES = 2 * TL::BYTES + 2 * BR * 4;

  using T = typename E::T;
  using V8 = typename E::V8;
  using H8 = f16x8;
  using H4 = f16x4;

  struct State {
    int lane, wave, hl, l32;
    int b, kw0, key, kv_limit;
    typename TL::Bases lb;      // LDS lane bases
    int64_t head_bytes;         // bytes between the Q (dO) rows of consecutive heads
    int64_t row_bytes;          // bytes per Q row
    int64_t end_bytes;          // bytes from a head's row 0 to the end of row Nq-1
    const char* q0p;            // Q / dO of head 0 of this batch
    const char* d0p;
    uint32_t off[TL::IPW];
    float c;
    int nq1;                    // Nq - 1
    int wq_lo, wq_hi;           // LOCAL: rows that may see one of this wave's keys
    LocalVis lvt;               // LOCAL: the visibility with queries and keys exchanged
    LocalVis::Row lrow;         // LOCAL: this lane's key, as a position of lvt
    float cap_a, cap_c2;        // SOFTCAP constants
    H8 kf[KS], vf[KS];
    f32x16 dk[DT], dv[DT];
  };

  // Q and dO rows q0..q0+BR-1 of head h (rows past Nq load as zero), and the
  // tile's nl2 and D rows (16 bytes = 4 rows per lane: lanes 0..BR/4-1 nl2,
  // the next BR/4 lanes D) into the stage's tail.
  static __device__ __forceinline__ void issue(const BwdArgs& a, const State& st, int h, int q0,
                                               char* stage) {
    if (st.wave == 0) {
      // rows q0 .. q0+BR-1 lie inside the head's ld_rows-long block.  Buffer
      // loads, not global ones: a global load into LDS is a FLAT instruction,
      // which may also touch LDS, and after one the compiler waits for every
      // LDS read (lgkmcnt(0)) where the pipeline needs only the oldest
      const int64_t row0 = ((int64_t)st.b * a.Hq + h) * a.ld_rows + q0;
      const uint32_t voff = (uint32_t)(st.lane % (BR / 4)) * 16;
      if (st.lane < BR / 4)
        dma16_buf(make_rsrc(a.nl2 + row0, BR * 4), voff, stage + 2 * TL::BYTES);
      else if (st.lane < BR / 2)
        dma16_buf(make_rsrc(a.delta + row0, BR * 4), voff, stage + 2 * TL::BYTES);
    }
    const int64_t o = (int64_t)h * st.head_bytes + (int64_t)q0 * st.row_bytes;
    const uint32_t n =
        (uint32_t)min(st.end_bytes - (int64_t)q0 * st.row_bytes, (int64_t)kBufLimit);
    TL::load(make_rsrc(st.q0p + o, n), st.off, stage, st.wave);
    TL::load(make_rsrc(st.d0p + o, n), st.off, stage + TL::BYTES, st.wave);
  }

  // ---- software-pipelined tile ----
  // Blocks of MFMAs, one S/dP set in flight:
  //   SD(0) | exp/dS(0) | SD(1) | GR(0)+exp/dS(1) | SD(2) | GR(1)+exp/dS(2) | ...
  //   | SD(QB-1) | GR(QB-2)+exp/dS(QB-1) | GR(QB-1)
  // SD(i): the 2 KS S/dP MFMAs of 32-row sub-block i; GR(i): its 4 DT dV/dK
  // MFMAs (16 each at d = 128).
  // LDS operands are read PF MFMAs ahead across block boundaries.
  static constexpr int NBLK = 2 * QB + 1;
  static constexpr int SDN = 2 * KS;   // MFMAs of an SD block
  static constexpr int GRN = 4 * DT;   // MFMAs of a GR block
  static __host__ __device__ constexpr int blk_len(int b) {
    return (b % 2 == 0) ? (b / 2 < QB ? SDN : GRN) : (b == 1 ? 0 : GRN);
  }
  static __host__ __device__ constexpr int blk_start(int b) {
    int s = 0;
    for (int q = 0; q < b; ++q) s += blk_len(q);
    return s;
  }
  static constexpr int NSLOT = QB * (SDN + GRN);
  static __host__ __device__ constexpr int slot_blk(int s) {
    int b = 0;
    for (int q = 0; q < NBLK; ++q)
      if (blk_len(q) > 0 && blk_start(q) <= s) b = q;
    return b;
  }
  // kind 0: S/dP MFMA; kind 1: dV/dK MFMA
  static __host__ __device__ constexpr int slot_kind(int s) {
    const int b = slot_blk(s);
    return (b % 2 == 0 && b / 2 < QB) ? 0 : 1;
  }
  static __host__ __device__ constexpr int slot_sub(int s) {
    const int b = slot_blk(s);
    return slot_kind(s) == 0 ? b / 2 : (b % 2 == 1 ? (b - 1) / 2 - 1 : QB - 1);
  }
  static __host__ __device__ constexpr int slot_m(int s) { return s - blk_start(slot_blk(s)); }
  // exp/dS group g of sub-block i: after the MFMA of this slot (i >= 1), or
  // (i = 0) all four before the first MFMA of SD(1)
  static __host__ __device__ constexpr int group_slot(int i, int g) {
    return i == 0 ? blk_start(2) : blk_start(2 * i + 1) + g * (GRN / 4);
  }

  struct Pipe {
    const char* qc;
    const char* dc;
    const char* sc;
    int dlt;                    // key - qt0 - 4 hl (causal mask)
    bool msk;                   // causal: the tile crosses this wave's diagonal
    int qt0;                    // first row of the tile
    uint32_t lw[QB];            // LOCAL: visibility words per sub-block (bit 8 (r/4) + r%4)
    const float* mcol;          // additive mask column of this lane's key, tile's head (MASK)
    int64_t msq;                // mask row stride
    float mv[QB][16];           // additive mask values per sub-block (MASK)
    f32x16 s, dp;
    H8 pp[2][2], dsp[2][2];
    H8 opd[NSLOT];
  };
  template <int SL>
  static __device__ __forceinline__ void pipe_load(const State& st, Pipe& c) {
    constexpr int i = slot_sub(SL), m = slot_m(SL);
    if constexpr (slot_kind(SL) == 0) {
      c.opd[SL] = TL::template row<H8>((m & 1) ? c.dc : c.qc, st.lb, i * 32, m >> 1);
    } else {
      c.opd[SL] = TL::template tr<H8, H4>((m & 1) ? c.qc : c.dc, st.lb, i * 32 + (m / (2 * DT)) * 16,
                                          (m >> 1) % DT);
    }
  }
  // Additive mask values of sub-block I for this lane's key: register r holds
  // row qt0 + 32 I + 8 (r / 4) + 4 hl + r % 4 (clamped to the last row; rows
  // past Nq have P = 0 through nl2).
  template <int I>
  static __device__ __forceinline__ void pipe_mask(const State& st, Pipe& c) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      c.mv[I][r] = c.mcol[min(c.qt0 + I * 32 + (r >> 2) * 8 + st.hl * 4 + (r & 3), st.nq1) * c.msq];
  }
  template <int I, int GQ>
  static __device__ __forceinline__ void pipe_group(const State& st, Pipe& c) {
    constexpr int par = I & 1;
    const int lr = I * 32 + GQ * 8 + st.hl * 4;
    const f32x4 nl = *(const LDS_AS f32x4*)(const LDS_AS void*)(c.sc + lr * 4);
    const f32x4 dd = *(const LDS_AS f32x4*)(const LDS_AS void*)(c.sc + BR * 4 + lr * 4);
    float pv[4], dsv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // P = exp2(s c + mask log2(e) - LSE log2(e))
      const float ml = MASK ? __builtin_fmaf(c.mv[I][GQ * 4 + e], kLog2e, nl[e]) : nl[e];
      if constexpr (SOFTCAP) {
        float g;
        const float t = softcap_grad(c.s[GQ * 4 + e], st.cap_a, st.cap_c2, g);
        const float p = fast_exp2(t + ml);
        pv[e] = p;
        dsv[e] = p * g * (c.dp[GQ * 4 + e] - dd[e]);
      } else {
        const float p = fast_exp2(__builtin_fmaf(c.s[GQ * 4 + e], st.c, ml));
        pv[e] = p;
        dsv[e] = p * (c.dp[GQ * 4 + e] - dd[e]);
      }
    }
    constexpr int t2 = GQ >> 1, half = (GQ & 1) * 4;
    const f16x2 p01 = FP16::cvt2(pv[0], pv[1]), p23 = FP16::cvt2(pv[2], pv[3]);
    const f16x2 s01 = FP16::cvt2(dsv[0], dsv[1]), s23 = FP16::cvt2(dsv[2], dsv[3]);
    c.pp[par][t2][half + 0] = p01[0];
    c.pp[par][t2][half + 1] = p01[1];
    c.pp[par][t2][half + 2] = p23[0];
    c.pp[par][t2][half + 3] = p23[1];
    c.dsp[par][t2][half + 0] = s01[0];
    c.dsp[par][t2][half + 1] = s01[1];
    c.dsp[par][t2][half + 2] = s23[0];
    c.dsp[par][t2][half + 3] = s23[1];
  }
  template <int SL, int VI>
  static __device__ __forceinline__ void pipe_groups_of(const State& st, Pipe& c) {
    if constexpr (group_slot(VI, 0) == SL) pipe_group<VI, 0>(st, c);
    if constexpr (group_slot(VI, 1) == SL) pipe_group<VI, 1>(st, c);
    if constexpr (group_slot(VI, 2) == SL) pipe_group<VI, 2>(st, c);
    if constexpr (group_slot(VI, 3) == SL) pipe_group<VI, 3>(st, c);
  }
  template <int PF, int SL>
  static __device__ __forceinline__ void pipe_slot(State& st, Pipe& c) {
    if constexpr (SL + PF < NSLOT) pipe_load<SL + PF>(st, c);
    constexpr int i = slot_sub(SL), m = slot_m(SL), par = i & 1;
    if constexpr (SL == blk_start(2)) {
      pipe_groups_of<SL, 0>(st, c);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MASK && slot_kind(SL) == 0 && m == 0) pipe_mask<i>(st, c);
    if constexpr (slot_kind(SL) == 0) {
      if constexpr (m == 0) {
        // Causal, on a tile that crosses the diagonal: S starts at -inf
        // where the key lies after the row (key <= row  <=>
        // key - qt0 - 4 hl <= 32 i + 8 (r / 4) + r % 4 for register r), so
        // that P = 0 and dS = 0 there; 0 elsewhere.  Other tiles start from
        // the MFMA's zero operand.
        // LOCAL: the same from the visibility word of sub-block i.
        if ((CAUSAL || LOCAL) && c.msk) {
          f32x16 init;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if constexpr (LOCAL)
              init[r] = keep_if_bit(0.f, c.lw[i], (r >> 2) * 8 + (r & 3));
            else
              init[r] = (c.dlt <= i * 32 + (r >> 2) * 8 + (r & 3)) ? 0.f : -INFINITY;
          }
          c.s = FP16::mfma(c.opd[SL], st.kf[0], init);
        } else {
          c.s = FP16::mfma(c.opd[SL], st.kf[0], f32x16{});
        }
      } else if constexpr (m == 1) {
        c.dp = FP16::mfma(c.opd[SL], st.vf[0], f32x16{});
      } else if constexpr (m & 1) {
        c.dp = FP16::mfma(c.opd[SL], st.vf[m >> 1], c.dp);
      } else {
        c.s = FP16::mfma(c.opd[SL], st.kf[m >> 1], c.s);
      }
    } else {
      constexpr int t2 = m / (2 * DT), dt = (m >> 1) % DT;
      if constexpr (m & 1) st.dk[dt] = FP16::mfma(c.dsp[par][t2], c.opd[SL], st.dk[dt]);
      else st.dv[dt] = FP16::mfma(c.pp[par][t2], c.opd[SL], st.dv[dt]);
    }
    if constexpr (slot_kind(SL) == 1 && slot_blk(SL) % 2 == 1)
      pipe_groups_of<SL, (slot_blk(SL) - 1) / 2>(st, c);
    __builtin_amdgcn_sched_barrier(0);
  }
  template <int PF, int... SL>
  static __device__ __forceinline__ void pipe_slots(State& st, Pipe& c,
                                                    std::integer_sequence<int, SL...>) {
    (pipe_slot<PF, SL>(st, c), ...);
  }
  template <int... SL>
  static __device__ __forceinline__ void pipe_prologue(State& st, Pipe& c,
                                                       std::integer_sequence<int, SL...>) {
    (pipe_load<SL>(st, c), ...);
  }
  // b0, b1 (LOCAL): rows qt0..qt0+63 and qt0+64..qt0+127 that see this
  // lane's key
  template <int PF>
  static __device__ __forceinline__ void pipe_tile(const BwdArgs& a, State& st, const char* stage,
                                                   int h, int qt0, uint64_t b0, uint64_t b1) {
    Pipe c;
    c.qc = stage;
    c.dc = stage + TL::BYTES;
    c.sc = stage + 2 * TL::BYTES;
    c.dlt = st.key - qt0 - 4 * st.hl;
    if constexpr (LOCAL) {
#pragma unroll
      for (int i = 0; i < QB; ++i)
        c.lw[i] = (uint32_t)(((i < 2) ? b0 : b1) >> ((i & 1) * 32 + 4 * st.hl));
      c.msk = __builtin_amdgcn_ballot_w64((b0 & b1) != ~0ull) != 0;
    } else {
      c.msk = qt0 < st.kw0 + 31;
    }
    c.qt0 = qt0;
    if (MASK) {
      c.mcol = a.mask + st.b * a.m_sb + h * a.m_sh + min(st.key, a.Nk - 1);
      c.msq = a.m_sq;
    }
    pipe_prologue(st, c, std::make_integer_sequence<int, PF>{});
    pipe_slots<PF>(st, c, std::make_integer_sequence<int, NSLOT>{});
  }

  // Iteration t over (head, q-tile) pairs: tile t (head hc, rows qt0..) is
  // in `cur`, tile t+1 (head hn, rows qn..) goes into `nxt`.
  static __device__ __forceinline__ void step(const BwdArgs& a, State& st, int t, int n_t, int hc,
                                              int qt0, int hn, int qn, char* cur, char* nxt,
                                              bool live) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < n_t) issue(a, st, hn, qn, nxt);
    if (!live) return;                                   // this wave's keys are all masked
    if (CAUSAL && qt0 + BR - 1 < st.kw0) return;         // no row of the tile sees them
    // Keys at or past kv_limit are not masked here: a key's P and dS only
    // reach its own rows of dK / dV, which are stored as zero.
    if constexpr (LOCAL) {
      if (qt0 + BR - 1 < st.wq_lo || qt0 > st.wq_hi) return;
      const uint64_t b0 = st.lvt.bits(st.lrow, qt0, a.Nq);
      const uint64_t b1 = st.lvt.bits(st.lrow, qt0 + 64, a.Nq);
      if (!__builtin_amdgcn_ballot_w64((b0 | b1) != 0)) return;   // no row sees these keys
      pipe_tile<PF>(a, st, cur, hc, qt0, b0, b1);
    } else {
      pipe_tile<PF>(a, st, cur, hc, qt0, 0, 0);
    }
  }

  static __device__ void run(const BwdArgs& a, char* s0, char* s1) {
    State st;
    st.lane = threadIdx.x & 63;
    st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    st.hl = st.lane >> 5;
    st.l32 = st.lane & 31;

    // block -> (key block, chunk, kv-head, batch); key blocks in increasing
    // order over the whole grid, i.e. (causal) the ones with the most query
    // rows first, and every XCD (each 8th work-group) holds blocks of every
    // batch, whose key lengths may differ
    const int n_combo = a.B * a.Hkv * a.kv_chunks;
    const int kblk = blockIdx.x / n_combo;
    int rest = blockIdx.x % n_combo;
    const int chunk = rest % a.kv_chunks;
    rest /= a.kv_chunks;
    const int g = rest % a.Hkv;
    const int b = rest / a.Hkv;
    st.b = b;
    const int key0 = kblk * KEYS;
    st.kw0 = key0 + st.wave * 32;
    st.key = st.kw0 + st.l32;

    st.kv_limit = a.Nk;
    if (a.kv_lens) st.kv_limit = min(max(a.kv_lens[b], 0), a.Nk);

    // K^T and V^T fragments of this lane's key, fp16 (zero beyond d)
    const BwdScales sc = bwd_scales(a);
    {
      const int krow = min(st.key, a.Nk - 1);
      const T* kp = (const T*)a.k + b * a.k_sb + g * a.k_sh + krow * a.k_sn;
      const T* vp = (const T*)a.v + b * a.k_sb + g * a.k_sh + krow * a.k_sn;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + st.hl * 8;
        st.kf[ks] = d0 < a.d ? to_f16x8_scaled<E>(*(const V8*)(kp + d0), sc.k) : H8{};
        st.vf[ks] = d0 < a.d ? to_f16x8_scaled<E>(*(const V8*)(vp + d0), sc.v) : H8{};
      }
      pin_agpr(st.kf);
      pin_agpr(st.vf);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      st.dk[dt] = f32x16{};
      st.dv[dt] = f32x16{};
    }
    st.c = a.c / (sc.q * sc.k);
    st.cap_a = a.cap_a;
    st.cap_c2 = a.cap_c2 / (sc.q * sc.k);
    const float dk_scale = a.scale / (sc.dout * sc.v * sc.q), dv_scale = 1.f / sc.dout;
    st.nq1 = a.Nq - 1;
    st.q0p = (const char*)((const _Float16*)a.q16 + b * a.q_sb);
    st.d0p = (const char*)((const _Float16*)a.do16 + b * a.q_sb);
    st.head_bytes = a.q_sh * 2;
    st.row_bytes = a.q_sn * 2;
    st.end_bytes = ((int64_t)(a.Nq - 1) * a.q_sn + a.d) * 2;
    const int dchunks = a.d / 8;
#pragma unroll
    for (int i = 0; i < TL::IPW; ++i)
      st.off[i] = TL::offset(i * NW + st.wave, st.lane, dchunks, a.q_sn);
    st.lb = TL::bases(st.lane);

    // query rows that can see some key of this block
    int q_start = CAUSAL ? (key0 / BR) * BR : 0;
    int n_qt = (key0 < st.kv_limit && q_start < a.Nq) ? (a.Nq - q_start + BR - 1) / BR : 0;
    if constexpr (LOCAL) {
      st.lvt = a.loc.transposed();
      int lo, hi;
      st.lvt.key_range(key0, min(key0 + KEYS, st.kv_limit) - 1, a.Nq, lo, hi);
      q_start = (lo / BR) * BR;
      n_qt = (key0 < st.kv_limit && hi >= lo) ? hi / BR + 1 - lo / BR : 0;
      st.wq_lo = 1;
      st.wq_hi = 0;
      if (st.kw0 < st.kv_limit)
        st.lvt.key_range(st.kw0, min(st.kw0 + 31, st.kv_limit - 1), a.Nq, st.wq_lo, st.wq_hi);
      st.lrow = st.lvt.row(min(st.key, a.Nk - 1));
    }
    const int q_stop = q_start + n_qt * BR;   // rows past the block's reach wrap to the next head
    const int HS = a.group / a.kv_chunks;
    const int h0 = g * a.group + chunk * HS;
    const int n_t = n_qt * HS;   // (head, q-tile) pairs, head-major
    const bool live = st.kw0 < st.kv_limit;

    // tiles walk the (head, q-tile) pairs head-major; tile t is in stage t % 2
    if (n_t > 0) issue(a, st, h0, q_start, s0);
    int hc = h0, q0 = q_start;     // head and rows of tile t
    int hn = h0, qn = q_start;     // head and rows of tile t + 1
    for (int t = 0; t < n_t; t += 2) {
      qn += BR;
      if (qn >= q_stop) {
        qn = q_start;
        ++hn;
      }
      step(a, st, t, n_t, hc, q0, hn, qn, s0, s1, live);
      hc = hn;
      q0 = qn;
      if (t + 1 >= n_t) break;
      qn += BR;
      if (qn >= q_stop) {
        qn = q_start;
        ++hn;
      }
      step(a, st, t + 1, n_t, hc, q0, hn, qn, s1, s0, live);
      hc = hn;
      q0 = qn;
    }

    // Store: lane holds d column dt*32 + l32, keys kw0 + (r/4)*8 + 4 hl + r%4.
    if (st.kw0 >= a.Nk) return;
    const bool direct = a.kv_chunks == 1;
    const int64_t part = (int64_t)a.B * a.Hkv * a.Nk * a.d;  // one partial tensor
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int col = dt * 32 + st.l32;
      if (col >= a.d) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = st.kw0 + (r >> 2) * 8 + st.hl * 4 + (r & 3);
        if (kr >= a.Nk) continue;
        const int64_t off = b * a.k_sb + g * a.k_sh + kr * a.k_sn + col;
        const bool kv_ok = kr < st.kv_limit;
        const float kval = kv_ok ? st.dk[dt][r] * dk_scale : 0.f;
        const float vval = kv_ok ? st.dv[dt][r] * dv_scale : 0.f;
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

template <class E, int D, int NW, int BR, bool CAUSAL, bool MASK, bool LOCAL = false,
          bool SOFTCAP = false>
__global__ __launch_bounds__(NW * 64) void bwd_kv_kernel(BwdArgs a) {
  using K = BwdKV<E, D, NW, BR, CAUSAL, MASK, LOCAL, SOFTCAP>;
  __shared__ __attribute__((aligned(1024))) char s0[K::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s1[K::STAGE_BYTES];
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
