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
// nl2 = -LSE * log2(e) (-inf for a fully masked row and for the padding rows
// past Nq, so that P = 0 there without further masking).
//
// Tiles stream through LDS with a padded row pitch of D/8 + 1 16-byte slots,
// filled by direct buffer->LDS loads (rows or columns past the tensor read as
// zero).  Row-fragment reads (16 rows x one 16-byte chunk per 16 lanes) are
// conflict-free; transposed reads (4 rows x 64 bytes per half-wave) share
// banks pairwise.  Every read address is a per-lane base plus a compile-time
// offset.  Causal and key-length masking is applied only to tiles that
// cross a boundary.
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
  // In-place bf16 -> fp16 conversion of the slots this lane loaded (after its
  // own loads have landed; identity for fp16 inputs).
  template <class E>
  static __device__ __forceinline__ void to_f16(char* buf, int wave, int lane) {
    if constexpr (!std::is_same<E, FP16>::value) {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int ins = i * NW + wave;
        if (ins < INS) {
          char* p = buf + ins * 1024 + lane * 16;
          *(LDS_AS f16x8*)(LDS_AS void*)(p) = to_f16x8<E>(lds_read16<typename E::V8>(p));
        }
      }
    }
  }
  // Lane bases: row fragment (row l32, chunk hl) and transposed read (row
  // 4 (group / 2) + i / 4, column 16 (group % 2) + 4 (i % 4) for lane i of
  // 16-lane group `group`).
  static __device__ __forceinline__ int row_base(int l32, int hl) { return l32 * P + hl * 16; }
  static __device__ __forceinline__ int tr_base(int lane) {
    const int grp = lane >> 4, gi = lane & 15;
    return (4 * (grp >> 1) + (gi >> 2)) * P + (16 * (grp & 1) + 4 * (gi & 3)) * 2;
  }
  // MFMA operand from rows r0 + (lane % 32), k-step ks (d = 16 ks + 8 hl ..).
  template <class V8>
  static __device__ __forceinline__ V8 row(const char* buf, int rb, int r0, int ks) {
    return lds_read16<V8>(buf + rb + r0 * P + ks * 32);
  }
  // MFMA operand read transposed: column dt*32 + lane%32, rows r0 + slot
  // order 8 (s / 4) + 4 hl + s % 4 for slot s.
  template <class V8, class V4>
  static __device__ __forceinline__ V8 tr(const char* buf, int tb, int r0, int dt) {
    const char* p = buf + tb + r0 * P + dt * 64;
    const V4 lo = lds_read_tr4<V4>(p);
    const V4 hi = lds_read_tr4<V4>(p + 8 * P);
    return concat4<V8, V4>(lo, hi);
  }
};

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
  using TL = PadTile<BC, D, NW>;
  static constexpr int ROWS = NW * 32;
  static constexpr int KB = BC / 32;
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int PT = BC / 16;

  using T = typename E::T;
  using V8 = typename E::V8;
  using H8 = f16x8;
  using H4 = f16x4;

  struct State {
    int lane, wave, hl, l32;
    int q_w0, qrow, kv_limit;
    int rb, tb;                 // LDS lane bases
    const char* kp;             // K / V of this (batch, kv-head), key 0
    const char* vp;
    int64_t tile_bytes, end_bytes;
    uint32_t off[TL::IPW];
    float c, nl2;
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

  template <bool EDGE>
  static __device__ __forceinline__ void tile(State& st, const char* kc, const char* vc, int j0) {
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
        s[k] = FP16::mfma(TL::template row<H8>(kc, st.rb, k * 32, ks), st.qf[ks], s[k]);
        dp[k] = E::mfma(TL::template row<V8>(vc, st.rb, k * 32, ks), st.df[ks], dp[k]);
      }
    H8 pf[PT], xf[PT];
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      const int k = t >> 1, r0 = (t & 1) * 8;
      float pv[8], xv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = r0 + e;
        float p = fast_exp2(__builtin_fmaf(s[k][r], st.c, st.nl2));
        if constexpr (EDGE) {
          const int key = j0 + k * 32 + (r >> 2) * 8 + st.hl * 4 + (r & 3);
          const bool vis = key < st.kv_limit && (!CAUSAL || key <= st.qrow);
          p = vis ? p : 0.f;
        }
        pv[e] = p;
        xv[e] = p * dp[k][r];
        st.dsum[e & 3] += xv[e];
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
#pragma unroll
    for (int t = 0; t < PT; ++t)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const H8 kt = TL::template tr<H8, H4>(kc, st.tb, t * 16, dt);
        st.acc_a[dt] = FP16::mfma(kt, xf[t], st.acc_a[dt]);
        st.acc_b[dt] = FP16::mfma(kt, pf[t], st.acc_b[dt]);
      }
  }

  // Iteration j: tile j is in (kc, vc); tile j+1 goes into (kn, vn).
  static __device__ __forceinline__ void step(State& st, int j, int n, int n_act, char* kc,
                                              const char* vc, char* kn, char* vn) {
    __builtin_amdgcn_s_waitcnt(0);
    TL::template to_f16<E>(kc, st.wave, st.lane);
    __syncthreads();
    if (j + 1 < n) issue(st, j + 1, kn, vn);
    if (j >= n_act) return;
    const int j0 = j * BC;
    const bool edge = (j0 + BC > st.kv_limit) || (CAUSAL && j0 + BC - 1 > st.q_w0);
    if (edge) tile<true>(st, kc, vc, j0);
    else tile<false>(st, kc, vc, j0);
  }

  static __device__ void run(const BwdArgs& a, char* k0, char* v0, char* k1, char* v1) {
    State st;
    st.lane = threadIdx.x & 63;
    st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    st.hl = st.lane >> 5;
    st.l32 = st.lane & 31;

    const int nqb = (a.Nq + ROWS - 1) / ROWS;
    const int wid = xcd_remap(blockIdx.x, gridDim.x);
    int qblk = wid % nqb;
    const int bh = wid / nqb;
    const int h = bh % a.Hq, b = bh / a.Hq;
    if (CAUSAL) qblk = nqb - 1 - qblk;
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
    {
      const T* qp = (const T*)a.q + b * a.q_sb + h * a.q_sh + crow * a.q_sn;
      const T* dp = (const T*)a.dout + b * a.q_sb + h * a.q_sh + crow * a.q_sn;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + st.hl * 8;
        st.qf[ks] = d0 < a.d ? to_f16x8<E>(*(const V8*)(qp + d0)) : H8{};
        st.df[ks] = d0 < a.d ? *(const V8*)(dp + d0) : V8{};
      }
    }
    const float lse = a.lse[((int64_t)b * a.Hq + h) * a.Nq + crow];
    st.nl2 = (st.qrow < a.Nq && lse != -INFINITY) ? -lse * kLog2e : -INFINITY;
    st.c = a.c;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      st.acc_a[dt] = f32x16{};
      st.acc_b[dt] = f32x16{};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) st.dsum[i] = 0.f;

    st.kp = (const char*)((const T*)a.k + b * a.k_sb + g * a.k_sh);
    st.vp = (const char*)((const T*)a.v + b * a.k_sb + g * a.k_sh);
    st.tile_bytes = (int64_t)BC * a.k_sn * 2;
    st.end_bytes = ((int64_t)(a.Nk - 1) * a.k_sn + a.d) * 2;
    const int dchunks = a.d / 8;
#pragma unroll
    for (int i = 0; i < TL::IPW; ++i)
      st.off[i] = TL::offset(i * NW + st.wave, st.lane, dchunks, a.k_sn);
    st.rb = TL::row_base(st.l32, st.hl);
    st.tb = TL::tr_base(st.lane);

    if (n_tiles > 0) issue(st, 0, k0, v0);
    for (int j = 0; j < n_tiles; j += 2) {
      step(st, j, n_tiles, n_act, k0, v0, k1, v1);
      if (j + 1 >= n_tiles) break;
      step(st, j + 1, n_tiles, n_act, k1, v1, k0, v0);
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
          x[e] = a.scale * (st.acc_a[dt][gq * 4 + e] - dtot * st.acc_b[dt][gq * 4 + e]);
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
  __shared__ __attribute__((aligned(1024))) char k0[K::TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[K::TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[K::TL::BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[K::TL::BYTES];
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
  using TL = PadTile<BR, D, NW>;
  static constexpr int KEYS = NW * 32;
  static constexpr int QB = BR / 32;
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  // per stage: Q tile | dO tile | nl2[BR] | D[BR]
  static constexpr int STAGE_BYTES = 2 * TL::BYTES + 2 * BR * 4;

  using T = typename E::T;
  using V8 = typename E::V8;
  using H8 = f16x8;
  using H4 = f16x4;

  struct State {
    int lane, wave, hl, l32;
    int b, kw0, key, kv_limit;
    int rb, tb;
    int64_t head_bytes;         // bytes between the Q (dO) rows of consecutive heads
    int64_t row_bytes;          // bytes per Q row
    int64_t end_bytes;          // bytes from a head's row 0 to the end of row Nq-1
    const char* q0p;            // Q / dO of head 0 of this batch
    const char* d0p;
    uint32_t off[TL::IPW];
    float c;
    H8 kf[KS], vf[KS];
    f32x16 dk[DT], dv[DT];
  };

  // Q and dO rows q0..q0+BR-1 of head h (rows past Nq load as zero), and the
  // tile's nl2 and D rows (16 bytes = 4 rows per lane: lanes 0..BR/4-1 nl2,
  // the next BR/4 lanes D) into the stage's tail.
  static __device__ __forceinline__ void issue(const BwdArgs& a, const State& st, int h, int q0,
                                               char* stage) {
    if (st.wave == 0 && st.lane < BR / 2) {
      // rows q0 .. q0+BR-1 lie inside the head's ld_rows-long block
      const float* src = (st.lane < BR / 4 ? a.nl2 : a.delta) +
                         ((int64_t)st.b * a.Hq + h) * a.ld_rows + q0 + (st.lane % (BR / 4)) * 4;
      dma16(src, stage + 2 * TL::BYTES);
    }
    const int64_t o = (int64_t)h * st.head_bytes + (int64_t)q0 * st.row_bytes;
    const uint32_t n =
        (uint32_t)min(st.end_bytes - (int64_t)q0 * st.row_bytes, (int64_t)kBufLimit);
    TL::load(make_rsrc(st.q0p + o, n), st.off, stage, st.wave);
    TL::load(make_rsrc(st.d0p + o, n), st.off, stage + TL::BYTES, st.wave);
  }

  template <bool EDGE>
  static __device__ __forceinline__ void tile(State& st, const char* stage, int qt0) {
    const char* qc = stage;
    const char* dc = stage + TL::BYTES;
    const char* sc = stage + 2 * TL::BYTES;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = FP16::mfma(TL::template row<H8>(qc, st.rb, qb * 32, ks), st.kf[ks], s);
        dp = FP16::mfma(TL::template row<H8>(dc, st.rb, qb * 32, ks), st.vf[ks], dp);
      }
      // rows of register r: qt0 + qb*32 + (r/4)*8 + 4 hl + r%4
      H8 pp[2], dsp[2];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int lr = qb * 32 + gq * 8 + st.hl * 4;   // local row of e = 0
        const f32x4 nl = *(const LDS_AS f32x4*)(const LDS_AS void*)(sc + lr * 4);
        const f32x4 dd = *(const LDS_AS f32x4*)(const LDS_AS void*)(sc + BR * 4 + lr * 4);
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = gq * 4 + e;
          float p = fast_exp2(__builtin_fmaf(s[r], st.c, nl[e]));
          if constexpr (EDGE) {
            const int qr = qt0 + lr + e;
            const bool vis = st.key < st.kv_limit && (!CAUSAL || st.key <= qr);
            p = vis ? p : 0.f;
          }
          pv[e] = p;
          dsv[e] = p * (dp[r] - dd[e]);
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
          const int r0 = qb * 32 + t2 * 16;
          st.dv[dt] = FP16::mfma(pp[t2], TL::template tr<H8, H4>(dc, st.tb, r0, dt), st.dv[dt]);
          st.dk[dt] = FP16::mfma(dsp[t2], TL::template tr<H8, H4>(qc, st.tb, r0, dt), st.dk[dt]);
        }
    }
  }

  // Iteration t over (head, q-tile) pairs: tile t (rows qt0..) is in `cur`,
  // tile t+1 (head hn, rows qn..) goes into `nxt`.
  static __device__ __forceinline__ void step(const BwdArgs& a, State& st, int t, int n_t, int qt0,
                                              int hn, int qn, char* cur, char* nxt, bool live) {
    __builtin_amdgcn_s_waitcnt(0);
    TL::template to_f16<E>(cur, st.wave, st.lane);
    TL::template to_f16<E>(cur + TL::BYTES, st.wave, st.lane);
    __syncthreads();
    if (t + 1 < n_t) issue(a, st, hn, qn, nxt);
    if (!live) return;                                   // this wave's keys are all masked
    if (CAUSAL && qt0 + BR - 1 < st.kw0) return;         // no row of the tile sees them
    const bool edge = (CAUSAL && qt0 < st.kw0 + 31) || (st.kw0 + 32 > st.kv_limit);
    if (edge) tile<true>(st, cur, qt0);
    else tile<false>(st, cur, qt0);
  }

  static __device__ void run(const BwdArgs& a, char* s0, char* s1) {
    State st;
    st.lane = threadIdx.x & 63;
    st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    st.hl = st.lane >> 5;
    st.l32 = st.lane & 31;

    // block -> (key block, chunk, kv-head, batch); key blocks in increasing
    // order, i.e. (causal) the ones with the most query rows first
    int kblk, rest;
    rank_combo(blockIdx.x, a.B * a.Hkv * a.kv_chunks, kblk, rest);
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
    {
      const int krow = min(st.key, a.Nk - 1);
      const T* kp = (const T*)a.k + b * a.k_sb + g * a.k_sh + krow * a.k_sn;
      const T* vp = (const T*)a.v + b * a.k_sb + g * a.k_sh + krow * a.k_sn;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + st.hl * 8;
        st.kf[ks] = d0 < a.d ? to_f16x8<E>(*(const V8*)(kp + d0)) : H8{};
        st.vf[ks] = d0 < a.d ? to_f16x8<E>(*(const V8*)(vp + d0)) : H8{};
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      st.dk[dt] = f32x16{};
      st.dv[dt] = f32x16{};
    }
    st.c = a.c;
    st.q0p = (const char*)((const T*)a.q + b * a.q_sb);
    st.d0p = (const char*)((const T*)a.dout + b * a.q_sb);
    st.head_bytes = a.q_sh * 2;
    st.row_bytes = a.q_sn * 2;
    st.end_bytes = ((int64_t)(a.Nq - 1) * a.q_sn + a.d) * 2;
    const int dchunks = a.d / 8;
#pragma unroll
    for (int i = 0; i < TL::IPW; ++i)
      st.off[i] = TL::offset(i * NW + st.wave, st.lane, dchunks, a.q_sn);
    st.rb = TL::row_base(st.l32, st.hl);
    st.tb = TL::tr_base(st.lane);

    // query rows that can see some key of this block
    const int q_start = CAUSAL ? (key0 / BR) * BR : 0;
    const int n_qt = (key0 < st.kv_limit && q_start < a.Nq) ? (a.Nq - q_start + BR - 1) / BR : 0;
    const int HS = a.group / a.kv_chunks;
    const int h0 = g * a.group + chunk * HS;
    const int n_t = n_qt * HS;   // (head, q-tile) pairs, head-major
    const bool live = st.kw0 < st.kv_limit;

    // tiles walk the (head, q-tile) pairs head-major; tile t is in stage t % 2
    if (n_t > 0) issue(a, st, h0, q_start, s0);
    int q0 = q_start;              // rows of tile t
    int hn = h0, qn = q_start;     // head and rows of tile t + 1
    for (int t = 0; t < n_t; t += 2) {
      qn += BR;
      if (qn >= a.Nq) {
        qn = q_start;
        ++hn;
      }
      step(a, st, t, n_t, q0, hn, qn, s0, s1, live);
      q0 = qn;
      if (t + 1 >= n_t) break;
      qn += BR;
      if (qn >= a.Nq) {
        qn = q_start;
        ++hn;
      }
      step(a, st, t + 1, n_t, q0, hn, qn, s1, s0, live);
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
        const float kval = st.dk[dt][r] * a.scale, vval = st.dv[dt][r];
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
