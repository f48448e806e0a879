// Software-pipelined forward attention kernel for gfx950 (16-bit inputs,
// optional causal mask, no additive mask).
//
// Same arithmetic as FwdKernel in attn_fwd_kernel.h -- the tiled online
// softmax of "FlashAttention技术解析：优化Transformer注意力计算效率"
// (jsqmd.com/news/722897) §2.2 with the single final normalisation of its
// §4.1 -- and bit-identical results; only the order of issue differs.
//
// Each wave owns 32 query rows; the NW waves of a work-group (8, two per
// SIMD; or 4, with two work-groups per CU) share K/V tiles of BC keys that
// stream through LDS, filled by direct buffer->LDS loads.  K runs
// one tile ahead of V: iteration j computes S of tile j+1 while it finishes
// tile j, so the matrix cores have independent work while the vector unit
// evaluates the exponentials:
//
//   phase 1 (NQ steps):  one QK^T MFMA of tile j+1 per step, interleaved with
//                        part of tile j's exponentials (p = exp2(s*c - m),
//                        row sum, conversion to the 16-bit P operand), and
//                        at every other step (every step with 4 waves) one
//                        of this wave's loads of V(j+1) / K(j+2) into the
//                        buffers iteration j-1 used;
//   phase 2 (NP steps):  one PV MFMA of tile j per step; the first half of
//                        the steps finish the exponentials (each 16-key
//                        chunk before its first PV), the second half reduce
//                        tile j+1's row maximum.
//
// A single wave hides only a handful of vector instructions under each MFMA,
// so the vector work is spread evenly over both phases.  sched_barrier fences
// keep the compiler from regrouping the steps, and empty asm statements pin
// the running sum and maximum to their step (otherwise they are sunk to the
// end of the block as one serial chain).  LDS fragments are read two steps
// ahead of their MFMA.
//
// Tiles that reach past the key range (kv_lens, ragged Nk) or, under the
// causal mask, past some row's own position (key i visible to query rows
// >= i) are masked after the main block and their maximum recomputed; the
// lazy rescale (reference point moved only when a tile's maximum exceeds it
// by more than TH) follows.  Causal work-groups stop at the tile holding
// their last row's key; the waves with earlier rows run the remaining tiles
// fully masked (exponentials of -inf are 0), which keeps every wave in the
// shared loads and barriers.
#pragma once

#include "attn_kernels.h"
#include "device_common.h"

namespace attn {

// DK: the width of the QK^T contraction, D or (D = 64, d <= 48) 48: the
// k-step over columns 48..63 then multiplies only the zeros past d and is
// skipped (a quarter of the QK^T products and K reads of a d = 40 call).
template <class E, int D, int BC, bool CAUSAL, int NW = 8, int DK = D>
struct FwdPipeKernel {
  static_assert(DK == D || (D == 64 && DK == 48), "QK^T width");
  static constexpr float TH = 8.0f;                 // rescale threshold, log2 units
  // NW waves per work-group: 8 (one work-group per CU), or 4 for short key
  // ranges, where two independent work-groups per CU overlap one's start
  // (Q and first K tile loads) with the other's tiles
  static constexpr int ROWS = NW * 32;              // query rows per work-group
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  // LDS rows of CPR 16-byte slots, unpadded (a pad slot would be a load lane
  // that moves nothing); chunk c of row r sits at slot c ^ f(r), which puts
  // the 16 rows one K read touches at a time (same chunk) on 16 different
  // bank groups, and likewise the 4 rows x 4 chunks of a half-wave's
  // transposed V read: at d = 128 (256-byte rows) f_K(r) = r mod 16 and
  // f_V(r) = 4 (r mod 4); at d = 64 (two rows per 256 bytes)
  // f_K(r) = (r / 2) mod 8 and f_V(r) = 4 ((r / 2) mod 2).  The loads pick
  // their source chunk accordingly; the read bases fold the XOR in.
  static constexpr int KPS = CPR;
  static constexpr int VPS = CPR;
  static __host__ __device__ constexpr int fk(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  static __host__ __device__ constexpr int fv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
  static constexpr int KP = KPS * 16, VP = VPS * 16;
  static constexpr int K_BYTES = BC * KP, V_BYTES = BC * VP;
  static constexpr int K_INS = (BC * KPS + 63) / 64;   // load instructions per K tile
  static constexpr int V_INS = (BC * VPS + 63) / 64;
  static constexpr int K_IPW = (K_INS + NW - 1) / NW;  // ... per wave
  static constexpr int V_IPW = (V_INS + NW - 1) / NW;
  static constexpr int KB = BC / 32;                   // 32-key blocks per tile
  static constexpr int KS = DK / 16;                   // k-steps of QK^T
  static constexpr int DT = D / 32;                    // 32-wide d tiles of O
  static constexpr int PT = BC / 16;                   // 16-key chunks (PV k-steps)
  static constexpr int NQ = KS * KB;                   // QK^T MFMAs per tile
  static constexpr int NP = PT * DT;                   // PV MFMAs per tile
  static constexpr int NPAIR = PT * 4;                 // pairs of exponentials per tile
  static constexpr int P1 = (NPAIR * 5) / 8;           // pairs done in phase 1
  static constexpr int NE = NP / 2;                    // phase-2 steps that do exponentials
  static constexpr int PF = 2;                         // LDS read-ahead, in steps
  static_assert((NPAIR - P1) <= NE * 2, "phase 2 must finish the exponentials");

  using T = typename E::T;
  using V8 = typename E::V8;
  using V4 = typename E::V4;
  using V2 = typename E::V2;
  using Scores = f32x16[KB];

  struct State {
    int lane, wave, hl, l32;
    int q_w0;                   // first query row of this wave
    int kv_limit;               // keys >= kv_limit are excluded
    int n_act;                  // tiles with keys for this work-group
    const char* kp;             // K / V of this (batch, kv-head), key 0
    const char* vp;
    int64_t k_tile, v_tile;     // bytes between consecutive tiles
    int64_t k_end, v_end;       // bytes from kp / vp to the end of key kv_limit-1
    uint32_t koff[K_IPW], voff[V_IPW];  // per load instruction: byte offset in a tile
    int kofs[KS], vofs[DT];     // per-lane LDS byte offsets: K per k-step, V per d-tile
    float c;                    // scale * log2(e)
    V8 qf[KS];                  // Q fragments (B operand of S^T = K Q^T)
    f32x16 acc[DT];             // O^T accumulators
    float m_run, l_run;
  };

  // Byte offset, within a tile of row pitch sn elements, of the 16-byte
  // chunk lane `lane` copies in load instruction `ins` of a tile with `ps`
  // LDS slots per row; pad slots and columns past d get an out-of-range
  // offset (the load returns zero).
  static __device__ __forceinline__ uint32_t dma_offset(int ins, int lane, int ps, int dchunks,
                                                        int64_t sn, bool is_v) {
    const int s = ins * 64 + lane;
    const int r = s / ps;
    const int ch = (s % ps) ^ (is_v ? fv(r) : fk(r));
    if (r >= BC || ch >= dchunks) return kBufOutOfRange;
    return (uint32_t)((r * sn + ch * 8) * 2);
  }

  static __device__ __forceinline__ void issue_k(const State& st, int j, char* kb) {
    const int64_t ko = (int64_t)j * st.k_tile;
    const BufRsrc rk = make_rsrc(st.kp + ko, (uint32_t)min(st.k_end - ko, (int64_t)kBufLimit));
#pragma unroll
    for (int i = 0; i < K_IPW; ++i) {
      const int ins = i * NW + st.wave;
      if (ins < K_INS) dma16_buf(rk, st.koff[i], kb + ins * 1024);
    }
  }
  static __device__ __forceinline__ void issue_v(const State& st, int j, char* vb) {
    const int64_t vo = (int64_t)j * st.v_tile;
    const BufRsrc rv = make_rsrc(st.vp + vo, (uint32_t)min(st.v_end - vo, (int64_t)kBufLimit));
#pragma unroll
    for (int i = 0; i < V_IPW; ++i) {
      const int ins = i * NW + st.wave;
      if (ins < V_INS) dma16_buf(rv, st.voff[i], vb + ins * 1024);
    }
  }

  static __device__ __forceinline__ const char* kaddr(const State& st, const char* kbuf, int i) {
    return kbuf + st.kofs[i / KB] + (i % KB) * 32 * KP;
  }

  static __device__ __forceinline__ void qk_plain(const State& st, const char* kbuf, Scores& s) {
#pragma unroll
    for (int k = 0; k < KB; ++k) s[k] = f32x16{};
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      s[i % KB] = E::mfma(lds_read16<V8>(kaddr(st, kbuf, i)), st.qf[i / KB], s[i % KB]);
  }

  static __device__ __forceinline__ bool is_edge(const State& st, int j) {
    return j * BC + BC > st.kv_limit || (CAUSAL && j * BC + BC - 1 > st.q_w0);
  }
  static __device__ __forceinline__ void mask_edge(const State& st, Scores& s, int j) {
    const int j0 = j * BC;
    // keys >= lim are excluded for this lane's query row q_w0 + l32
    const int lim = CAUSAL ? min(st.kv_limit, st.q_w0 + st.l32 + 1) : st.kv_limit;
#pragma unroll
    for (int k = 0; k < KB; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = j0 + k * 32 + (e >> 2) * 8 + st.hl * 4 + (e & 3);
        if (key >= lim) s[k][e] = -INFINITY;
      }
  }
  static __device__ __forceinline__ float row_max(const Scores& s) {
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < KB; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[k][e]);
    return max_with_other_half(mx);
  }
  // Lazy rescale given a tile's row maximum mx (raw score units).
  static __device__ __forceinline__ void rescale(State& st, float mx) {
    const float cand = mx * st.c;
    if (__builtin_amdgcn_ballot_w64(cand > st.m_run + TH)) {
      const float m_new = fmaxf(st.m_run, cand);
      if (m_new > st.m_run) {
        const float alpha = (st.m_run == -INFINITY) ? 0.f : fast_exp2(st.m_run - m_new);
        st.l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) st.acc[dt] *= alpha;
        st.m_run = m_new;
      }
    }
  }

  // Main block of iteration j: exponentials and PV of tile j (scores sc, V
  // tile vc) with S of tile j+1 (into sn, from K tile kn).  Returns this
  // lane's share of tile j+1's unmasked row maximum.
  static __device__ __forceinline__ float main_block(State& st, const Scores& sc, Scores& sn,
                                                     const char* kn, const char* vc, int j, int n,
                                                     char* kdst, char* vdst) {
    // This iteration's loads (V(j+1), then K(j+2)), one at every other
    // phase-1 step: issued together after the barrier, the 8 waves' loads
    // queue behind each other and hold the last waves back by ~600 cycles.
    const bool do_v = j + 1 < n, do_k = j + 2 < n;
    const int64_t vo = (int64_t)(j + 1) * st.v_tile, ko = (int64_t)(j + 2) * st.k_tile;
    const BufRsrc rv = make_rsrc(st.vp + vo, (uint32_t)min(st.v_end - vo, (int64_t)kBufLimit));
    const BufRsrc rk = make_rsrc(st.kp + ko, (uint32_t)min(st.k_end - ko, (int64_t)kBufLimit));
    auto load_one = [&](int x) {
      if (x < V_IPW) {
        const int ins = x * NW + st.wave;
        if (do_v && ins < V_INS) dma16_buf(rv, st.voff[x], vdst + ins * 1024);
      } else if (x < V_IPW + K_IPW) {
        const int ins = (x - V_IPW) * NW + st.wave;
        if (do_k && ins < K_INS) dma16_buf(rk, st.koff[x - V_IPW], kdst + ins * 1024);
      }
    };
    constexpr int LSTEP = (V_IPW + K_IPW) * 2 <= NQ + 1 ? 2 : 1;   // steps per load
    static_assert(V_IPW + K_IPW <= (NQ + LSTEP - 1) / LSTEP, "the loads fit in phase 1");
    const float mref = st.m_run == -INFINITY ? 0.f : st.m_run;
    float lsum = 0.f;
    V2 pp[NPAIR];
    V8 kf[NQ];
    V8 vf[NP];
    auto vload = [&](int i) {
      const char* p = vc + st.vofs[i % DT] + (i / DT) * 16 * VP;
      const V4 lo = lds_read_tr4<V4>(p);
      const V4 hi = lds_read_tr4<V4>(p + 8 * VP);
      vf[i] = concat4<V8, V4>(lo, hi);
    };
    // pair p: elements 2q, 2q+1 of 16-key chunk t = p / 4 (slot order of the
    // P operand, see FwdKernel)
    auto pair = [&](int p) {
      const int t = p / 4, q = p % 4, k = t >> 1, e = (t & 1) * 8 + 2 * q;
      const float x0 = fast_exp2(__builtin_fmaf(sc[k][e], st.c, -mref));
      const float x1 = fast_exp2(__builtin_fmaf(sc[k][e + 1], st.c, -mref));
      lsum += x0 + x1;  // fp32 sum of the unrounded p
      pp[p] = E::cvt2(x0, x1);
      asm volatile("" : "+v"(lsum));
      asm volatile("" : "+v"(pp[p]));
    };
    auto pfrag = [&](int t) {
      const V4 lo = __builtin_shufflevector(pp[4 * t], pp[4 * t + 1], 0, 1, 2, 3);
      const V4 hi = __builtin_shufflevector(pp[4 * t + 2], pp[4 * t + 3], 0, 1, 2, 3);
      return concat4<V8, V4>(lo, hi);
    };

#pragma unroll
    for (int k = 0; k < KB; ++k) sn[k] = f32x16{};
#pragma unroll
    for (int i = 0; i < PF; ++i) kf[i] = lds_read16<V8>(kaddr(st, kn, i));
    // phase 1
    // In phase 1 the older wave of each SIMD pair (waves 0..3) otherwise wins
    // the issue arbitration and the younger one finishes ~80 % later; raising
    // the younger wave's priority for phase 1 evens them out a little.
    if (NW == 8 && st.wave >= NW / 2) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i % LSTEP == 0) load_one(i / LSTEP);
      if (i + PF < NQ) kf[i + PF] = lds_read16<V8>(kaddr(st, kn, i + PF));
      else vload(i + PF - NQ);
      sn[i % KB] = E::mfma(kf[i], st.qf[i / KB], sn[i % KB]);
#pragma unroll
      for (int p = (i * P1) / NQ; p < ((i + 1) * P1) / NQ; ++p) pair(p);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (NW == 8 && st.wave >= NW / 2) __builtin_amdgcn_s_setprio(0);
    // phase 2
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + PF < NP) vload(i + PF);
      st.acc[i % DT] = E::mfma(vf[i], pfrag(i / DT), st.acc[i % DT]);
      if (i < NE) {
#pragma unroll
        for (int p = P1 + (i * (NPAIR - P1)) / NE; p < P1 + ((i + 1) * (NPAIR - P1)) / NE; ++p)
          pair(p);
      } else {
        constexpr int NM = NP - NE, NV = KB * 16;
#pragma unroll
        for (int e = ((i - NE) * NV) / NM; e < ((i - NE + 1) * NV) / NM; ++e)
          mx = fmaxf(mx, sn[e / 16][e % 16]);
        asm volatile("" : "+v"(mx));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    st.l_run += lsum;
    return mx;
  }

  // Top of iteration j: K(j+1) and V(j) (loaded during iteration j-1) have
  // landed for every wave once all pass the barrier; K(j+2) and V(j+1) then
  // go, during iteration j, into the buffers iteration j-1 has finished with.
  static __device__ __forceinline__ void sync(const State& st) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // After the main block of iteration j: tile j+1's maximum and rescale.
  static __device__ __forceinline__ void finish_next(State& st, Scores& sn, int j, float mx) {
    if (j + 1 < st.n_act) {
      if (is_edge(st, j + 1)) {
        mask_edge(st, sn, j + 1);
        mx = row_max(sn);
      } else {
        mx = max_with_other_half(mx);
      }
      rescale(st, mx);
    }
  }

  static __device__ __forceinline__ void run(const FwdArgs& a, char* k0, char* v0, char* k1,
                                             char* v1) {
    State st;
    st.lane = threadIdx.x & 63;
    st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    st.hl = st.lane >> 5;
    st.l32 = st.lane & 31;

    int qblk, bh;
    block_coords(CAUSAL, blockIdx.x, a.B * a.Hq, a.nqb, qblk, bh);
    const int h = bh % a.Hq;
    const int b = bh / a.Hq;
    const int g = h / a.group;
    st.q_w0 = qblk * ROWS + st.wave * 32;

    st.kv_limit = a.Nk;
    if (a.kv_lens) st.kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
    int kv_end = st.kv_limit;
    if (CAUSAL) kv_end = min(kv_end, min(qblk * ROWS + ROWS, a.Nq));
    st.n_act = (kv_end + BC - 1) / BC;
    const int n_tiles = st.n_act;
    const int dchunks = a.d / 8;
    st.c = a.c;
    st.kp = (const char*)((const T*)a.k + b * a.k_sb + g * a.k_sh);
    st.vp = (const char*)((const T*)a.v + b * a.v_sb + g * a.v_sh);
    st.k_tile = (int64_t)BC * a.k_sn * 2;
    st.v_tile = (int64_t)BC * a.v_sn * 2;
    // the resources end at the last valid key: rows past kv_lens (which may
    // hold anything, e.g. an unwritten cache tail) read as zero, so that
    // their P = 0 never meets a NaN or an infinity
    st.k_end = max(((int64_t)(st.kv_limit - 1) * a.k_sn + a.d) * 2, (int64_t)0);
    st.v_end = max(((int64_t)(st.kv_limit - 1) * a.v_sn + a.d) * 2, (int64_t)0);
#pragma unroll
    for (int i = 0; i < K_IPW; ++i)
      st.koff[i] = dma_offset(i * NW + st.wave, st.lane, KPS, dchunks, a.k_sn, false);
#pragma unroll
    for (int i = 0; i < V_IPW; ++i)
      st.voff[i] = dma_offset(i * NW + st.wave, st.lane, VPS, dchunks, a.v_sn, true);
    // K read: lane holds key row l32 (+32 k), chunk 2 ks + hl.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      st.kofs[ks] = st.l32 * KP + (((2 * ks + st.hl) ^ fk(st.l32)) * 16);
    // V transposed read: in each 16-lane group lane i points at row
    // 4 (group / 2) + i / 4 (+16 t, +8), column 16 (group % 2) + 4 (i % 4)
    // (+32 dt), so that lane l gets column l of four consecutive rows.
    {
      const int grp = st.lane >> 4, gi = st.lane & 15;
      const int vr = 4 * (grp >> 1) + (gi >> 2), vcol = 2 * (grp & 1) + ((gi & 3) >> 1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        st.vofs[dt] = vr * VP + (((vcol + 4 * dt) ^ fv(vr)) * 16) + (gi & 1) * 8;
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

    Scores s0, s1;
    if (n_tiles > 0) {
      // tile j: K in k[j%2], V in v[j%2]
      issue_k(st, 0, k0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      qk_plain(st, k0, s0);
      if (is_edge(st, 0)) mask_edge(st, s0, 0);
      rescale(st, row_max(s0));
      issue_v(st, 0, v0);
      if (1 < n_tiles) issue_k(st, 1, k1);
      // Every iteration also computes S of the following tile; after the
      // last tile that result is not used (the K buffer then holds stale
      // data, which is harmless).
      for (int j = 0; j < n_tiles; j += 2) {
        sync(st);
        finish_next(st, s1, j, main_block(st, s0, s1, k1, v0, j, n_tiles, k0, v1));
        if (j + 1 >= n_tiles) break;
        sync(st);
        finish_next(st, s0, j + 1, main_block(st, s1, s0, k0, v1, j + 1, n_tiles, k1, v0));
      }
    }

    // Epilogue: O /= l, LSE = ln2 (m + log2 l).
    T* op = (T*)a.o + b * a.o_sb + h * a.o_sh;
    const float l_tot = add_with_other_half(st.l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const int row = st.q_w0 + st.l32;
    V8 seg[DT][2];   // 16-byte row segments (all lanes take part in the swaps)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        V4 g[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int r = 8 * p + 4 * q;
          const auto lo = E::cvt2(st.acc[dt][r + 0] * inv, st.acc[dt][r + 1] * inv);
          const auto hi = E::cvt2(st.acc[dt][r + 2] * inv, st.acc[dt][r + 3] * inv);
          g[q] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
        }
        seg[dt][p] = out_segment16<V8, V4>(g[0], g[1]);
      }
    if (row < a.Nq) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int col = dt * 32 + (2 * p + st.hl) * 8;
          if (col < a.d) *(V8*)(op + row * a.o_sn + col) = seg[dt][p];
        }
      if (st.hl == 0)
        a.lse[((int64_t)b * a.Hq + h) * a.Nq + row] =
            l_tot > 0.f ? (st.m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
  }
};

template <class E, int D, int BC, bool CAUSAL, int NW, int DK = D>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pipe_kernel(FwdArgs a) {
  using K = FwdPipeKernel<E, D, BC, CAUSAL, NW, DK>;
  __shared__ __attribute__((aligned(1024))) char k0[K::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[K::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[K::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[K::V_BYTES];
  K::run(a, k0, v0, k1, v1);
}

}  // namespace attn
