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
// registers.  K/V tiles of BC keys stream through LDS (padded row pitches),
// filled by direct global->LDS loads: at d = 128 double-buffered (the load of
// tile j+1 runs while tile j is in use), at d <= 64 in three stages (loads two
// tiles ahead; such a tile is too short to cover one load).  With NW = 8 (two
// waves per SIMD) the waves of a SIMD overlap each other's LDS and VALU
// latency.
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
//
// Local attention (LOCAL: sliding window and/or 2-D neighbourhood, with
// causal masking folded into the window, see local_mask.h): the work-group
// loads only the key tiles that may be visible to one of its rows, and each
// wave computes only the tiles inside its own rows' key range that hold a
// visible key for at least one of its lanes; the elements of those tiles are
// masked through a 64-bit visibility word per lane (skipped when every key
// of the tile is visible to every row).  SOFTCAP replaces each scaled logit
// by cap * tanh(logit / cap) right after QK^T.
#pragma once

#include "attn_kernels.h"
#include "device_common.h"
#include "local_mask.h"

namespace attn {

constexpr float kRescaleThreshold = 8.0f;  // log2 units: p stays <= 256

template <class E, int D, int NW, int BC, bool CAUSAL, bool MASK, bool LOCAL = false,
          bool SOFTCAP = false>
struct FwdKernel {
  static_assert(!(LOCAL && CAUSAL), "causal masking is part of the window under LOCAL");
  static_assert(!LOCAL || BC == 64, "LOCAL masks a tile through one 64-bit word");
  // scores leave the QK^T step already in log2 units (otherwise the scale
  // is folded into the exponent)
  static constexpr bool PRE = MASK || SOFTCAP;
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  // LDS row pitches in 16-byte slots.  At d = 128 K rows get one pad slot:
  // the 16 rows that one read instruction touches at a time (same chunk) then
  // fall on 16 different bank groups; V rows get a pitch of 64 (mod 256)
  // bytes: the transposed read takes 4 consecutive rows x 64 bytes per
  // half-wave, which then cover all 64 banks.  At d <= 64 (SWZ) rows are not
  // padded -- a pad slot is a load lane that moves nothing, and short tiles
  // are bound by load instructions -- and chunk c of row r sits at slot
  // c ^ f(r) instead: f_K(r) = (r / 2) mod 8 spreads the 16 rows of a K read
  // over the 16 bank groups, f_V(r) = 4 ((r / 2) mod 2) does the same for the
  // 4 rows x 4 chunks of a half-wave's transposed V read.  Read addresses are
  // per-lane bases plus compile-time offsets (one base per K k-step and per V
  // d-tile under SWZ).
  static constexpr bool SWZ = D == 64;
  static constexpr int KPS = SWZ ? CPR : CPR + 1;
  static constexpr int VPS = SWZ ? CPR : CPR + 4;
  static constexpr int KP = KPS * 16, VP = VPS * 16;   // pitches in bytes
  static constexpr int K_BYTES = BC * KP, V_BYTES = BC * VP;
  static constexpr int K_INS = (BC * KPS + 63) / 64;   // DMA instructions per K tile
  static constexpr int V_INS = (BC * VPS + 63) / 64;
  static constexpr int K_IPW = (K_INS + NW - 1) / NW;  // ... per wave
  static constexpr int V_IPW = (V_INS + NW - 1) / NW;
  // LDS stages.  At d <= 64 a tile is too short to cover a load issued one
  // tile ahead, so three stages (loads two tiles ahead) are kept; three still
  // leave room for two work-groups per CU.  At d = 128 two.
  static constexpr int NST = D <= 64 ? 3 : 2;
  static constexpr int ROWS = NW * 32;              // query rows per block
  static constexpr int KB = BC / 32;                // 32-key blocks per tile
  static constexpr int KS = D / 16;                 // k-steps of QK^T
  static constexpr int DT = D / 32;                 // 32-wide d tiles of O
  static constexpr int PT = BC / 16;                // k-steps of PV

  using T = typename E::T;
  using V8 = typename E::V8;
  using V4 = typename E::V4;

  struct State {
    int lane, wave, hl, l32;
    int b, h;                   // batch and q-head of this block
    int q_w0;                   // first query row of this wave
    int kv_limit;               // keys >= kv_limit are excluded
    int n_act;                  // tiles this wave has to visit (causal)
    int dma_n;                  // DMA instructions this wave issues per tile
    int ld_j0;                  // first key of the tile to load during this tile (-1: none)
    char* ld_kb;
    char* ld_vb;
    int t_lo, t_hi;             // LOCAL: this wave's tiles [t_lo, t_hi)
    LocalVis::Row lrow;         // LOCAL: this lane's query position
    const char* kp;             // K / V of this (batch, kv-head), key 0
    const char* vp;
    int64_t k_tile, v_tile;     // bytes between consecutive tiles
    int64_t k_end, v_end;       // bytes from kp / vp to the end of key kv_limit-1
    // per DMA instruction of this lane: byte offset (within a tile) of the
    // chunk it copies, kBufOutOfRange for pad slots and columns past d
    uint32_t koff[K_IPW], voff[V_IPW];
    int kbase, vbase;           // per-lane LDS byte offsets of the read patterns
    int kofs[SWZ ? KS : 1];     // SWZ: per k-step K read offsets
    int vofs[SWZ ? DT : 1];     // SWZ: per d-tile V read offsets
    float c;                    // scale * log2(e)
    V8 qf[KS];                  // Q fragments (B operand of S^T = K Q^T)
    f32x16 acc[DT];             // O^T accumulators
    float m_run, l_run;
  };

  // Byte offset, within a tile of row pitch sn elements, of the chunk that
  // lane copies in DMA instruction `ins` of a tile with `ps` slots per row
  // (is_v: the V tile, whose swizzle differs under SWZ).
  static __device__ __forceinline__ uint32_t dma_offset(int ins, int lane, int ps, int dchunks,
                                                        int64_t sn, bool is_v) {
    const int s = ins * 64 + lane;
    const int r = s / ps;
    int ch = s % ps;
    if (SWZ) ch ^= is_v ? 4 * ((r >> 1) & 1) : (r >> 1) & 7;
    if (r >= BC || ch >= dchunks) return kBufOutOfRange;
    return (uint32_t)((r * sn + ch * 8) * 2);
  }

  // Direct loads of one K tile and one V tile (keys j0..j0+BC-1), through
  // buffer resources that end at the last valid key (kv_limit-1): rows past
  // it, pad slots and columns past d read as zero.  Keys past the end are masked to -inf and
  // zero K columns meet zero Q columns, so none of them reach the result.
  static __device__ __forceinline__ void issue(const State& st, int j0, char* kb, char* vb) {
    const int64_t ko = (int64_t)(j0 / BC) * st.k_tile, vo = (int64_t)(j0 / BC) * st.v_tile;
    const BufRsrc rk = make_rsrc(st.kp + ko, (uint32_t)min(st.k_end - ko, (int64_t)kBufLimit));
    const BufRsrc rv = make_rsrc(st.vp + vo, (uint32_t)min(st.v_end - vo, (int64_t)kBufLimit));
#pragma unroll
    for (int i = 0; i < K_IPW; ++i) {
      const int ins = i * NW + st.wave;
      if (ins < K_INS) dma16_buf(rk, st.koff[i], kb + ins * 1024);
    }
#pragma unroll
    for (int i = 0; i < V_IPW; ++i) {
      const int ins = i * NW + st.wave;
      if (ins < V_INS) dma16_buf(rv, st.voff[i], vb + ins * 1024);
    }
  }

  // One KV tile: S^T, masking, online softmax, PV.  bits (LOCAL): bit i set
  // iff key j0 + i is visible to this lane's row.
  static __device__ __forceinline__ void tile(const FwdArgs& a, State& st, const char* kbuf,
                                              const char* vbuf, int j0, uint64_t bits) {
    // S^T = K_j Q^T, with this wave's loads of the next tile (ld_j0, if any)
    // spread over its first MFMAs: issued together after the barrier, the 8
    // waves' loads queue behind each other and hold the last waves back
    const bool ld = st.ld_j0 >= 0;
    const int64_t lko = (int64_t)(st.ld_j0 / BC) * st.k_tile, lvo = (int64_t)(st.ld_j0 / BC) * st.v_tile;
    const BufRsrc lrk = make_rsrc(st.kp + lko, (uint32_t)min(st.k_end - lko, (int64_t)kBufLimit));
    const BufRsrc lrv = make_rsrc(st.vp + lvo, (uint32_t)min(st.v_end - lvo, (int64_t)kBufLimit));
    auto load_one = [&](int x) {
      if (!ld) return;
      if (x < K_IPW) {
        const int ins = x * NW + st.wave;
        if (ins < K_INS) dma16_buf(lrk, st.koff[x], st.ld_kb + ins * 1024);
      } else if (x < K_IPW + V_IPW) {
        const int ins = (x - K_IPW) * NW + st.wave;
        if (ins < V_INS) dma16_buf(lrv, st.voff[x - K_IPW], st.ld_vb + ins * 1024);
      }
    };
    f32x16 s[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) s[k] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks * 2 < K_IPW + V_IPW) { load_one(ks * 2); load_one(ks * 2 + 1); }
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const V8 kf = SWZ ? lds_read16<V8>(kbuf + st.kofs[SWZ ? ks : 0] + k * 32 * KP)
                          : lds_read16<V8>(kbuf + st.kbase + k * 32 * KP + ks * 32);
        s[k] = E::mfma(kf, st.qf[ks], s[k]);
      }
    }

    const int qrow = st.q_w0 + st.l32;
    if constexpr (SOFTCAP) {
#pragma unroll
      for (int k = 0; k < KB; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[k][r] = softcap_log2(s[k][r], a.cap_a, a.cap_c2);
    }
    if constexpr (MASK) {
      const int mrow = min(qrow, a.Nq - 1);
      const float* mp = a.mask + st.b * a.m_sb + st.h * a.m_sh + (int64_t)mrow * a.m_sq;
#pragma unroll
      for (int k = 0; k < KB; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + k * 32 + (r >> 2) * 8 + st.hl * 4 + (r & 3);
          s[k][r] = (SOFTCAP ? s[k][r] : s[k][r] * st.c) + mp[min(key, a.Nk - 1)] * kLog2e;
        }
    }
    if constexpr (LOCAL) {
      // lane half hl holds keys k*32 + (r/4)*8 + 4 hl + r%4 of the tile
      if (__builtin_amdgcn_ballot_w64(bits != ~0ull)) {
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          const uint32_t w = (uint32_t)(bits >> (k * 32 + st.hl * 4));
#pragma unroll
          for (int r = 0; r < 16; ++r) s[k][r] = keep_if_bit(s[k][r], w, (r >> 2) * 8 + (r & 3));
        }
      }
    } else {
      const bool edge = (j0 + BC > st.kv_limit) || (CAUSAL && j0 + BC - 1 > st.q_w0);
      if (edge) {
        // register r of block k holds key j0 + 4 hl + k*32 + (r/4)*8 + r%4: one
        // limit per lane relative to j0 + 4 hl (key lengths and the diagonal
        // together), so each element costs a compare with a constant and a
        // select; the empty asm keeps the compares in this branch
        int lim = st.kv_limit - j0 - 4 * st.hl;
        if (CAUSAL) lim = min(lim, qrow + 1 - j0 - 4 * st.hl);
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int k = 0; k < KB; ++k)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (k * 32 + (r >> 2) * 8 + (r & 3) >= lim) s[k][r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < KB; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[k][r]);
    mx = max_with_other_half(mx);
    const float cand = PRE ? mx : mx * st.c;
    if (__builtin_amdgcn_ballot_w64(cand > st.m_run + kRescaleThreshold)) {
      // while no row of the wave has a finite reference point O and l are
      // still zero: nothing to rescale
      const bool any_ref = __builtin_amdgcn_ballot_w64(st.m_run != -INFINITY) != 0;
      const float m_new = fmaxf(st.m_run, cand);
      if (m_new > st.m_run) {
        if (any_ref) {
          const float alpha = (st.m_run == -INFINITY) ? 0.f : fast_exp2(st.m_run - m_new);
          st.l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) st.acc[dt] *= alpha;
        }
        st.m_run = m_new;
      }
    }
    const float mref = st.m_run == -INFINITY ? 0.f : st.m_run;
    float lsum = 0.f;
    // 16-key chunks wholly past kv_limit (the ragged end of the key range)
    // hold only p = 0: their exponentials and PV products are skipped
    const int live = __builtin_amdgcn_readfirstlane(st.kv_limit - j0);
    V8 pf[PT];
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      pf[t] = V8{};
      if (t > 0 && t * 16 >= live) continue;
      const int k = t >> 1, r0 = (t & 1) * 8;
      typename E::V2 pp[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x0 = s[k][r0 + 2 * q], x1 = s[k][r0 + 2 * q + 1];
        x0 = fast_exp2(PRE ? x0 - mref : __builtin_fmaf(x0, st.c, -mref));
        x1 = fast_exp2(PRE ? x1 - mref : __builtin_fmaf(x1, st.c, -mref));
        lsum += x0 + x1;
        pp[q] = E::cvt2(x0, x1);
      }
      V4 lo = __builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3);
      V4 hi = __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3);
      pf[t] = concat4<V8, V4>(lo, hi);
    }
    st.l_run += lsum;

    // O^T += V_j^T P^T
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      if (t > 0 && t * 16 >= live) continue;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const char* p = SWZ ? vbuf + st.vofs[SWZ ? dt : 0] + t * 16 * VP
                            : vbuf + st.vbase + t * 16 * VP + dt * 64;
        const V4 lo = lds_read_tr4<V4>(p);
        const V4 hi = lds_read_tr4<V4>(p + 8 * VP);
        st.acc[dt] = E::mfma(concat4<V8, V4>(lo, hi), pf[t], st.acc[dt]);
      }
    }
  }

  // Tile j with loads kept two tiles ahead (NST = 3): this wave's share of
  // tile j has landed once at most the dma_n loads of tile j+1 are
  // outstanding; after the barrier every wave's share has, and every wave is
  // done with tile j-1, whose stage takes tile j+2.  A plain s_barrier: the
  // workgroup fence of __syncthreads would wait for tile j+1 as well.  The
  // empty asm statements keep LDS accesses on their side of it.
  static __device__ __forceinline__ void step3(const FwdArgs& a, State& st, int j, int t_end,
                                               const char* kc, const char* vc, char* kn, char* vn) {
    if (j + 1 < t_end) wait_vmem(st.dma_n);
    else wait_vmem(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    st.ld_j0 = j + 2 < t_end ? (j + 2) * BC : -1;
    st.ld_kb = kn;
    st.ld_vb = vn;
    body(a, st, j, kc, vc);
  }

  static __device__ __forceinline__ void step(const FwdArgs& a, State& st, int j, int t_end,
                                              const char* kc, const char* vc, char* kn, char* vn) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's share of tile j has landed
    __syncthreads();
    st.ld_j0 = j + 1 < t_end ? (j + 1) * BC : -1;
    st.ld_kb = kn;
    st.ld_vb = vn;
    body(a, st, j, kc, vc);
  }

  // tile j unless this wave has nothing to do in it
  static __device__ __forceinline__ void body(const FwdArgs& a, State& st, int j, const char* kc,
                                              const char* vc) {
    bool done = false;
    if constexpr (LOCAL) {
      if (j >= st.t_lo && j < st.t_hi) {
        const uint64_t bits = a.loc.bits(st.lrow, j * BC, st.kv_limit);
        if (__builtin_amdgcn_ballot_w64(bits != 0)) {
          tile(a, st, kc, vc, j * BC, bits);
          done = true;
        }
      }
    } else {
      if (j < st.n_act) {
        tile(a, st, kc, vc, j * BC, 0);
        done = true;
      }
    }
    if (!done && st.ld_j0 >= 0) issue(st, st.ld_j0, st.ld_kb, st.ld_vb);
  }


  // Per-wave set-up: block `wid` -> (batch, head, query block), key range,
  // load offsets, Q fragments, zero accumulators.  Returns the number of key
  // tiles the block spans (before LOCAL narrows it).
  static __device__ __forceinline__ int setup(const FwdArgs& a, State& st, int hw_id) {
    st.lane = threadIdx.x & 63;
    st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    st.hl = st.lane >> 5;
    st.l32 = st.lane & 31;

    int qblk, bh;
    block_coords(CAUSAL, hw_id, a.B * a.Hq, a.nqb, qblk, bh);
    const int h = bh % a.Hq;
    const int b = bh / a.Hq;
    st.b = b;
    st.h = h;
    const int g = h / a.group;
    const int q_blk0 = qblk * ROWS;
    st.q_w0 = q_blk0 + st.wave * 32;

    st.kv_limit = a.Nk;
    if (a.kv_lens) st.kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
    int kv_end = st.kv_limit;
    if (CAUSAL) kv_end = min(kv_end, min(q_blk0 + ROWS, a.Nq));
    const int n_tiles = (kv_end + BC - 1) / BC;
    // causal: a wave sees no key beyond its last row; a wave whose rows all
    // lie past Nq only helps with the loads
    st.n_act = CAUSAL ? min(n_tiles, (st.q_w0 + 31) / BC + 1) : n_tiles;
    if (st.q_w0 >= a.Nq) st.n_act = 0;
    const int dchunks = a.d / 8;
    st.c = a.c;
    st.kp = (const char*)((const T*)a.k + b * a.k_sb + g * a.k_sh);
    st.vp = (const char*)((const T*)a.v + b * a.v_sb + g * a.v_sh);
    st.k_tile = (int64_t)BC * a.k_sn * 2;
    st.v_tile = (int64_t)BC * a.v_sn * 2;
    // rows past kv_lens read as zero (their contents never reach O)
    st.k_end = max(((int64_t)(st.kv_limit - 1) * a.k_sn + a.d) * 2, (int64_t)0);
    st.v_end = max(((int64_t)(st.kv_limit - 1) * a.v_sn + a.d) * 2, (int64_t)0);
#pragma unroll
    for (int i = 0; i < K_IPW; ++i)
      st.koff[i] = dma_offset(i * NW + st.wave, st.lane, KPS, dchunks, a.k_sn, false);
#pragma unroll
    for (int i = 0; i < V_IPW; ++i)
      st.voff[i] = dma_offset(i * NW + st.wave, st.lane, VPS, dchunks, a.v_sn, true);
    st.dma_n = 0;
#pragma unroll
    for (int i = 0; i < K_IPW; ++i) st.dma_n += i * NW + st.wave < K_INS;
#pragma unroll
    for (int i = 0; i < V_IPW; ++i) st.dma_n += i * NW + st.wave < V_INS;
    // K read: lane holds key row l32 (+32 k), chunk 2 ks + hl.
    st.kbase = st.l32 * KP + st.hl * 16;
    // V transposed read: in each 16-lane group lane i points at row
    // 4 (group / 2) + i / 4 (+16 t, +8), column 16 (group % 2) + 4 (i % 4)
    // (+32 dt), so that lane l gets column l of four consecutive rows.
    {
      const int grp = st.lane >> 4, gi = st.lane & 15;
      st.vbase = (4 * (grp >> 1) + (gi >> 2)) * VP + (16 * (grp & 1) + 4 * (gi & 3)) * 2;
      if constexpr (SWZ) {
        // K: chunk 2 ks + hl of row l32 (+32 k: same f_K); V: chunk
        // 2 (group % 2) + (i % 4) / 2 + 4 dt of row 4 (group / 2) + i / 4
        // (+16 t, +8: same f_V), byte 8 (i % 2) within it
        const int fk = (st.l32 >> 1) & 7;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          st.kofs[SWZ ? ks : 0] = st.l32 * KP + (((2 * ks + st.hl) ^ fk) * 16);
        const int vr = 4 * (grp >> 1) + (gi >> 2);
        const int vc = 2 * (grp & 1) + ((gi & 3) >> 1);
        const int fv = 4 * ((vr >> 1) & 1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          st.vofs[SWZ ? dt : 0] = vr * VP + (((vc + 4 * dt) ^ fv) * 16) + (gi & 1) * 8;
      }
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
    return n_tiles;
  }

  // k[s] / v[s]: the K and V buffers of stage s, each its own LDS array, so
  // that the compiler sees that a load into one stage does not write the
  // stage being read (one array with offsets makes it wait for every
  // outstanding load before each read of a tile)
  static __device__ __forceinline__ void run(const FwdArgs& a, char* const (&k)[NST],
                                             char* const (&v)[NST]) {
    auto kb = [&](int s) { return k[s]; };
    auto vb = [&](int s) { return v[s]; };
    State st;
    const int n_tiles = setup(a, st, blockIdx.x);
    const int q_blk0 = st.q_w0 - st.wave * 32;

    // tiles [t_begin, t_end) pass through LDS
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
      st.lrow = a.loc.row(min(st.q_w0 + st.l32, a.Nq - 1));
    }
    if (t_begin < t_end) issue(st, t_begin * BC, kb(0), vb(0));
    if constexpr (NST == 2) {
      for (int j = t_begin; j < t_end; j += 2) {
        step(a, st, j, t_end, kb(0), vb(0), kb(1), vb(1));
        if (j + 1 >= t_end) break;
        step(a, st, j + 1, t_end, kb(1), vb(1), kb(0), vb(0));
      }
    } else {
      if (t_begin + 1 < t_end) issue(st, (t_begin + 1) * BC, kb(1), vb(1));
      for (int j = t_begin; j < t_end; j += 3) {
        step3(a, st, j, t_end, kb(0), vb(0), kb(2), vb(2));
        if (j + 1 >= t_end) break;
        step3(a, st, j + 1, t_end, kb(1), vb(1), kb(0), vb(0));
        if (j + 2 >= t_end) break;
        step3(a, st, j + 2, t_end, kb(2), vb(2), kb(1), vb(1));
      }
    }

    epilogue(a, st);
  }

  // O /= l (one reciprocal per row), rounded to the output type; LSE.
  static __device__ __forceinline__ void epilogue(const FwdArgs& a, const State& st) {
    T* op = (T*)a.o + st.b * a.o_sb + st.h * a.o_sh;
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
        a.lse[((int64_t)st.b * a.Hq + st.h) * a.Nq + row] =
            l_tot > 0.f ? (st.m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
  }
};

template <class E, int D, int NW, int BC, bool CAUSAL, bool MASK, bool LOCAL = false,
          bool SOFTCAP = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4)))
void fwd_kernel(FwdArgs a) {
  using K = FwdKernel<E, D, NW, BC, CAUSAL, MASK, LOCAL, SOFTCAP>;
  __shared__ __attribute__((aligned(1024))) char k0[K::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[K::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[K::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[K::V_BYTES];
  if constexpr (K::NST == 3) {
    __shared__ __attribute__((aligned(1024))) char k2[K::K_BYTES];
    __shared__ __attribute__((aligned(1024))) char v2[K::V_BYTES];
    char* const kb[3] = {k0, k1, k2};
    char* const vb[3] = {v0, v1, v2};
    K::run(a, kb, vb);
  } else {
    char* const kb[2] = {k0, k1};
    char* const vb[2] = {v0, v1};
    K::run(a, kb, vb);
  }
}

}  // namespace attn
