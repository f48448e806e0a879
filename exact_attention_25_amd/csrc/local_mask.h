// Local visibility of keys -- a sliding window and a 2-D neighbourhood -- as
// key ranges (for skipping whole tiles) and 64-bit masks over 64 consecutive
// keys (for the elements of the tiles that remain), plus the tanh soft cap.
//
//   window (flash_attn_func's window_size, "如何在ChatGLM2-6B中集成
//   Flash-Attention2？" §3 step 3): key j is visible to the query at position
//   p iff p - win_l <= j <= p + win_r.  The host stores an open side as
//   Nq + Nk, and folds causal masking in as win_r <= 0.
//
//   grid (the neighbourhood mask_mod of the PyTorch attention-options
//   article, atyun.com/61003, "Mask Mod示例：邻域屏蔽"): position t is cell
//   (t / cols, t % cols) of a row-major grid, and key j is visible iff its
//   row differs from the query's by less than nbr_r and its column by less
//   than nbr_c.  cols == 0 disables it.
//
// Both relations are monotone in p (the visible range of p + 1 starts and
// ends no earlier than that of p), so the keys visible to any of the rows
// p0..p1 lie in [lo(p0), hi(p1)].  Both are symmetric under swapping the
// query and the key with win_l and win_r exchanged, which gives the
// transposed masks the dK/dV pass needs.
#pragma once

#include <stdint.h>

namespace attn {

struct LocalVis {
  int32_t win_l, win_r;         // window bounds (an open side: Nq + Nk)
  int32_t cols, nbr_r, nbr_c;   // grid; cols == 0: no grid

  // Per-lane constants of the query at position p.
  struct Row {
    int p;
    int r;          // grid row of p
    int c_lo, c_hi; // visible grid columns
  };

  __device__ __forceinline__ Row row(int p) const {
    Row w;
    w.p = p;
    w.r = 0;
    w.c_lo = 0;
    w.c_hi = -1;
    if (cols > 0) {
      w.r = p / cols;
      const int c = p - w.r * cols;
      w.c_lo = max(c - nbr_c + 1, 0);
      w.c_hi = min(c + nbr_c - 1, cols - 1);
    }
    return w;
  }

  // Keys [lo, hi] that may be visible to one of the positions p0 <= p1,
  // within [0, lim).  Empty when hi < lo.
  __device__ __forceinline__ void key_range(int p0, int p1, int lim, int& lo, int& hi) const {
    lo = max(p0 - win_l, 0);
    hi = min(p1 + win_r, lim - 1);
    if (cols > 0) {
      lo = max(lo, (p0 / cols - nbr_r + 1) * cols);
      hi = min(hi, (p1 / cols + nbr_r) * cols - 1);
    }
  }

  // Bits a..b (clamped to 0..63) of a 64-bit word; 0 when a > b.
  static __device__ __forceinline__ uint64_t span_bits(int a, int b) {
    a = max(a, 0);
    b = min(b, 63);
    return a > b ? 0ull : ((~0ull >> (63 - (b - a))) << a);
  }

  // Bit i set iff key j0 + i (< lim) is visible to the query of `w`.
  __device__ __forceinline__ uint64_t bits(const Row& w, int j0, int lim) const {
    const int lo = max(w.p - win_l, 0), hi = min(w.p + win_r, lim - 1);
    uint64_t m = span_bits(lo - j0, hi - j0);
    if (cols > 0) {
      uint64_t g = 0;
      const int r0 = max(j0 / cols, w.r - nbr_r + 1);
      const int r1 = min((j0 + 63) / cols, w.r + nbr_r - 1);
      for (int r = r0; r <= r1; ++r)
        g |= span_bits(r * cols + w.c_lo - j0, r * cols + w.c_hi - j0);
      m &= g;
    }
    return m;
  }

  // The same relation with queries and keys exchanged: the queries that see
  // key j are those p with j - win_r <= p <= j + win_l (and the same grid
  // test).
  __device__ __forceinline__ LocalVis transposed() const {
    LocalVis t = *this;
    t.win_l = win_r;
    t.win_r = win_l;
    return t;
  }
};

// s -> -inf where bit `bit` of w is clear; w's bits are per-lane.
__device__ __forceinline__ float keep_if_bit(float s, uint32_t w, int bit) {
  const int t = (int)(w << (31 - bit)) >> 31;  // all ones iff the bit is set
  return __int_as_float((__float_as_int(s) & t) | (int)(0xff800000u & ~(uint32_t)t));
}

// Soft cap in log2 units: for the raw product z = q.k, returns
// cap * tanh(scale * z / cap) * log2(e) through tanh(u) = 1 - 2 / (1 + e^2u):
// a = cap * log2(e), c2 = 2 * scale * log2(e) / cap.  Saturates to +-a
// (exp2 -> inf gives 1 / inf = 0, exp2 -> 0 gives 1).
__device__ __forceinline__ float softcap_log2(float z, float a, float c2) {
  return __builtin_fmaf(-2.0f * a, __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * c2)), a);
}

// The soft cap in the backward: the capped logit (log2 units) of the raw
// product z and, in g, the cap's derivative factor 1 - tanh^2 = 4 r (1 - r)
// with r = 1 / (1 + 2^(z c2)) (t = a (1 - 2 r)).  A masked score (z = -inf)
// stays at -inf, where the cap alone would give -a.
__device__ __forceinline__ float softcap_grad(float z, float a, float c2, float& g) {
  const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * c2));
  const float fr = 4.0f * r;
  g = __builtin_fmaf(-fr, r, fr);
  const float t = __builtin_fmaf(-2.0f * a, r, a);
  return z == -INFINITY ? -INFINITY : t;
}

}  // namespace attn
