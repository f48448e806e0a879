// Split-KV decode attention for gfx950: few new queries (Nq, typically 1 to
// 16) against a long key/value cache.  The pages leave decode to
// FlashDecoding ("FlashAttention技术解析：优化Transformer注意力计算效率"
// (jsqmd.com/news/722897) §5.2, decode phase): the key range is cut into
// splits that run in parallel, each producing a partial result of the same
// online softmax as the forward (§2.2), and the partials are merged through
// their log-sum-exp.  For split s with partial output O_s (normalised) and
// LSE_s:  LSE = log sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s.
//
// The Nq queries of the `group` q-heads that share a kv-head are stacked as
// the rows of one tile, so every K/V byte read serves all of them.  One
// wave per (batch, kv-head, 32-row block, split): it streams its key range
// in tiles of 32 keys through its own double-buffered LDS (direct
// buffer->LDS loads; a work-group is a single wave, so waiting for its own
// loads is all the synchronisation there is), computes S^T = K Q^T and
// O^T += V^T P^T on MFMA exactly as the forward kernel does, and writes
// the normalised partial O (fp32) and its LSE to the workspace.
//
// Query i of a batch with L valid keys sits at position p = L - Nq + i and
// sees keys p - win_l .. p + win_r (causal and the sliding window, see
// local_mask.h).  The splits tile only the keys some query can see, from
// max(0, L - Nq - win_l) on, so a bounded window reads just its last keys.
// SOFTCAP applies the tanh soft cap to the scaled logits.
#include "attn_kernels.h"
#include "device_common.h"
#include "local_mask.h"

namespace attn {

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima, i.e. not waited for).
__host__ __device__ constexpr int vm_wait(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}
// ... that waits for all LDS operations only (vmcnt and expcnt at their maxima)
constexpr int kLdsOnly = 0xC07F;

template <class E, int D, bool SOFTCAP>
struct DecodeSplit {
  static constexpr int BC = 32;                 // keys per tile
  static constexpr int CPR = D / 8;
  static constexpr int KPS = CPR + 1, VPS = CPR + 4;   // LDS pitches in 16-byte slots (as the forward)
  static constexpr int KP = KPS * 16, VP = VPS * 16;
  static constexpr int K_BYTES = BC * KP, V_BYTES = BC * VP;
  static constexpr int K_INS = (BC * KPS + 63) / 64;
  static constexpr int V_INS = (BC * VPS + 63) / 64;
  static constexpr int KS = D / 16, DT = D / 32, PT = BC / 16;

  using T = typename E::T;
  using V8 = typename E::V8;
  using V4 = typename E::V4;

  struct State {
    int hl, l32;
    int row_lo, row_lim;        // this lane's row sees keys row_lo .. row_lim - 1
    const char* kp;
    const char* vp;
    int64_t tile_bytes, k_end;
    uint32_t koff[K_INS], voff[V_INS];
    int kbase, vbase;
    float c;
    float cap_a, cap_c2;        // soft cap constants (SOFTCAP)
    V8 qf[KS];
    f32x16 acc[DT];
    float m, l;
  };

  static __device__ __forceinline__ uint32_t dma_offset(int ins, int lane, int ps, int dchunks,
                                                        int64_t sn) {
    const int s = ins * 64 + lane;
    const int r = s / ps, ch = s % ps;
    if (r >= BC || ch >= dchunks) return kBufOutOfRange;
    return (uint32_t)((r * sn + ch * 8) * 2);
  }

  // K and V rows key_lo + jr .. +31 (rows past the valid length read as
  // zero); jr is a multiple of BC
  static __device__ __forceinline__ void issue(const State& st, int jr, char* kb, char* vb) {
    // the buffer may have just been read by this wave: its LDS reads finish first
    __builtin_amdgcn_s_waitcnt(kLdsOnly);
    const int64_t o = (int64_t)(jr / BC) * st.tile_bytes;
    const uint32_t n = (uint32_t)min(st.k_end - o, (int64_t)kBufLimit);
    const BufRsrc rk = make_rsrc(st.kp + o, n);
    const BufRsrc rv = make_rsrc(st.vp + o, n);
#pragma unroll
    for (int i = 0; i < K_INS; ++i) dma16_buf(rk, st.koff[i], kb + i * 1024);
#pragma unroll
    for (int i = 0; i < V_INS; ++i) dma16_buf(rv, st.voff[i], vb + i * 1024);
  }

  // One tile: S^T (lane = row l32, register r = key j0 + 8 (r/4) + 4 hl + r%4),
  // exact online softmax update, O^T += V^T P^T.
  static __device__ __forceinline__ void tile(State& st, const char* kb, const char* vb, int j0) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = E::mfma(lds_read16<V8>(kb + st.kbase + ks * 32), st.qf[ks], s);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + (r >> 2) * 8 + st.hl * 4 + (r & 3);
      const float t = SOFTCAP ? softcap_log2(s[r], st.cap_a, st.cap_c2) : s[r] * st.c;
      s[r] = (key >= st.row_lo && key < st.row_lim) ? t : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    mx = max_with_other_half(mx);
    const float m_new = fmaxf(st.m, mx);
    // rows with no visible key so far keep m = -inf and take the reference 0,
    // so that every p and the rescale factor are exp2(-inf) = 0 (no branch:
    // the products below need the whole wave)
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(st.m - mref);
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc[dt] *= alpha;
    V8 pf[PT];
#pragma unroll
    for (int t = 0; t < PT; ++t) {
      typename E::V2 pp[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x0 = fast_exp2(s[t * 8 + 2 * q] - mref);
        const float x1 = fast_exp2(s[t * 8 + 2 * q + 1] - mref);
        st.l += x0 + x1;
        pp[q] = E::cvt2(x0, x1);
      }
      const V4 lo = __builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3);
      const V4 hi = __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3);
      pf[t] = concat4<V8, V4>(lo, hi);
    }
#pragma unroll
    for (int t = 0; t < PT; ++t)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const char* p = vb + st.vbase + t * 16 * VP + dt * 64;
        const V4 lo = lds_read_tr4<V4>(p);
        const V4 hi = lds_read_tr4<V4>(p + 8 * VP);
        st.acc[dt] = E::mfma(concat4<V8, V4>(lo, hi), pf[t], st.acc[dt]);
      }
  }

  static __device__ __forceinline__ void run(const DecodeArgs& a, char* k0, char* v0, char* k1,
                                             char* v1) {
    State st;
    const int lane = threadIdx.x & 63;
    st.hl = lane >> 5;
    st.l32 = lane & 31;

    int w = blockIdx.x;
    const int sp = w % a.n_splits;
    w /= a.n_splits;
    const int rb = w % a.n_rb;
    w /= a.n_rb;
    const int g = w % a.Hkv;
    const int b = w / a.Hkv;

    const int row = rb * 32 + st.l32;
    const bool valid = row < a.rows;
    const int hh = valid ? row / a.Nq : 0;
    const int qi = valid ? row % a.Nq : 0;
    const int h = g * a.group + hh;

    int kv_limit = a.Nk;
    if (a.kv_lens) kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
    const int pos = kv_limit - a.Nq + qi;   // this row's position (may be < 0)
    st.row_lo = max(pos - a.win_l, 0);
    st.row_lim = min(kv_limit, pos + a.win_r + 1);
    if (!valid) st.row_lo = st.row_lim = 0;
    // the splits start at the first key visible to the batch's first query
    const int key_lo = max(kv_limit - a.Nq - a.win_l, 0) + sp * a.split_keys;
    const int key_hi = min(key_lo + a.split_keys, kv_limit);
    const int n_tiles = key_hi > key_lo ? (key_hi - key_lo + BC - 1) / BC : 0;

    st.c = a.c;
    st.cap_a = a.cap_a;
    st.cap_c2 = a.cap_c2;
    {
      const T* qp = (const T*)a.q + b * a.q_sb + h * a.q_sh + (int64_t)qi * a.q_sn;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + st.hl * 8;
        st.qf[ks] = (valid && d0 < a.d) ? *(const V8*)(qp + d0) : V8{};
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc[dt] = f32x16{};
    st.m = -INFINITY;
    st.l = 0.f;

    st.kp = (const char*)((const T*)a.k + b * a.k_sb + g * a.k_sh + (int64_t)key_lo * a.k_sn);
    st.vp = (const char*)((const T*)a.v + b * a.k_sb + g * a.k_sh + (int64_t)key_lo * a.k_sn);
    st.tile_bytes = (int64_t)BC * a.k_sn * 2;
    // bytes from key key_lo to the end of the last valid key kv_limit-1 (used
    // only when n_tiles > 0, i.e. key_lo < kv_limit): cache rows past the
    // valid length read as zero, whatever they hold
    st.k_end = ((int64_t)(kv_limit - 1 - key_lo) * a.k_sn + a.d) * 2;
    const int dchunks = a.d / 8;
#pragma unroll
    for (int i = 0; i < K_INS; ++i) st.koff[i] = dma_offset(i, lane, KPS, dchunks, a.k_sn);
#pragma unroll
    for (int i = 0; i < V_INS; ++i) st.voff[i] = dma_offset(i, lane, VPS, dchunks, a.k_sn);
    st.kbase = st.l32 * KP + st.hl * 16;
    {
      const int grp = lane >> 4, gi = lane & 15;
      st.vbase = (4 * (grp >> 1) + (gi >> 2)) * VP + (16 * (grp & 1) + 4 * (gi & 3)) * 2;
    }

    // tile t lives in buffer t % 2; the loads of tile t+1 are issued before
    // tile t is computed, and waiting for tile t leaves them in flight
    if (n_tiles > 0) issue(st, 0, k0, v0);
    for (int t = 0; t < n_tiles; t += 2) {
      if (t + 1 < n_tiles) {
        issue(st, (t + 1) * BC, k1, v1);
        __builtin_amdgcn_s_waitcnt(vm_wait(K_INS + V_INS));
      } else {
        __builtin_amdgcn_s_waitcnt(vm_wait(0));
      }
      tile(st, k0, v0, key_lo + t * BC);
      if (t + 1 >= n_tiles) break;
      if (t + 2 < n_tiles) {
        issue(st, (t + 2) * BC, k0, v0);
        __builtin_amdgcn_s_waitcnt(vm_wait(K_INS + V_INS));
      } else {
        __builtin_amdgcn_s_waitcnt(vm_wait(0));
      }
      tile(st, k1, v1, key_lo + (t + 1) * BC);
    }

    const float l_tot = add_with_other_half(st.l);
    if (!valid) return;
    const int64_t prow = (((int64_t)sp * a.B + b) * a.Hq + h) * a.Nq + qi;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    float* po = a.part_o + prow * a.d;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = dt * 32 + gq * 8 + st.hl * 4;
        if (col < a.d) {
          f32x4 v = {st.acc[dt][gq * 4 + 0] * inv, st.acc[dt][gq * 4 + 1] * inv,
                     st.acc[dt][gq * 4 + 2] * inv, st.acc[dt][gq * 4 + 3] * inv};
          *(f32x4*)(po + col) = v;
        }
      }
    if (st.hl == 0) a.part_lse[prow] = l_tot > 0.f ? (st.m + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
};

template <class E, int D, bool SOFTCAP>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  using K = DecodeSplit<E, D, SOFTCAP>;
  __shared__ __attribute__((aligned(1024))) char k0[K::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[K::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[K::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[K::V_BYTES];
  K::run(a, k0, v0, k1, v1);
}

// One work-group of 4 waves per (batch, q-head, query):
// LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.
//  - the weights: lanes own splits (strided by 256), max and sum reduced
//    across the work-group; the weights w_s = exp(LSE_s - LSE) go to LDS;
//  - the output: wave v sums the splits s = v, v+4, ... for its columns (two
//    per lane), and the four partial sums are added in a fixed order.
// A row with no visible key in any split gets O = 0 and LSE = -inf.
constexpr int kMergeThreads = 256;
constexpr int kMergeMaxSplits = 1024;   // decode_split keeps n_splits below this

__device__ __forceinline__ float block_reduce(float x, float* red, bool is_max) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float y = __shfl_xor(x, o, 64);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  x = is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))
             : (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return x;
}

template <class E>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  using T = typename E::T;
  __shared__ float wts[kMergeMaxSplits];
  __shared__ float red[4];
  __shared__ f32x2 part[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nrow = (int64_t)a.B * a.Hq * a.Nq;
  const int64_t row = blockIdx.x;   // (b * Hq + h) * Nq + i
  const int qi = (int)(row % a.Nq);
  const int64_t bh = row / a.Nq;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int ns = a.n_splits;

  float mx = -INFINITY;
  for (int s = tid; s < ns; s += kMergeThreads) mx = fmaxf(mx, a.part_lse[s * nrow + row]);
  mx = block_reduce(mx, red, true);
  T* op = (T*)a.o + b * a.q_sb + h * a.q_sh + (int64_t)qi * a.q_sn;
  if (mx == -INFINITY) {
    for (int col = tid; col < a.d; col += kMergeThreads) op[col] = (T)0.f;
    if (tid == 0) a.lse[row] = -INFINITY;
    return;
  }
  float ws = 0.f;
  for (int s = tid; s < ns; s += kMergeThreads) ws += fast_exp2((a.part_lse[s * nrow + row] - mx) * kLog2e);
  ws = block_reduce(ws, red, false);
  const float lse = mx + fast_log2(ws) * kLn2;
  for (int s = tid; s < ns; s += kMergeThreads)
    wts[s] = fast_exp2((a.part_lse[s * nrow + row] - lse) * kLog2e);
  __syncthreads();

  // columns 2 lane, 2 lane + 1 (d <= 128); splits wave, wave + 4, ...
  const int col = 2 * lane;
  f32x2 o = {0.f, 0.f};
  if (col < a.d) {
    const float* po = a.part_o + row * a.d + col;
    const int64_t sstride = nrow * a.d;
    int s = wave;
    for (; s + 12 < ns; s += 16) {
      const f32x2 x0 = *(const f32x2*)(po + (int64_t)s * sstride);
      const f32x2 x1 = *(const f32x2*)(po + (int64_t)(s + 4) * sstride);
      const f32x2 x2 = *(const f32x2*)(po + (int64_t)(s + 8) * sstride);
      const f32x2 x3 = *(const f32x2*)(po + (int64_t)(s + 12) * sstride);
      o += wts[s] * x0;
      o += wts[s + 4] * x1;
      o += wts[s + 8] * x2;
      o += wts[s + 12] * x3;
    }
    for (; s < ns; s += 4) o += wts[s] * *(const f32x2*)(po + (int64_t)s * sstride);
  }
  part[wave][lane] = o;
  __syncthreads();
  if (wave == 0 && col < a.d) {
    const f32x2 r = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
    op[col] = (T)r[0];
    if (col + 1 < a.d) op[col + 1] = (T)r[1];
  }
  if (tid == 0) a.lse[row] = lse;
}

// Keys per split: about 2048 (batch, kv-head, row block, split) waves, eight
// per CU (4096 measured 6 % slower on a 32K-key cache: twice the merge work
// and shorter streams per wave), in multiples of 32 keys, at least 256 keys
// per split so that the merge stays small (smaller splits measured slower).
void decode_split(int B, int Hkv, int rows, int Nk, int* split_keys, int* n_splits) {
  const long rbs = (long)B * Hkv * ((rows + 31) / 32);
  long want = rbs > 0 ? (2048 + rbs - 1) / rbs : 1;
  if (want < 1) want = 1;
  long sk = Nk > 0 ? (Nk + want - 1) / want : 32;
  sk = (sk + 31) / 32 * 32;
  if (sk < 256) sk = 256;
  // at most kMergeMaxSplits splits (the merge keeps one weight per split in LDS)
  const long min_sk = ((long)Nk + kMergeMaxSplits - 1) / kMergeMaxSplits;
  if (sk < min_sk) sk = (min_sk + 31) / 32 * 32;
  *split_keys = (int)sk;
  *n_splits = Nk > 0 ? (int)((Nk + sk - 1) / sk) : 1;
}

template <class E, bool SOFTCAP>
static hipError_t launch_decode_e(const DecodeArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((long)a.B * a.Hkv * a.n_rb * a.n_splits);
  if (grid > 0) {
    if (a.d > 64)
      hipLaunchKernelGGL((decode_split_kernel<E, 128, SOFTCAP>), dim3(grid), dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<E, 64, SOFTCAP>), dim3(grid), dim3(64), 0, st, a);
  }
  const long nrow = (long)a.B * a.Hq * a.Nq;
  if (nrow > 0)
    hipLaunchKernelGGL((decode_merge_kernel<E>), dim3((unsigned)nrow), dim3(kMergeThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bool is_bf16, bool softcap, hipStream_t st) {
  if (softcap) return is_bf16 ? launch_decode_e<BF16, true>(a, st) : launch_decode_e<FP16, true>(a, st);
  return is_bf16 ? launch_decode_e<BF16, false>(a, st) : launch_decode_e<FP16, false>(a, st);
}

}  // namespace attn
