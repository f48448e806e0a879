// FP8 attention forward for gfx950 with per-block scales, and the block
// quantiser that produces its inputs.
//
// The pages' FP8 variant ("FlashAttention技术解析：优化Transformer注意力计算效率"
// (jsqmd.com/news/722897) §4.2 item 3 and §6.3 item 2): block quantisation,
// both matrix products on FP8 operands, an independent scale per block, the
// softmax statistics in fp32.  Here:
//   - format OCP E4M3FN (the conversion instructions' format on gfx950);
//   - blocks of 64 rows of one (batch, head): scale = amax / 448, so a block's
//     largest magnitude maps to 448;
//   - V is stored transposed ([B, Hkv, d, Nk rounded up to 64], keys
//     contiguous), so the operand of the PV product is read as plain rows;
//   - the products run on v_mfma_scale_f32_32x32x64_f8f6f4 (K = 64 per
//     instruction, unit hardware scales); the fp32 block scales are folded
//     into the exponent: s -> s * scale * sq * sk * log2(e) per (wave, tile).
//
// Forward, per (batch, q-head, 256 query rows); 8 waves of 32 rows; 64-key
// tiles of K (row-major) and V^T through double-buffered LDS filled by
// direct buffer->LDS loads.  Per tile and wave:
//   S^T = K Q^T    A = K rows read in a permuted order, B = Q^T from
//                  registers.  The MFMA contracts slot i of lane half h of A
//                  with slot i of lane half h of B, and its result puts row
//                  8 (r / 4) + 4 h + r % 4 in register r; reading key
//                  32 ((i / 4) % 2) + 16 blk + 4 (i / 8) + i % 4 for row i
//                  of 32-key block blk makes register r of lane half h hold
//                  key 32 h + 16 blk + r, so a lane half holds 32
//                  consecutive keys.
//   softmax        p = exp2(s c sq sk - m + log2(sv / svmax) + 6), with the
//                  reference m moved lazily, only when a tile exceeds it by
//                  more than 2.75 (so p <= 2^8.75 < 448); the V block scale
//                  sv enters through p (relative to the head's largest
//                  svmax) and the factor 2^6 keeps p above E4M3's subnormal
//                  range down to 2^-12 of the row's largest weight;
//   O^T += V^T P^T  P packed to E4M3 (slot 16 blk + r = key 32 h + 16 blk + r)
//                  as the B operand; A = 32 consecutive keys of a V^T row;
//   sums           one more MFMA with all-ones codes as A sums the rounded
//                  P over the tile's keys (every row of its result holds
//                  the column sums), the divisor of O; an fp32 sum of the
//                  unrounded p gives the LSE.
// All 16 LDS fragment reads of a tile are issued before its first MFMA.
// The block scales of tile j+1 are loaded before the barrier of tile j.
// Epilogue: O = acc * svmax * 2^-6 / l_rounded, LSE = ln2 (m + log2 l).
#include "attn_kernels.h"
#include "device_common.h"

namespace attn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // unit E8M0 scales (127) for both operands
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// E4M3 codes of four floats (nearest even) in one word, a in the low byte.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}

// ------------------------------------------------------------- quantiser
// One work-group of 256 threads per (batch, head, block of 64 rows).  The
// block is read once, in 16-byte chunks kept in registers: amax, then
// scale = amax / 448 and the codes of x * (448 / amax), both divisions and
// the product in fp32 (a zero block gets scale 1 and zero codes).  Natural
// layout: each chunk's codes are stored at once.  transpose: the codes go
// through an LDS tile to [B, H, d, ld] with keys contiguous, and the block
// writes all 64 of its columns (zeros past N).
template <class T>
__global__ __launch_bounds__(256) void fp8_quant_kernel(QuantArgs a) {
  constexpr int CH = 16 / sizeof(T);                  // elements per 16-byte chunk
  constexpr int MAXC = 64 * 128 / CH / 256;           // chunks per thread (d <= 128)
  __shared__ float red[4];
  __shared__ float sc[2];
  __shared__ __attribute__((aligned(16))) uint8_t tile[64 * 128];   // transposed path
  const int tid = threadIdx.x;
  int w = blockIdx.x;
  const int blk = w % a.nblk;
  w /= a.nblk;
  const int h = w % a.H, b = w / a.H;
  const int r0 = blk * 64;
  const int rows = min(64, a.N - r0);
  const int cpr = a.d / CH;                           // chunks per row
  const T* x = (const T*)a.x + b * a.x_sb + h * a.x_sh + (int64_t)r0 * a.x_sn;

  typedef T TV __attribute__((ext_vector_type(CH)));
  TV v[MAXC];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + i * 256;
    if (c < rows * cpr) {
      const int r = c / cpr, ch = c - r * cpr;
      v[i] = *(const TV*)(x + r * a.x_sn + ch * CH);
#pragma unroll
      for (int e = 0; e < CH; ++e) amax = fmaxf(amax, fabsf((float)v[i][e]));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  if (tid == 0) {
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    sc[0] = m > 0.f ? m / 448.0f : 1.0f;
    sc[1] = m > 0.f ? 448.0f / m : 1.0f;
    a.scale[((int64_t)b * a.H + h) * a.nblk + blk] = sc[0];
  }
  __syncthreads();
  const float inv = sc[1];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = tid + i * 256;
    if (c < rows * cpr) {
      const int r = c / cpr, ch = c - r * cpr;
      int wds[CH / 4];
#pragma unroll
      for (int q = 0; q < CH / 4; ++q)
        wds[q] = pack_fp8x4((float)v[i][4 * q] * inv, (float)v[i][4 * q + 1] * inv,
                            (float)v[i][4 * q + 2] * inv, (float)v[i][4 * q + 3] * inv);
      uint8_t* dst = a.transpose ? tile + r * a.d + ch * CH
                                 : (uint8_t*)a.out + b * a.o_sb + h * a.o_sh +
                                       (int64_t)(r0 + r) * a.o_sn + ch * CH;
#pragma unroll
      for (int q = 0; q < CH / 4; ++q) ((int*)dst)[q] = wds[q];
    }
  }
  if (!a.transpose) return;
  __syncthreads();
  // column c of the block: keys r0 .. r0+63 at o + c * ld + r0
  uint8_t* o = (uint8_t*)a.out + ((int64_t)b * a.H + h) * a.d * a.o_ld + r0;
  for (int e = tid; e < a.d * 16; e += 256) {
    const int c = e >> 4, j = (e & 15) * 4;
    int wd = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (j + i < rows) wd |= (int)tile[(j + i) * a.d + c] << (8 * i);
    *(int*)(o + (int64_t)c * a.o_ld + j) = wd;
  }
}

hipError_t launch_fp8_quant(const QuantArgs& a, int in_dtype, hipStream_t st) {
  const long n = (long)a.B * a.H * a.nblk;
  if (n == 0) return hipSuccess;
  if (in_dtype == 2)
    hipLaunchKernelGGL(fp8_quant_kernel<__bf16>, dim3((unsigned)n), dim3(256), 0, st, a);
  else if (in_dtype == 1)
    hipLaunchKernelGGL(fp8_quant_kernel<_Float16>, dim3((unsigned)n), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(fp8_quant_kernel<float>, dim3((unsigned)n), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- forward
template <class E, int D, bool CAUSAL>
struct Fp8Fwd {
  static constexpr int NW = 8, ROWS = NW * 32, BC = 64;
  static constexpr int KS = D / 64;                    // K = 64 steps of QK^T
  static constexpr int DT = D / 32;                    // 32-row blocks of O^T
  static constexpr int KPS = D / 16 + 1;               // K row: D bytes + one pad slot
  static constexpr int VPS = BC / 16 + 1;              // V^T row: 64 bytes + one pad slot
  static constexpr int KP = KPS * 16, VP = VPS * 16;
  static constexpr int K_BYTES = BC * KP, V_BYTES = D * VP;
  static constexpr int K_INS = (BC * KPS + 63) / 64, V_INS = (D * VPS + 63) / 64;
  static constexpr int K_IPW = (K_INS + NW - 1) / NW, V_IPW = (V_INS + NW - 1) / NW;
  static constexpr float TH = 2.75f;                   // lazy rescale threshold (log2)
  static constexpr float PSHIFT = 6.0f;                // log2 of p's scale factor
  static_assert(TH + PSHIFT < 8.807f, "p must stay below E4M3's 448");
  using T = typename E::T;
  using V4 = typename E::V4;

  struct State {
    int lane, wave, hl, l32;
    int b, h;
    int q_w0, kv_limit, n_act;
    float svm;                  // the head's largest V block scale
    const uint8_t* kp;          // K of this (batch, kv-head), key 0
    const uint8_t* vp;          // V^T of this (batch, kv-head), column 0
    const float* ksc;           // K / V block scales of this (batch, kv-head)
    const float* vsc;
    int64_t k_tile, k_end;
    uint32_t koff[K_IPW], voff[V_IPW];
    int kbase, vbase;
    float cq;                   // scale * log2(e) * sq
    float lsv_max;              // log2 of the head's largest V block scale
    i32x8 qf[KS];
    f32x16 acc[DT];
    float m_run;
    float l_run;                // fp32 sum of p (this lane half's keys): the LSE
    float l_rnd;                // sum of the E4M3-rounded p (whole row): O's divisor
    i32x8 one;                  // E4M3 1.0 in every byte (A of the row-sum MFMA)
  };

  static __device__ __forceinline__ void issue(const Fp8Args& a, const State& st, int j,
                                               char* kb, char* vb) {
    const int64_t ko = (int64_t)j * st.k_tile;
    const BufRsrc rk = make_rsrc(st.kp + ko, (uint32_t)min(st.k_end - ko, (int64_t)kBufLimit));
    const BufRsrc rv = make_rsrc(st.vp + (int64_t)j * BC, (uint32_t)kBufLimit);
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

  static __device__ __forceinline__ i32x8 ones() {
    const int c = 0x38383838;   // E4M3 1.0 in every byte
    return i32x8{c, c, c, c, c, c, c, c};
  }
  static __device__ __forceinline__ i32x8 read32(const char* p) {
    const i32x4 lo = lds_read16<i32x4>(p), hi = lds_read16<i32x4>(p + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }

  // sk, sv: the tile's K and V block scales
  static __device__ __forceinline__ void tile(const Fp8Args& a, State& st, const char* kb,
                                              const char* vb, int j, float sk, float sv) {
    const int j0 = j * BC;
    // every LDS fragment of the tile first (K for S^T, V^T for PV), so the
    // reads overlap each other and the first products
    i32x8 kf[2 * KS], vf[DT];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[blk * KS + ks] = read32(kb + st.kbase + blk * 16 * KP + ks * 64);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[dt] = read32(vb + st.vbase + dt * 32 * VP);
    __builtin_amdgcn_sched_barrier(0);
    // S^T of the tile's two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[blk] = mfma_fp8(kf[blk * KS + ks], st.qf[ks], s[blk]);
    }
    // register r of block blk: key j0 + 32 hl + 16 blk + r
    const int qrow = st.q_w0 + st.l32;
    const bool edge = (j0 + BC > st.kv_limit) || (CAUSAL && j0 + BC - 1 > st.q_w0);
    if (edge) {
      // relative limits through an empty asm: the compares stay in the branch
      int lim = st.kv_limit - j0 - 32 * st.hl;
      int dia = qrow - j0 - 32 * st.hl;
      asm volatile("" : "+v"(lim), "+v"(dia));
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * blk + r >= lim || (CAUSAL && 16 * blk + r > dia)) s[blk][r] = -INFINITY;
    }
    const float cs = st.cq * sk;
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
    mx = max_with_other_half(mx) * cs;
    if (__builtin_amdgcn_ballot_w64(mx > st.m_run + TH)) {
      const float m_new = fmaxf(st.m_run, mx);
      if (m_new > st.m_run) {
        const float alpha = (st.m_run == -INFINITY) ? 0.f : fast_exp2(st.m_run - m_new);
        st.l_run *= alpha;
        st.l_rnd *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) st.acc[dt] *= alpha;
        st.m_run = m_new;
      }
    }
    const float mref = st.m_run == -INFINITY ? 0.f : st.m_run;
    // p' = p sv / svmax 2^6 = exp2(s cs - mref + log2(sv) - log2(svmax) + 6)
    const float lr = fast_log2(sv) - st.lsv_max + PSHIFT;
    const float off = lr - mref;
    i32x8 pf;
    float psum;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int blk = w >> 2, r = (w & 3) * 4;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(__builtin_fmaf(s[blk][r + i], cs, off));
        psum = (w == 0 && i == 0) ? p[0] : psum + p[i];
      }
      // the high half of the first conversion's old value is overwritten by
      // the second: any register will do (no zeroing move)
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __builtin_bit_cast(int, p[0]), false);
      pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
    }
    // both sums in units of p (over 2^lr); the rounded one from an MFMA
    // with all-ones codes as A, which puts the column sums of P^T in every row
    const f32x16 ls = mfma_fp8(st.one, pf, f32x16{});
    const float rl = fast_exp2(-lr);
    st.l_run = __builtin_fmaf(psum, rl, st.l_run);
    st.l_rnd = __builtin_fmaf(ls[0], rl, st.l_rnd);
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      st.acc[dt] = mfma_fp8(vf[dt], pf, st.acc[dt]);
  }

  // sc: the block scales (K, V) of tile j, loaded one iteration ahead;
  // replaced by those of tile j+1 (their loads are issued before the barrier
  // and land while tile j is computed)
  static __device__ __forceinline__ void step(const Fp8Args& a, State& st, int j, int n,
                                              const char* kc, const char* vc, char* kn,
                                              char* vn, float2& sc) {
    const int jn = min(j + 1, n - 1);
    const float2 nx = {st.ksc[jn], st.vsc[jn]};
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < n) issue(a, st, j + 1, kn, vn);
    if (j < st.n_act) tile(a, st, kc, vc, j, sc.x, sc.y);
    sc = nx;
  }

  // Everything before the key loop; n_tiles: key tiles of this work-group.
  static __device__ __forceinline__ void setup(const Fp8Args& a, State& st, int& n_tiles) {
    st.lane = threadIdx.x & 63;
    st.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    st.hl = st.lane >> 5;
    st.l32 = st.lane & 31;

    int qblk, bh;
    block_coords(CAUSAL, blockIdx.x, a.B * a.Hq, a.nqb, qblk, bh);
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int g = h / a.group;
    st.b = b;
    st.h = h;
    const int q_blk0 = qblk * ROWS;
    st.q_w0 = q_blk0 + st.wave * 32;

    st.kv_limit = a.Nk;
    if (a.kv_lens) st.kv_limit = min(max(a.kv_lens[b], 0), a.Nk);
    int kv_end = st.kv_limit;
    if (CAUSAL) kv_end = min(kv_end, min(q_blk0 + ROWS, a.Nq));
    n_tiles = (kv_end + BC - 1) / BC;
    st.n_act = CAUSAL ? min(n_tiles, (st.q_w0 + 31) / BC + 1) : n_tiles;

    st.kp = a.k + b * a.k_sb + g * a.k_sh;
    st.vp = a.vt + ((int64_t)b * a.Hkv + g) * a.d * a.vt_ld;
    st.ksc = a.k_scale + ((int64_t)b * a.Hkv + g) * a.nks;
    st.vsc = a.v_scale + ((int64_t)b * a.Hkv + g) * a.nks;
    st.k_tile = (int64_t)BC * a.k_sn;
    st.k_end = (int64_t)(a.Nk - 1) * a.k_sn + a.d;
    const int dch = a.d / 16;
    // K tile: slot s = row s / KPS, chunk s % KPS (pad slot and chunks past d
    // load zero); V^T tile: row (d index) s / VPS, chunk s % VPS of 64 keys
#pragma unroll
    for (int i = 0; i < K_IPW; ++i) {
      const int s = (i * NW + st.wave) * 64 + st.lane;
      const int r = s / KPS, ch = s % KPS;
      st.koff[i] = (r < BC && ch < dch) ? (uint32_t)(r * a.k_sn + ch * 16) : kBufOutOfRange;
    }
#pragma unroll
    for (int i = 0; i < V_IPW; ++i) {
      const int s = (i * NW + st.wave) * 64 + st.lane;
      const int r = s / VPS, ch = s % VPS;
      st.voff[i] = (r < a.d && ch < BC / 16) ? (uint32_t)(r * a.vt_ld + ch * 16) : kBufOutOfRange;
    }
    {
      // K row of S^T row l32 in 32-key block 0 (block 1 adds 16 rows)
      const int i = st.l32;
      const int key = 32 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
      st.kbase = key * KP + st.hl * 32;
      st.vbase = st.l32 * VP + st.hl * 32;
    }

    // Q^T operand: 32 bytes of row q_w0 + l32 per K = 64 step (zero past d)
    const int crow = min(st.q_w0 + st.l32, a.Nq - 1);
    const uint8_t* qp = a.q + b * a.q_sb + h * a.q_sh + (int64_t)crow * a.q_sn;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 64 + st.hl * 32;
      const i32x4 lo = d0 < a.d ? *(const i32x4*)(qp + d0) : i32x4{};
      const i32x4 hi = d0 + 16 < a.d ? *(const i32x4*)(qp + d0 + 16) : i32x4{};
      st.qf[ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    const float sq = a.q_scale[((int64_t)b * a.Hq + h) * a.nqs + min(st.q_w0, a.Nq - 1) / 64];
    st.cq = a.c * sq;
    // the head's largest V block scale over the tiles this block reads
    float svm = 0.f;
    for (int t = st.lane; t < n_tiles; t += 64) svm = fmaxf(svm, st.vsc[t]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) svm = fmaxf(svm, __shfl_xor(svm, o, 64));
    st.svm = svm;
    st.lsv_max = svm > 0.f ? fast_log2(svm) : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc[dt] = f32x16{};
    st.m_run = -INFINITY;
    // kept in registers for the whole loop (not rematerialised every tile)
    st.one = ones();
    asm volatile("" : "+v"(st.one));
    st.l_run = 0.f;
    st.l_rnd = 0.f;
  }

  static __device__ __forceinline__ void run(const Fp8Args& a, char* k0, char* v0, char* k1,
                                             char* v1) {
    State st;
    int n_tiles;
    setup(a, st, n_tiles);
    float2 sc = {1.f, 1.f};
    if (n_tiles > 0) {
      issue(a, st, 0, k0, v0);
      sc = float2{st.ksc[0], st.vsc[0]};
    }
    for (int j = 0; j < n_tiles; j += 2) {
      step(a, st, j, n_tiles, k0, v0, k1, v1, sc);
      if (j + 1 >= n_tiles) break;
      step(a, st, j + 1, n_tiles, k1, v1, k0, v0, sc);
    }
    epilogue(a, st);
  }

  // O = acc svmax 2^-6 / l_rnd (the row-sum MFMA already covers both lane
  // halves), LSE = ln2 (m + log2 l) with the fp32 sum l of both halves.
  static __device__ __forceinline__ void epilogue(const Fp8Args& a, const State& st) {
    T* op = (T*)a.o + st.b * a.o_sb + st.h * a.o_sh;
    const float l_tot = add_with_other_half(st.l_run);
    const float inv = st.l_rnd > 0.f ? st.svm * 0.015625f / st.l_rnd : 0.f;
    const int row = st.q_w0 + st.l32;
    if (row < a.Nq) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int col = dt * 32 + gq * 8 + st.hl * 4;
          if (col < a.d) {
            auto lo = E::cvt2(st.acc[dt][gq * 4 + 0] * inv, st.acc[dt][gq * 4 + 1] * inv);
            auto hi = E::cvt2(st.acc[dt][gq * 4 + 2] * inv, st.acc[dt][gq * 4 + 3] * inv);
            *(V4*)(op + row * a.o_sn + col) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
          }
        }
      if (st.hl == 0)
        a.lse[((int64_t)st.b * a.Hq + st.h) * a.Nq + row] =
            l_tot > 0.f ? (st.m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
  }
};

template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_fp8_kernel(Fp8Args a) {
  using K = Fp8Fwd<E, D, CAUSAL>;
  __shared__ __attribute__((aligned(1024))) char k0[K::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0[K::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1[K::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1[K::V_BYTES];
  K::run(a, k0, v0, k1, v1);
}

template <class E, int D>
static hipError_t launch_fp8_d(const Fp8Args& a0, bool causal, hipStream_t st) {
  Fp8Args a = a0;
  a.nqb = (a.Nq + 255) / 256;
  a.total_blocks = a.B * a.Hq * a.nqb;
  if (a.total_blocks == 0) return hipSuccess;
  if (causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<E, D, true>), dim3(a.total_blocks), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<E, D, false>), dim3(a.total_blocks), dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8Args& a, bool out_bf16, bool causal, hipStream_t st) {
  if (a.d > 64)
    return out_bf16 ? launch_fp8_d<BF16, 128>(a, causal, st) : launch_fp8_d<FP16, 128>(a, causal, st);
  return out_bf16 ? launch_fp8_d<BF16, 64>(a, causal, st) : launch_fp8_d<FP16, 64>(a, causal, st);
}

}  // namespace attn
