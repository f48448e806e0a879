// Backward attention: kernel instances, work split and dispatch (the kernels
// are in attn_bwd_kernel.h; the local and soft-capped instances are built in
// the attn_bwd_var_*.hip files).
#include <type_traits>

#include "attn_bwd_variants.h"

namespace attn {

// q-head chunks per kv-head for the dK/dV pass: the smallest divisor of the
// group size that gives enough work-groups to fill the chip (every chunk
// adds one partial dK/dV tensor to the workspace and to the final sum).
int bwd_kv_chunks(int B, int Hkv, int Nk, int group) {
  const long nkb = (Nk + kBwdKeysPerBlock - 1) / kBwdKeysPerBlock;
  const long base = (long)B * Hkv * nkb;
  for (int c = 1; c < group; ++c)
    if (group % c == 0 && base * c >= 2048) return c;
  return group;
}

// Largest magnitude of 8 bf16 values (NaN ignored).
__device__ __forceinline__ float amax8(bf16x8 x) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf((float)x[i]));
  return m;
}

// Maxima of 4 values over a 256-thread work-group; thread 0 gets them.
__device__ __forceinline__ void block_max4(float (&m)[4], float* red) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m[t] = fmaxf(m[t], __shfl_xor(m[t], o));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int t = 0; t < 4; ++t) red[w * 4 + t] = m[t];
  __syncthreads();
  if (threadIdx.x == 0)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      m[t] = fmaxf(fmaxf(red[t], red[4 + t]), fmaxf(red[8 + t], red[12 + t]));
}

// bf16 -> fp16 copies of q, dout (n8q 8-element chunks each) and k (n8k),
// 16 bytes per access, and the largest magnitudes of q, k, v and dout over
// this work-group's share (v is read for its maximum only).
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a, int64_t n8q, int64_t n8k) {
  __shared__ float red[16];
  float m[4] = {0.f, 0.f, 0.f, 0.f};   // q, k, v, dout
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < 2 * n8q + 2 * n8k; i += stride) {
    int64_t j = i;
    if (j < n8q) {
      const bf16x8 x = ((const bf16x8*)a.q)[j];
      m[0] = fmaxf(m[0], amax8(x));
      ((f16x8*)a.q16)[j] = to_f16x8<BF16>(x);
    } else if ((j -= n8q) < n8q) {
      const bf16x8 x = ((const bf16x8*)a.dout)[j];
      m[3] = fmaxf(m[3], amax8(x));
      ((f16x8*)a.do16)[j] = to_f16x8<BF16>(x);
    } else if ((j -= n8q) < n8k) {
      const bf16x8 x = ((const bf16x8*)a.k)[j];
      m[1] = fmaxf(m[1], amax8(x));
      ((f16x8*)a.k16)[j] = to_f16x8<BF16>(x);
    } else {
      j -= n8k;
      m[2] = fmaxf(m[2], amax8(((const bf16x8*)a.v)[j]));
    }
  }
  block_max4(m, red);
  if (threadIdx.x == 0)
#pragma unroll
    for (int t = 0; t < 4; ++t) a.amax_part[blockIdx.x * 4 + t] = m[t];
}

// The operand scales (BwdScales) from the pre-pass maxima; one work-group.
__global__ __launch_bounds__(256) void bwd_scale_kernel(BwdArgs a) {
  __shared__ float red[16];
  float m[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = threadIdx.x; i < a.amax_blocks; i += 256)
#pragma unroll
    for (int t = 0; t < 4; ++t) m[t] = fmaxf(m[t], a.amax_part[i * 4 + t]);
  block_max4(m, red);
  if (threadIdx.x == 0) {
    a.escale[0] = pow2_scale(m[0], kQkLo, kQkHi, kQkTarget);
    a.escale[1] = pow2_scale(m[1], kQkLo, kQkHi, kQkTarget);
    a.escale[2] = pow2_scale(m[2], kDvLo, kDvHi, kDvTarget);
    a.escale[3] = pow2_scale(m[3], kDvLo, kDvHi, kDvTarget);
  }
}

// Rewrites the fp16 copies with their scales when some scale is not 1 (the
// work-groups return at once otherwise).
__global__ __launch_bounds__(256) void bwd_rescale_kernel(BwdArgs a, int64_t n8q, int64_t n8k) {
  const float sq = a.escale[0], sk = a.escale[1], sd = a.escale[3];
  if (sq == 1.f && sk == 1.f && sd == 1.f) return;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < 2 * n8q + n8k; i += stride) {
    int64_t j = i;
    if (j < n8q) {
      ((f16x8*)a.q16)[j] = to_f16x8_scaled<BF16>(((const bf16x8*)a.q)[j], sq);
    } else if ((j -= n8q) < n8q) {
      ((f16x8*)a.do16)[j] = to_f16x8_scaled<BF16>(((const bf16x8*)a.dout)[j], sd);
    } else {
      j -= n8q;
      ((f16x8*)a.k16)[j] = to_f16x8_scaled<BF16>(((const bf16x8*)a.k)[j], sk);
    }
  }
}

template <class E, int D>
static hipError_t launch_bwd_t(const BwdArgs& args, FwdMode m, hipStream_t st) {
  BwdArgs a = args;
  if (std::is_same<E, BF16>::value) {
    // fp16 copies and maxima, then the scales, then (if some scale is not
    // 1) the copies again, scaled
    const int64_t n8q = (int64_t)a.B * a.Hq * a.Nq * a.d / 8;
    const int64_t n8k = (int64_t)a.B * a.Hkv * a.Nk * a.d / 8;
    const int64_t n = 2 * n8q + 2 * n8k;
    const int64_t nb = (n + 255) / 256;
    a.amax_blocks = (int)(nb < kBwdAmaxBlocks ? (nb > 0 ? nb : 1) : kBwdAmaxBlocks);
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(a.amax_blocks), dim3(256), 0, st, a, n8q, n8k);
    hipLaunchKernelGGL(bwd_scale_kernel, dim3(1), dim3(256), 0, st, a);
    hipLaunchKernelGGL(bwd_rescale_kernel, dim3(a.amax_blocks), dim3(256), 0, st, a, n8q, n8k);
  } else {
    a.escale = nullptr;
  }
  if (m.local || m.softcap) {
    launch_bwd_variant<E, D>(a, m, st);
  } else if (m.mask) {
    if (m.causal) launch_bwd_qkv<E, D, true, true, false, false>(a, st);
    else launch_bwd_qkv<E, D, false, true, false, false>(a, st);
  } else {
    if (m.causal) launch_bwd_qkv<E, D, true, false, false, false>(a, st);
    else launch_bwd_qkv<E, D, false, false, false, false>(a, st);
  }
  if (a.Nk > 0 && a.kv_chunks > 1) {
    const int64_t n = (int64_t)a.B * a.Hkv * a.Nk * a.d;
    const int blocks = (int)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
    hipLaunchKernelGGL((bwd_kv_reduce_kernel<typename E::T>), dim3(blocks), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <class E>
static hipError_t launch_bwd_e(const BwdArgs& a, FwdMode m, hipStream_t st) {
  if (a.d > 64) return launch_bwd_t<E, 128>(a, m, st);
  return launch_bwd_t<E, 64>(a, m, st);
}

hipError_t launch_bwd16(const BwdArgs& a, bool is_bf16, FwdMode m, hipStream_t st) {
  return is_bf16 ? launch_bwd_e<BF16>(a, m, st) : launch_bwd_e<FP16>(a, m, st);
}

}  // namespace attn
