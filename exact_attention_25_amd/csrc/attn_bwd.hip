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

// bf16 -> fp16 copies of q, dout (n16q elements each) and k (n16k), 8
// elements per 16-byte access (the element counts are multiples of 8).
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a, int64_t n8q, int64_t n8k) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < 2 * n8q + n8k; i += stride) {
    const bf16x8* src;
    f16x8* dst;
    int64_t j = i;
    if (j < n8q) {
      src = (const bf16x8*)a.q; dst = (f16x8*)a.q16;
    } else if ((j -= n8q) < n8q) {
      src = (const bf16x8*)a.dout; dst = (f16x8*)a.do16;
    } else {
      j -= n8q;
      src = (const bf16x8*)a.k; dst = (f16x8*)a.k16;
    }
    dst[j] = to_f16x8<BF16>(src[j]);
  }
}

template <class E, int D>
static hipError_t launch_bwd_t(const BwdArgs& a, FwdMode m, hipStream_t st) {
  if (std::is_same<E, BF16>::value) {
    const int64_t n8q = (int64_t)a.B * a.Hq * a.Nq * a.d / 8;
    const int64_t n8k = (int64_t)a.B * a.Hkv * a.Nk * a.d / 8;
    const int64_t n = 2 * n8q + n8k;
    if (n > 0) {
      const int blocks = (int)((n + 255) / 256 < 16384 ? (n + 255) / 256 : 16384);
      hipLaunchKernelGGL(bwd_prep_kernel, dim3(blocks), dim3(256), 0, st, a, n8q, n8k);
    }
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
