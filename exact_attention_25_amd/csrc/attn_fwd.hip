// Forward attention: kernel instances and dispatch.  Calls without an
// additive mask whose work-groups see at least 8 key tiles (causal: min(Nq,
// Nk) >= 8 tiles) take the software-pipelined kernel
// (attn_fwd_pipe_kernel.h); the others take FwdKernel
// (attn_fwd_kernel.h).  Both compute the same values.  Local and
// soft-capped calls go to attn_fwd_local.hip.
#include "attn_fwd_kernel.h"
#include "attn_fwd_pipe_kernel.h"

namespace attn {

template <class E, int D, int NW, int BC>
static hipError_t launch_fwd_t(const FwdArgs& a0, bool causal, bool mask, hipStream_t st) {
  // The pipelined kernel computes one tile more than it uses and has a longer
  // prologue, which short key ranges do not amortise.
  if (!mask && (causal ? min(a0.Nq, a0.Nk) : a0.Nk) >= 8 * BC) {
    using P = FwdPipeKernel<E, D, BC, false>;
    FwdArgs a = a0;
    a.nqb = (a.Nq + P::ROWS - 1) / P::ROWS;
    a.total_blocks = a.B * a.Hq * a.nqb;
    if (causal)
      hipLaunchKernelGGL((fwd_pipe_kernel<E, D, BC, true>), dim3(a.total_blocks), dim3(P::NW * 64),
                         0, st, a);
    else
      hipLaunchKernelGGL((fwd_pipe_kernel<E, D, BC, false>), dim3(a.total_blocks), dim3(P::NW * 64),
                         0, st, a);
    return hipGetLastError();
  }
  using K = FwdKernel<E, D, NW, BC, false, false>;
  FwdArgs a = a0;
  a.nqb = (a.Nq + K::ROWS - 1) / K::ROWS;
  a.total_blocks = a.B * a.Hq * a.nqb;
  dim3 grid(a.total_blocks), block(NW * 64);
  if (causal) {
    if (mask) hipLaunchKernelGGL((fwd_kernel<E, D, NW, BC, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<E, D, NW, BC, true, false>), grid, block, 0, st, a);
  } else {
    if (mask) hipLaunchKernelGGL((fwd_kernel<E, D, NW, BC, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<E, D, NW, BC, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <class E>
static hipError_t launch_fwd_e(const FwdArgs& a, bool causal, bool mask, hipStream_t st) {
  if (a.d > 64) return launch_fwd_t<E, 128, 8, 64>(a, causal, mask, st);
  return launch_fwd_t<E, 64, 8, 64>(a, causal, mask, st);
}

hipError_t launch_fwd16(const FwdArgs& a, bool is_bf16, FwdMode m, hipStream_t st) {
  if (m.local || m.softcap) return launch_fwd16_local(a, is_bf16, m, st);
  return is_bf16 ? launch_fwd_e<BF16>(a, m.causal, m.mask, st)
                 : launch_fwd_e<FP16>(a, m.causal, m.mask, st);
}

}  // namespace attn
