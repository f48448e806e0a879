// Forward attention: kernel instances and dispatch.  Calls without an
// additive mask whose work-groups see at least 8 key tiles (causal: min(Nq,
// Nk) >= 8 tiles) take the software-pipelined kernel
// (attn_fwd_pipe_kernel.h); the others take FwdKernel
// (attn_fwd_kernel.h).  Both compute the same values.  Local and
// soft-capped calls go to attn_fwd_local.hip; short key ranges at d <= 64
// (Nk <= kResidentMaxKeys, no mask) to attn_fwd_resident.hip.
#include "attn_fwd_kernel.h"
#include "attn_fwd_pipe_kernel.h"

namespace attn {

template <class E, int D, int BC, int PNW, int DK>
static hipError_t launch_pipe_dk(const FwdArgs& a0, bool causal, hipStream_t st) {
  using P = FwdPipeKernel<E, D, BC, false, PNW, DK>;
  FwdArgs a = a0;
  a.nqb = (a.Nq + P::ROWS - 1) / P::ROWS;
  a.total_blocks = a.B * a.Hq * a.nqb;
  if (causal)
    hipLaunchKernelGGL((fwd_pipe_kernel<E, D, BC, true, PNW, DK>), dim3(a.total_blocks),
                       dim3(PNW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((fwd_pipe_kernel<E, D, BC, false, PNW, DK>), dim3(a.total_blocks),
                       dim3(PNW * 64), 0, st, a);
  return hipGetLastError();
}

// d <= 48 at D = 64: the QK^T contraction stops at column 48
template <class E, int D, int BC, int PNW>
static hipError_t launch_pipe(const FwdArgs& a, bool causal, hipStream_t st) {
  if constexpr (D == 64) {
    if (a.d <= 48) return launch_pipe_dk<E, D, BC, PNW, 48>(a, causal, st);
  }
  return launch_pipe_dk<E, D, BC, PNW, D>(a, causal, st);
}

template <class E, int D, int NW, int BC>
static hipError_t launch_fwd_t(const FwdArgs& a0, bool causal, bool mask, hipStream_t st) {
  // The pipelined kernel computes one tile more than it uses and has a longer
  // prologue, which short key ranges do not amortise.
  const int span = causal ? min(a0.Nq, a0.Nk) : a0.Nk;
  if (!mask && span >= 8 * BC) {
    // up to 16 key tiles: 4-wave work-groups, two per CU (measured +3.5 % at
    // 1024 keys, -3 % at 4096)
    if (span <= 16 * BC) return launch_pipe<E, D, BC, 4>(a0, causal, st);
    // d <= 64: 128-key tiles, which halve the per-tile work outside the
    // products (row-maximum exchange, rescale test, barrier) per key; the
    // scores of two such tiles still fit in the registers (measured +10 % at
    // N = 4096, d = 40)
    if constexpr (D == 64) return launch_pipe<E, D, 2 * BC, 8>(a0, causal, st);
    else return launch_pipe<E, D, BC, 8>(a0, causal, st);
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
  if (!m.mask && a.d <= 64 && a.Nk <= kResidentMaxKeys)
    return launch_fwd16_resident(a, is_bf16, m.causal, st);
  return is_bf16 ? launch_fwd_e<BF16>(a, m.causal, m.mask, st)
                 : launch_fwd_e<FP16>(a, m.causal, m.mask, st);
}

}  // namespace attn
