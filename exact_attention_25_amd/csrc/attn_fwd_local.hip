// Forward attention with local masks (sliding window, 2-D neighbourhood) or
// the tanh soft cap: FwdKernel (attn_fwd_kernel.h) instances with LOCAL and
// SOFTCAP, 8 waves x 32 rows per work-group and 64-key tiles.  Under LOCAL
// the causal rule is part of the window (a.loc.win_r <= 0), so CAUSAL is
// only instantiated for soft-capped calls without a window or grid.
#include "attn_fwd_kernel.h"

namespace attn {

template <class E, int D, bool CAUSAL, bool MASK, bool LOCAL, bool SOFTCAP>
static hipError_t go(const FwdArgs& a0, hipStream_t st) {
  constexpr int NW = 8, BC = 64;
  using K = FwdKernel<E, D, NW, BC, CAUSAL, MASK, LOCAL, SOFTCAP>;
  FwdArgs a = a0;
  a.nqb = (a.Nq + K::ROWS - 1) / K::ROWS;
  a.total_blocks = a.B * a.Hq * a.nqb;
  hipLaunchKernelGGL((fwd_kernel<E, D, NW, BC, CAUSAL, MASK, LOCAL, SOFTCAP>),
                     dim3(a.total_blocks), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <class E, int D, bool MASK>
static hipError_t pick(const FwdArgs& a, FwdMode m, hipStream_t st) {
  if (m.local) {
    return m.softcap ? go<E, D, false, MASK, true, true>(a, st)
                     : go<E, D, false, MASK, true, false>(a, st);
  }
  // soft cap only
  return m.causal ? go<E, D, true, MASK, false, true>(a, st)
                  : go<E, D, false, MASK, false, true>(a, st);
}

template <class E>
static hipError_t pick_e(const FwdArgs& a, FwdMode m, hipStream_t st) {
  if (a.d > 64) return m.mask ? pick<E, 128, true>(a, m, st) : pick<E, 128, false>(a, m, st);
  return m.mask ? pick<E, 64, true>(a, m, st) : pick<E, 64, false>(a, m, st);
}

hipError_t launch_fwd16_local(const FwdArgs& a, bool is_bf16, FwdMode m, hipStream_t st) {
  return is_bf16 ? pick_e<BF16>(a, m, st) : pick_e<FP16>(a, m, st);
}

}  // namespace attn
