// Launch of the backward's dQ and dK/dV kernels for one compile-time variant,
// and the dispatch of the local / soft-capped variants, whose instances are
// compiled in the attn_bwd_var_*.hip files (one per element type and head
// dimension, so that they build in parallel).
#pragma once

#include "attn_bwd_kernel.h"

namespace attn {

template <class E, int D, bool CAUSAL, bool MASK, bool LOCAL, bool SOFTCAP>
void launch_bwd_qkv(const BwdArgs& a, hipStream_t st) {
  constexpr int NW_KV = kBwdKeysPerBlock / 32, BR = 128;
  constexpr int NW_Q = 4, BC = 128;
  // dQ, and D / nl2 per row for the dK/dV pass
  if (a.Nq > 0) {
    const int nqb = (a.Nq + NW_Q * 32 - 1) / (NW_Q * 32);
    hipLaunchKernelGGL((bwd_q_kernel<E, D, NW_Q, BC, CAUSAL, MASK, LOCAL, SOFTCAP>),
                       dim3((unsigned)(a.B * a.Hq * nqb)), dim3(NW_Q * 64), 0, st, a);
  }
  // dK / dV (after dQ: it reads D and nl2)
  if (a.Nk > 0) {
    const int nkb = (a.Nk + kBwdKeysPerBlock - 1) / kBwdKeysPerBlock;
    hipLaunchKernelGGL((bwd_kv_kernel<E, D, NW_KV, BR, CAUSAL, MASK, LOCAL, SOFTCAP>),
                       dim3((unsigned)(a.B * a.Hkv * a.kv_chunks * nkb)), dim3(NW_KV * 64), 0, st,
                       a);
  }
}

// Local and/or soft-capped calls.  Under LOCAL causal masking is part of
// a.loc; without it only the soft cap differs from the plain kernels.
template <class E, int D>
void launch_bwd_variant(const BwdArgs& a, FwdMode m, hipStream_t st) {
  if (m.local) {
    if (m.mask) {
      if (m.softcap) launch_bwd_qkv<E, D, false, true, true, true>(a, st);
      else launch_bwd_qkv<E, D, false, true, true, false>(a, st);
    } else {
      if (m.softcap) launch_bwd_qkv<E, D, false, false, true, true>(a, st);
      else launch_bwd_qkv<E, D, false, false, true, false>(a, st);
    }
  } else if (m.causal) {
    if (m.mask) launch_bwd_qkv<E, D, true, true, false, true>(a, st);
    else launch_bwd_qkv<E, D, true, false, false, true>(a, st);
  } else {
    if (m.mask) launch_bwd_qkv<E, D, false, true, false, true>(a, st);
    else launch_bwd_qkv<E, D, false, false, false, true>(a, st);
  }
}

extern template void launch_bwd_variant<BF16, 64>(const BwdArgs&, FwdMode, hipStream_t);
extern template void launch_bwd_variant<BF16, 128>(const BwdArgs&, FwdMode, hipStream_t);
extern template void launch_bwd_variant<FP16, 64>(const BwdArgs&, FwdMode, hipStream_t);
extern template void launch_bwd_variant<FP16, 128>(const BwdArgs&, FwdMode, hipStream_t);

}  // namespace attn
