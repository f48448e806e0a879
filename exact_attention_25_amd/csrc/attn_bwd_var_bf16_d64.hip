// Local / soft-capped backward instances for bf16 inputs, head dimension <= 64
// (see attn_bwd_variants.h).
#include "attn_bwd_variants.h"

namespace attn {

template void launch_bwd_variant<BF16, 64>(const BwdArgs&, FwdMode, hipStream_t);

}  // namespace attn
