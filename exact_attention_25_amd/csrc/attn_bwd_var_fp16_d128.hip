// Local / soft-capped backward instances for fp16 inputs, head dimension <= 128
// (see attn_bwd_variants.h).
#include "attn_bwd_variants.h"

namespace attn {

template void launch_bwd_variant<FP16, 128>(const BwdArgs&, FwdMode, hipStream_t);

}  // namespace attn
