// Instantiations of the balanced decode kernel's suffix pass of the shared-prefix decode
// (PRE) for fp8 caches, with bf16 or f16 queries.
#define PKV_SK_DEFINE
#include "decode_sk_kernel.h"

namespace pkv {

PKV_SK_FOR_DTYPES(PKV_SK_INSTANTIATE_PRE, kFP8, kBF16)
PKV_SK_FOR_DTYPES(PKV_SK_INSTANTIATE_PRE, kFP8, kF16)

}  // namespace pkv
