// Instantiations of the balanced decode kernel for fp8 caches with bf16 queries.
#define PKV_SK_DEFINE
#include "decode_sk_kernel.h"

namespace pkv {

PKV_SK_FOR_DTYPES(PKV_SK_INSTANTIATE, kFP8, kBF16)

}  // namespace pkv
