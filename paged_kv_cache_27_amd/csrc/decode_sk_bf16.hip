// Instantiations of the balanced decode kernel for bf16 caches.
#define PKV_SK_DEFINE
#include "decode_sk_kernel.h"

namespace pkv {

PKV_SK_FOR_DTYPES(PKV_SK_INSTANTIATE, kBF16, kBF16)

}  // namespace pkv
