// Instantiations of the balanced decode kernel for f16 caches.
#define PKV_SK_DEFINE
#include "decode_sk_kernel.h"

namespace pkv {

PKV_SK_FOR_DTYPES(PKV_SK_INSTANTIATE, kF16, kF16)

}  // namespace pkv
