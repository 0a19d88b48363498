// Instantiations of the balanced decode kernel as the suffix pass of the shared-prefix
// decode (16-bit caches, streaming loads).
#define PKV_SK_DEFINE
#include "decode_sk_kernel.h"

namespace pkv {

PKV_SK_FOR_DTYPES(PKV_SK_INSTANTIATE_PRE, kBF16, kBF16)
PKV_SK_FOR_DTYPES(PKV_SK_INSTANTIATE_PRE, kF16, kF16)

}  // namespace pkv
