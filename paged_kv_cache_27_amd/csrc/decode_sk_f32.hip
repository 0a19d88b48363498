// Instantiations of the balanced decode kernel for f32 caches.
#define PKV_SK_DEFINE
#include "decode_sk_kernel.h"

namespace pkv {

PKV_SK_FOR_DTYPES(PKV_SK_INSTANTIATE, kF32, kF32)

}  // namespace pkv
