// Paged decode attention for gfx950, balanced schedule: dispatch and planning.  The
// kernel is decode_sk_kernel.h; its instantiations are compiled per cache dtype in
// decode_sk_<dtype>.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "decode_sk_kernel.h"

namespace pkv {

// ---- dispatch --------------------------------------------------------------------
PKV_SK_FOR_DTYPES(PKV_SK_EXTERN, kBF16, kBF16)
PKV_SK_FOR_DTYPES(PKV_SK_EXTERN, kF16, kF16)
PKV_SK_FOR_DTYPES(PKV_SK_EXTERN, kF32, kF32)
PKV_SK_FOR_DTYPES(PKV_SK_EXTERN, kFP8, kBF16)
PKV_SK_FOR_DTYPES(PKV_SK_EXTERN, kFP8, kF16)
PKV_SK_FOR_DTYPES(PKV_SK_EXTERN_PRE, kBF16, kBF16)
PKV_SK_FOR_DTYPES(PKV_SK_EXTERN_PRE, kF16, kF16)
PKV_SK_FOR_DTYPES(PKV_SK_EXTERN_PRE, kFP8, kBF16)
PKV_SK_FOR_DTYPES(PKV_SK_EXTERN_PRE, kFP8, kF16)

// Resolve (cache dtype, q dtype, head dim, padded group, load policy, suffix pass of
// the shared-prefix decode) to the kernel and run f.
template <typename F>
static hipError_t with_sk(int kv, int q, int d, int gp, bool nt, bool pre, F&& f) {
  if (pre) {  // 16-bit and fp8 caches, streaming loads
#define PKV_SK_PRE_GP(KV, Q, D)                                       \
  switch (gp) {                                                       \
    case 1: return f(SkKernels<KV, Q, D, 1, true, true>());           \
    case 2: return f(SkKernels<KV, Q, D, 2, true, true>());           \
    case 4: return f(SkKernels<KV, Q, D, 4, true, true>());           \
    case 8: return f(SkKernels<KV, Q, D, 8, true, true>());           \
    case 16: return f(SkKernels<KV, Q, D, 16, true, true>());         \
    default: return hipErrorInvalidValue;                             \
  }
#define PKV_SK_PRE_D(KV, Q)                                            \
  if (d == 64) { PKV_SK_PRE_GP(KV, Q, 64) }                            \
  if (d == 128) { PKV_SK_PRE_GP(KV, Q, 128) }                          \
  return hipErrorInvalidValue;
    if (!nt) return hipErrorInvalidValue;
    if (kv == kBF16 && q == kBF16) { PKV_SK_PRE_D(kBF16, kBF16) }
    if (kv == kF16 && q == kF16) { PKV_SK_PRE_D(kF16, kF16) }
    if (kv == kFP8 && q == kBF16) { PKV_SK_PRE_D(kFP8, kBF16) }
    if (kv == kFP8 && q == kF16) { PKV_SK_PRE_D(kFP8, kF16) }
#undef PKV_SK_PRE_D
#undef PKV_SK_PRE_GP
    return hipErrorInvalidValue;
  }
#define PKV_SK_NT(KV, Q, D, GP)                                      \
  return nt ? f(SkKernels<KV, Q, D, GP, true>()) : f(SkKernels<KV, Q, D, GP, false>());
#define PKV_SK_GP(KV, Q, D)                                   \
  switch (gp) {                                               \
    case 1: PKV_SK_NT(KV, Q, D, 1)                            \
    case 2: PKV_SK_NT(KV, Q, D, 2)                            \
    case 4: PKV_SK_NT(KV, Q, D, 4)                            \
    case 8: PKV_SK_NT(KV, Q, D, 8)                            \
    case 16: PKV_SK_NT(KV, Q, D, 16)                          \
    default: return hipErrorInvalidValue;                     \
  }
#define PKV_SK_D(KV, Q)                                       \
  if (d == 64) { PKV_SK_GP(KV, Q, 64) }                       \
  if (d == 128) { PKV_SK_GP(KV, Q, 128) }                     \
  return hipErrorInvalidValue;
  if (kv == kBF16 && q == kBF16) { PKV_SK_D(kBF16, kBF16) }
  if (kv == kF16 && q == kF16) { PKV_SK_D(kF16, kF16) }
  if (kv == kF32 && q == kF32) { PKV_SK_D(kF32, kF32) }
  if (kv == kFP8 && q == kBF16) { PKV_SK_D(kFP8, kBF16) }
  if (kv == kFP8 && q == kF16) { PKV_SK_D(kFP8, kF16) }
#undef PKV_SK_D
#undef PKV_SK_GP
#undef PKV_SK_NT
  return hipErrorInvalidValue;
}

int pad_group(int G) {
  int gp = 1;
  while (gp < G) gp <<= 1;
  return gp;
}

// Occupancy of each balanced-kernel instantiation, cached per device: the query is a
// pure function of (device, kernel, LDS bytes) and costs microseconds of host time per
// call otherwise.  Entries are filled once, racing writers store the same value.
namespace {
constexpr int kMaxDevices = 64;
constexpr int kCacheSlots = 5 * 5 * 2 * 5 * 2 * 2;  // cache x q dtype x head dim x group x policy x pre
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_per_cu[kMaxDevices][kCacheSlots];
int gp_index(int gp) { return gp == 1 ? 0 : gp == 2 ? 1 : gp == 4 ? 2 : gp == 8 ? 3 : 4; }
}  // namespace

int streamk_plan(int cache_dtype, int q_dtype, int head_dim, int group, int num_seqs, bool kv_stream,
                 bool pre, SkPlan* out) {
  const int gp = pad_group(group);
  const size_t lds = (size_t)(num_seqs + 1) * sizeof(int);
  hipError_t e = with_sk(cache_dtype, q_dtype, head_dim, gp, kv_stream, pre, [&](auto k) {
    using K = decltype(k);
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
      (void)hipGetLastError();
      cus = 256;  // no device visible (host-only use): size for a full MI355X
      per_cu = 1;
    } else {
      const bool cacheable = dev < kMaxDevices && cache_dtype >= 0 && cache_dtype < 5 && q_dtype >= 0 &&
                             q_dtype < 5 && lds <= 4096;  // small LDS requests share one entry
      const int slot =
          ((((cache_dtype * 5 + q_dtype) * 2 + (head_dim == 128)) * 5 + gp_index(gp)) * 2 + kv_stream) * 2 + pre;
      if (cacheable) {
        cus = g_cus[dev].load(std::memory_order_relaxed);
        per_cu = g_per_cu[dev][slot].load(std::memory_order_relaxed);
      }
      if (cus <= 0 || per_cu <= 0) {
        const size_t lds_q = cacheable ? 4096 : lds;  // a cached entry must hold for any small N
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K::decode(), 64 * K::NW, lds_q) != hipSuccess) {
          (void)hipGetLastError();
          cus = 256;
          per_cu = 1;
        } else if (cacheable && cus > 0 && per_cu > 0) {
          g_cus[dev].store(cus, std::memory_order_relaxed);
          g_per_cu[dev][slot].store(per_cu, std::memory_order_relaxed);
        }
      }
    }
    if (cus <= 0 || per_cu <= 0) return hipErrorInvalidValue;  // does not fit a CU
    const int wgs = cus * per_cu < kStreamKMaxGroups ? cus * per_cu : kStreamKMaxGroups;
    out->waves = wgs * K::NW;
    out->ws_bytes = kWsHeaderBytes + align256((size_t)2 * wgs * K::STRIDE * sizeof(float));
    return hipSuccess;
  });
  return e == hipSuccess ? 0 : -1;
}

hipError_t launch_decode_streamk(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  return with_sk(a.cache_dtype, a.q_dtype, a.head_dim, pad_group(G), a.kv_stream != 0, a.pre_part != nullptr,
                 [&](auto k) { return k.launch(a, stream); });
}

}  // namespace pkv
