// Paged decode attention for gfx950, balanced ("stream-K") schedule.
//
// The work of one decode step is the list of 16-token chunks of every (KV head,
// sequence) context, KV-head major: U = H_kv * sum_s ceil(ctx_s / 16) units.  The
// launch holds exactly as many waves W as the GPU keeps resident, and wave w takes
// the contiguous unit range [U w / W, U (w+1) / W): every wave gets the same amount
// of K/V to stream (to within one chunk), whatever the mix of context lengths, and
// the whole launch is a single round of resident waves.
//
// A wave walks its range one (sequence, KV head) segment at a time with the steps of
// decode_common.h.  A segment it covers entirely is written straight to `out`.  A
// segment shared with neighbouring waves leaves one partial (max, denominator,
// unnormalised output) per wave: a wave's first segment (if it started there
// mid-way) goes to slot 0 of the wave, its last segment (if it continues past the
// wave's range) to slot 1.  merge_sk_kernel then combines, per segment, the
// partials of the consecutive waves that covered it, with the log-sum-exp algebra
// of the online softmax; it also writes zeros for empty contexts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_common.h"

namespace pkv {

template <int GP, int D> struct SkLayout {
  static constexpr int STRIDE = 2 * GP + GP * D;  // floats per partial: m[GP], l[GP], acc[GP][D]
};

template <int KV, int Q, int D, int GP, int NW>
__global__ void __launch_bounds__(64 * NW)
decode_sk_kernel(const DecodeArgs a) {
  using W = Decoder<KV, Q, D, GP>;
  constexpr int PS = SkLayout<GP, D>::STRIDE;

  extern __shared__ int sk_cum[];  // [N + 1]: chunks of sequences before s
  __shared__ float lds_p[NW][16 * GP];
  __shared__ float lds_alpha[NW][GP];
  __shared__ float lds_inv[NW][GP];
  __shared__ int wave_tot[NW];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int N = a.num_seqs;
  constexpr int NTH = 64 * NW;

  // ---- exclusive prefix of per-sequence chunk counts, in LDS ----
  const int per = (N + NTH - 1) / NTH;
  const int i0 = min(N, tid * per), i1 = min(N, i0 + per);
  int local = 0;
  for (int i = i0; i < i1; ++i) local += (a.context_lens[i] + 15) >> 4;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int run_sum = incl - local;
  for (int w2 = 0; w2 < wv; ++w2) run_sum += wave_tot[w2];
  for (int i = i0; i < i1; ++i) {
    sk_cum[i] = run_sum;
    run_sum += (a.context_lens[i] + 15) >> 4;
  }
  if (tid == NTH - 1) sk_cum[N] = run_sum;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = tid; i <= N; i += NTH) a.sk_cum[i] = sk_cum[i];

  // With fewer units than waves only the first U waves work, one unit each, so that
  // every working wave owns at least one unit (the merge relies on it).
  const long long C = __builtin_amdgcn_readfirstlane(sk_cum[N]);
  const long long U = C * a.num_kv_heads;
  const long long Wn = min((long long)gridDim.x * NW, U);
  const long long w = (long long)blockIdx.x * NW + wv;
  long long u = w < Wn ? U * w / Wn : 0;
  const long long u_end = w < Wn ? U * (w + 1) / Wn : 0;
  const int G = a.num_q_heads / a.num_kv_heads;
  const float vnorm = KV == kFP8 ? a.v_scale : 1.0f;

  W wd;
  wd.init(a, lds_p[wv], lds_alpha[wv]);
  while (u < u_end) {
    const int g = (int)(u / C);
    const int r = (int)(u - (long long)g * C);
    int lo = 0, hi = N;  // largest s with sk_cum[s] <= r (skips empty contexts)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sk_cum[mid] <= r) lo = mid; else hi = mid;
    }
    // Values read from LDS are wave-uniform; say so, so that what derives from them
    // (block-table addresses in particular) stays on the scalar path.
    const int s = __builtin_amdgcn_readfirstlane(lo);
    const int cb = __builtin_amdgcn_readfirstlane(r - sk_cum[s]);
    const int n = __builtin_amdgcn_readfirstlane(sk_cum[s + 1] - sk_cum[s]);
    const int ce = (int)min((long long)n, (long long)cb + (u_end - u));

    wd.begin(a, s, g, a.context_lens[s]);
    run_chunks(wd, cb, ce, 1);
    wd.finish();
    float Mh[GP], Lh[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      Mh[h] = wd.head_m(h);
      Lh[h] = wd.head_l(h);
    }
    if (cb == 0 && ce == n) {
      // the whole context: final output
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) lds_inv[wv][h] = Lh[h] != 0.0f ? vnorm / Lh[h] : 0.0f;
      }
      wave_lds_sync();
      const size_t row0 = ((size_t)s * a.num_q_heads + (size_t)g * G) * D;
      wd.visit([&](int h, int d, float v) {
        store_out(a.out, row0 + (size_t)h * D + d, a.out_dtype, v * lds_inv[wv][h]);
      });
      wave_lds_sync();
    } else {
      float* part = a.sk_part + (2 * w + (cb == 0 ? 1 : 0)) * (long long)PS;
      wd.visit([&](int h, int d, float v) { part[2 * GP + h * D + d] = v; });
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          part[h] = Mh[h];
          part[GP + h] = Lh[h];
        }
      }
    }
    u += ce - cb;
  }
}

// Combine the partials of query head h of one (KV head g, sequence s) segment; zeros
// for an empty context.  The waves that covered the segment are recomputed from the
// same unit arithmetic as the decode kernel: worker_of(u) = floor(((u + 1) W - 1) / U)
// with W = min(waves launched, U), so every wave in [w0, w1] left a partial.
template <int D, int GP, int KV>
__global__ void __launch_bounds__(kMergeThreads) merge_sk_kernel(const DecodeArgs a) {
  constexpr int PS = SkLayout<GP, D>::STRIDE;
  const int h = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int N = a.num_seqs;
  const int G = a.num_q_heads / a.num_kv_heads;
  if (h >= G) return;
  const int cs = a.sk_cum[s];
  const int n = a.sk_cum[s + 1] - cs;
  const size_t row = ((size_t)s * a.num_q_heads + (size_t)g * G + h) * D;
  if (n == 0) {
    for (int d = threadIdx.x; d < D; d += kMergeThreads) store_out(a.out, row + d, a.out_dtype, 0.0f);
    return;
  }
  const long long C = a.sk_cum[N];
  const long long U = C * a.num_kv_heads;
  const long long Wn = min((long long)a.sk_workers, U);
  const long long start = (long long)g * C + cs, last = start + n - 1;
  const long long w0 = ((start + 1) * Wn - 1) / U;
  const long long w1 = ((last + 1) * Wn - 1) / U;
  if (w0 == w1) return;  // one wave covered it and wrote the output
  merge_head<D>((int)(w1 - w0 + 1), [&](int p) {
    const long long w = w0 + p;
    const float* q = a.sk_part + (2 * w + (p == 0 ? 1 : 0)) * (long long)PS;
    return PartialRef{q + h, q + GP + h, q + 2 * GP + h * D};
  }, a.out, row, a.out_dtype, KV == kFP8 ? a.v_scale : 1.0f);
}

// ---- dispatch --------------------------------------------------------------------
constexpr int kSkWaves = 4;

template <int KV, int Q, int D, int GP>
struct SkKernels {
  static const void* decode() { return (const void*)&decode_sk_kernel<KV, Q, D, GP, kSkWaves>; }
  static hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
    const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int);
    hipLaunchKernelGGL((decode_sk_kernel<KV, Q, D, GP, kSkWaves>), dim3(a.sk_workers / kSkWaves),
                       dim3(64 * kSkWaves), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int G = a.num_q_heads / a.num_kv_heads;
    hipLaunchKernelGGL((merge_sk_kernel<D, GP, KV>), dim3(G, a.num_kv_heads, a.num_seqs),
                       dim3(kMergeThreads), 0, stream, a);
    return hipGetLastError();
  }
};

// Resolve (cache dtype, q dtype, head dim, padded group) to the kernel pair and run f.
template <typename F>
static hipError_t with_sk(int kv, int q, int d, int gp, F&& f) {
#define PKV_SK_GP(KV, Q, D)                                   \
  switch (gp) {                                               \
    case 1: return f(SkKernels<KV, Q, D, 1>());               \
    case 2: return f(SkKernels<KV, Q, D, 2>());               \
    case 4: return f(SkKernels<KV, Q, D, 4>());               \
    case 8: return f(SkKernels<KV, Q, D, 8>());               \
    case 16: return f(SkKernels<KV, Q, D, 16>());             \
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
  return hipErrorInvalidValue;
}

int pad_group(int G) {
  int gp = 1;
  while (gp < G) gp <<= 1;
  return gp;
}

int streamk_workers(int cache_dtype, int q_dtype, int head_dim, int group, int num_seqs) {
  int dev = 0, cus = 0, per_cu = 0;
  const size_t lds = (size_t)(num_seqs + 1) * sizeof(int);
  int workers = 0;
  hipError_t e = with_sk(cache_dtype, q_dtype, head_dim, pad_group(group), [&](auto k) {
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k.decode(), 64 * kSkWaves, lds) != hipSuccess) {
      (void)hipGetLastError();
      cus = 256;  // no device visible (host-only use): size for a full MI355X
      per_cu = 8;
    }
    workers = (cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1) * kSkWaves;
    return hipSuccess;
  });
  return e == hipSuccess ? workers : 0;
}

size_t streamk_ws_bytes(int num_seqs, int group, int head_dim, int workers) {
  const int gp = pad_group(group);
  return align256((size_t)(num_seqs + 1) * sizeof(int)) +
         align256((size_t)2 * workers * (2 * gp + gp * head_dim) * sizeof(float));
}

hipError_t launch_decode_streamk(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  return with_sk(a.cache_dtype, a.q_dtype, a.head_dim, pad_group(G),
                 [&](auto k) { return k.launch(a, stream); });
}

}  // namespace pkv
