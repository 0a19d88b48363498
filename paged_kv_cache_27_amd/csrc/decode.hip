// Paged decode attention for gfx950 with fixed context partitions.
//
// What is computed: for each sequence s and query head h,
//   out[s][h] = softmax_t(scale * q[s][h] . K_t) V_t,  t = 0 .. ctx[s]-1,
// K_t / V_t of KV head h / G, found through the block table ("Capitulo 2", section
// "Que guarda realmente el KV cache"; "Optimizacion de Inferencia LLM", section
// "El Cuello de Botella...").
//
// This file holds the fixed-partition schedule: one workgroup of NW waves per
// (partition, KV head, sequence); the partition's 16-token chunks are dealt
// round-robin to the waves, which are merged through LDS at the end (both
// decoders of decode_common.h work here).  With one
// partition the workgroup writes the output; otherwise it stores (max,
// denominator, unnormalised output) and merge_kernel combines the partitions of
// each (sequence, query head).  The per-wave steps live in decode_common.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_common.h"

namespace pkv {

template <int KV, int Q, int D, int GP, int NW, bool NT>
__global__ void __launch_bounds__(64 * NW)
decode_kernel(const DecodeArgs a) {
  using W = Decoder<KV, Q, D, GP, NT>;

  __shared__ float lds_p[NW][16 * GP];
  __shared__ float lds_alpha[NW][GP];
  __shared__ float lds_m[NW][GP];
  __shared__ float lds_l[NW][GP];
  __shared__ float lds_acc[NW][GP * D];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int part = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int ctx = a.context_lens[s];
  const int tok_begin = part * a.partition;
  if (part > 0 && tok_begin >= ctx) return;  // whole workgroup: no barrier reached
  const int tok_end = min(ctx, tok_begin + a.partition);
  const int G = a.num_q_heads / a.num_kv_heads;

  W wd;
  wd.init(a, lds_p[wv], lds_alpha[wv]);
  wd.begin(a, s, g, ctx);
  // Partitions are multiples of 16 tokens, so chunks never straddle two partitions.
  // The partition's chunks, without those outside a window's attended ranges (in the
  // gap-free numbering of run_chunks; a partition wholly in the gap has none and
  // leaves a neutral partial).
  int ca, cw;
  attended_chunks(ctx, a.window, a.sinks, ca, cw);
  auto gapless = [&](int c) { return c < ca ? c : (c < cw ? ca : c - (cw - ca)); };
  run_chunks(wd, gapless(tok_begin / 16) + wv, gapless((tok_end + 15) / 16), NW, ca, cw - ca);

  wd.finish();
  wd.visit([&](int h, int d, float v) { lds_acc[wv][h * D + d] = v; });
  float mh[GP], lh[GP];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    mh[h] = wd.head_m(h);
    lh[h] = wd.head_l(h);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      lds_m[wv][h] = mh[h];
      lds_l[wv][h] = lh[h];
    }
  }
  __syncthreads();

  // ---- merge the waves; write the output (single pass) or the partition's partials ----
  const float vnorm = KV == kFP8 ? a.v_scale : 1.0f;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) {
    const int h = idx / D, d = idx - h * D;
    float M = kNegInf;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, lds_m[w2][h]);
    float L = 0.0f, A = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        const float f = fast_exp2(lds_m[w2][h] - M);
        L += f * lds_l[w2][h];
        A += f * lds_acc[w2][h * D + d];
      }
    }
    const size_t hq = (size_t)s * a.num_q_heads + (size_t)g * G + h;
    if (a.num_partitions == 1) {
      store_out(a.out, hq * D + d, a.out_dtype, L != 0.0f ? A / L * vnorm : 0.0f);
    } else {
      const size_t pi = hq * a.num_partitions + part;
      a.ws_acc[pi * D + d] = A;
      if (d == 0) {
        a.ws_m[pi] = M;
        a.ws_l[pi] = L;
      }
    }
  }
}

// Merge of the partitions of one (sequence, query head).  Partitions at or past
// the sequence's context were never written and are not read.
template <int D, int KV>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(const DecodeArgs a) {
  const int hq = blockIdx.x, s = blockIdx.y;
  const int ctx = a.context_lens[s];
  const int np = (ctx + a.partition - 1) / a.partition;
  const size_t base = ((size_t)s * a.num_q_heads + hq) * a.num_partitions;
  merge_head<D>(np, [&](int p) {
    return PartialRef{a.ws_m + base + p, a.ws_l + base + p, a.ws_acc + (base + p) * D};
  }, a.out, ((size_t)s * a.num_q_heads + hq) * D, a.out_dtype, KV == kFP8 ? a.v_scale : 1.0f);
}

// ---- dispatch --------------------------------------------------------------------
constexpr int kWaves = 4;

template <int KV, int Q, int D, int GP>
static hipError_t launch_gp(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
  if (a.kv_stream)
    hipLaunchKernelGGL((decode_kernel<KV, Q, D, GP, kWaves, true>), grid, dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<KV, Q, D, GP, kWaves, false>), grid, dim3(64 * kWaves), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions == 1) return e;
  hipLaunchKernelGGL((merge_kernel<D, KV>), dim3(a.num_q_heads, a.num_seqs), dim3(kMergeThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <int KV, int Q, int D>
static hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  if (G <= 1) return launch_gp<KV, Q, D, 1>(a, stream);
  if (G <= 2) return launch_gp<KV, Q, D, 2>(a, stream);
  if (G <= 4) return launch_gp<KV, Q, D, 4>(a, stream);
  if (G <= 8) return launch_gp<KV, Q, D, 8>(a, stream);
  if (G <= 16) return launch_gp<KV, Q, D, 16>(a, stream);
  return hipErrorInvalidValue;
}

template <int KV, int Q>
static hipError_t launch_kq(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) return launch_d<KV, Q, 64>(a, stream);
  if (a.head_dim == 128) return launch_d<KV, Q, 128>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.cache_dtype == kBF16 && a.q_dtype == kBF16) return launch_kq<kBF16, kBF16>(a, stream);
  if (a.cache_dtype == kF16 && a.q_dtype == kF16) return launch_kq<kF16, kF16>(a, stream);
  if (a.cache_dtype == kF32 && a.q_dtype == kF32) return launch_kq<kF32, kF32>(a, stream);
  if (a.cache_dtype == kFP8 && a.q_dtype == kBF16) return launch_kq<kFP8, kBF16>(a, stream);
  if (a.cache_dtype == kFP8 && a.q_dtype == kF16) return launch_kq<kFP8, kF16>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
