// Paged decode attention for gfx950, balanced schedule: the kernel template.  The
// instantiations live in decode_sk_<dtype>.hip, the dispatch in decode_sk.hip.
//
// The work of one decode step is the list of 16-token chunks of every (KV head,
// sequence) context, KV-head major: U = H_kv * sum_s ceil(ctx_s / 16) units.  A
// (KV head, sequence) context is a *segment*: a contiguous unit range.  The launch
// holds one workgroup per resident slot (on a full MI355X one per CU, NW waves that
// fill it), and the unit list is split evenly twice: workgroup b takes
// [U b / NB, U (b+1) / NB), and its waves split that range the same way.  Every wave
// streams the same number of K/V bytes (to within one chunk) whatever the mix of
// context lengths, and the whole launch is one round of resident waves.  (Several
// workgroups sharing a CU progress at very different speeds on gfx950 -- the older
// one gets priority -- while the waves of one workgroup stay within a few
// microseconds of each other, hence one workgroup per CU.)
//
// A wave walks its range one segment piece at a time with the per-wave steps of
// decode_common.h (online softmax, "Optimizacion de Inferencia LLM", sections
// "PagedAttention: Conceptos de SO..." and "FlashAttention-3...").  A segment it
// covers entirely is written straight to `out`.  Otherwise the piece's partial
// result (running max m, denominator l, unnormalised output acc) goes to LDS, and
// the partials are combined with the log-sum-exp algebra of the online softmax:
//   * inside a workgroup, by the wave that arrives last at the segment (an LDS
//     counter);
//   * a segment that crosses workgroups leaves one combined partial per workgroup in
//     the workspace, and the workgroup that arrives last at it (a device-wide counter
//     in the workspace header) combines those and writes the output.
// A wave does the piece that continues past its range first, so most cross-range
// partials are published early and their merges overlap other waves' streaming.  For the
// same reason the two ends of a workgroup's range, where segments cross into the
// neighbouring workgroups' ranges and need the device-scope merge, go to the older wave
// of each SIMD pair (waves 0-3): of the two waves sharing a SIMD the older one runs well
// ahead of the younger, which streams mostly after it (measured with per-wave
// timestamps), so those merges finish early instead of at the kernel's end (prefix-sharing
// workload 95 -> 89 us; the others unchanged).
//
// Visibility across XCDs.  Each XCD has its own L2, not coherent with the others for
// ordinary stores.  Cross-workgroup partials are therefore stored and loaded with the
// device-scope cache policy (sc1), which completes a store only once it is visible
// device-wide and serves a load from the device-coherent level; the publishing wave
// waits for its stores (s_waitcnt) before its counter increment, and the merging wave
// issues its loads only after the increment has returned.  (An agent-scope release
// fence would instead write back the whole L2.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_common.h"

namespace pkv {

// One partial: m[GP], l[GP], then acc[GP][D] from a 16-byte boundary.
template <int GP, int D> struct SkLayout {
  static constexpr int ACC = (2 * GP + 3) & ~3;
  static constexpr int STRIDE = ACC + GP * D;  // floats, a multiple of 4
};

// Waves per workgroup: as many as one CU keeps resident for the decoder's register
// footprint (2 per SIMD up to 8 query heads per KV head, 1 beyond or for fp32 caches),
// so that one workgroup fills a CU.  (Three per SIMD would cap a wave at 168 VGPRs,
// which spills; 8 waves of one chunk in flight each already stream at the rate 12 do.)
template <int KV, int GP> struct SkShape {
  static constexpr int NW = KV == kF32 ? 4 : (GP <= 8 ? 8 : 4);
};

// Quotient of non-negative operands: a 32-bit division (a few instructions) when both
// fit in 31 bits, as they do for any realistic unit count, else the 64-bit one.
__device__ __forceinline__ long long udiv(long long a, long long b) {
  if (((a | b) >> 31) == 0) return (long long)((uint32_t)a / (uint32_t)b);
  return a / b;
}

// floor-division split of T items into P parts: part p holds [T p / P, T (p+1) / P);
// owner(x) is the part holding item x (T >= P >= 1, so no part is empty).
__device__ __forceinline__ long long split_begin(long long T, long long P, long long p) { return udiv(T * p, P); }
__device__ __forceinline__ long long split_owner(long long T, long long P, long long x) {
  return udiv((x + 1) * P - 1, T);
}

// The largest s in [0, N) with cum[s] <= r, for non-decreasing cum (N + 1 entries) with
// cum[0] = 0 <= r < cum[N]: the sequence holding chunk r (an empty context, whose cum
// equals the next one's, is skipped).  Each round the wave samples 64 evenly spaced
// entries of the remaining span and counts those <= r with a ballot -- they form a
// prefix -- narrowing the span 64-fold (one round up to 64 sequences, two up to 4096).
__device__ __forceinline__ int find_seq(const int* cum, int N, int r) {
  const int lane = threadIdx.x & 63;
  int lo = 0, span = N;
  while (span > 1) {
    const int step = (span + 63) >> 6;
    const int idx = lo + lane * step;
    const bool le = idx < lo + span && cum[idx] <= r;
    const int c = __popcll(__ballot(le));  // >= 1: lane 0 reads cum[lo] <= r
    const int end = lo + span;
    lo += (c - 1) * step;
    span = min(step, end - lo);
  }
  return lo;
}

// Per-lane view of the G x D output rows of one segment: lane t handles float4 t,
// t + 64, ... (EPL of them).
template <int GP, int D> struct RowSet {
  static constexpr int D4 = D / 4;
  static constexpr int EPL = (GP * D4 + 63) / 64;
  int hh[EPL], dd[EPL];
  bool ok[EPL];
  float M[EPL], L[EPL];
  float4 A[EPL];
  __device__ __forceinline__ void init(int lane, int G) {
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int e = lane + 64 * k;
      hh[k] = e / D4;
      dd[k] = 4 * (e - hh[k] * D4);
      ok[k] = hh[k] < G;
      if (!ok[k]) hh[k] = 0, dd[k] = 0;
      M[k] = kNegInf;
      L[k] = 0.0f;
      A[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  }
  // fold one partial (m, l, acc) of element k into the running combination
  __device__ __forceinline__ void add(int k, float m, float l, float4 x) {
    const float Mn = fmaxf(M[k], m);
    const float base = Mn == kNegInf ? 0.0f : Mn;
    const float fo = fast_exp2(M[k] - base), fn = fast_exp2(m - base);
    L[k] = L[k] * fo + l * fn;
    A[k].x = A[k].x * fo + x.x * fn;
    A[k].y = A[k].y * fo + x.y * fn;
    A[k].z = A[k].z * fo + x.z * fn;
    A[k].w = A[k].w * fo + x.w * fn;
    M[k] = Mn;
  }
  __device__ __forceinline__ void write_out(const DecodeArgs& a, size_t row0, float vnorm) const {
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      if (!ok[k]) continue;
      const float inv = L[k] != 0.0f ? vnorm / L[k] : 0.0f;
      const size_t o = row0 + (size_t)hh[k] * D + dd[k];
      store_out(a.out, o + 0, a.out_dtype, A[k].x * inv);
      store_out(a.out, o + 1, a.out_dtype, A[k].y * inv);
      store_out(a.out, o + 2, a.out_dtype, A[k].z * inv);
      store_out(a.out, o + 3, a.out_dtype, A[k].w * inv);
    }
  }
};

// A segment: units [xs, xe) of KV head g, sequence s.
struct Seg {
  long long xs, xe;
  int g, s, n;
};

// PRE: each sequence's first seq_begin[s] tokens were attended by the shared-prefix
// kernel, which left pre_splits partials per (sequence, query head) in pre_part; this
// kernel streams only the rest of each context and folds those partials in once per
// segment: into the result of the segment's first piece, from LDS that the piece's wave
// filled while it streamed (when the segment's partial rows fit in its LDS area), or
// else, read from memory, wherever it writes a final output.  A piece covering a whole
// segment waits in a third LDS slot of its wave for that fold instead of being written
// straight out.
template <int KV, int Q, int D, int GP, int NW, bool NT, bool PRE>
__global__ void __launch_bounds__(64 * NW)
decode_sk_kernel(const DecodeArgs a) {
  using W = Decoder<KV, Q, D, GP, NT>;
  using L_ = SkLayout<GP, D>;
  using RS = RowSet<GP, D>;
  constexpr int NSLOT = PRE ? 3 : 2;
  constexpr int PSTRIDE = 4 + D;  // floats per prefix partial: m, l, pad, pad, acc[D]

  extern __shared__ int sk_cum[];  // [N + 1]: chunks of sequences before s
  __shared__ __attribute__((aligned(16))) float lds_part[NSLOT * NW][L_::STRIDE];
  __shared__ int lds_count[NW];    // arrivals at the segment whose first wave is i
  __shared__ float lds_p[NW][16 * GP];
  __shared__ float lds_alpha[NW][GP];
  __shared__ float lds_inv[NW][GP];
  __shared__ int wave_tot[NW];
  // PRE: the prefix partials of a segment (its G heads x pre_splits slices, contiguous
  // rows of 4 + D floats) are loaded straight into this wave's LDS area when the wave
  // starts the segment's first piece, and folded into that piece's result when it ends,
  // so no output waits on them.  Up to kPreRows rows, in whole 1 KiB wave loads.
  constexpr bool PRE_LDS = PRE && GP <= 4;
  constexpr int kPreRows = 16;
  constexpr int PRE_FLOATS = (kPreRows * (4 + D) * 4 + 1023) / 1024 * 256;
  __shared__ __attribute__((aligned(16))) float lds_pre[PRE_LDS ? NW : 1][PRE_LDS ? PRE_FLOATS : 4];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int N = a.num_seqs;
  constexpr int NTH = 64 * NW;

  // ---- exclusive prefix of per-sequence chunk counts, in LDS ----
  const int per = (N + NTH - 1) / NTH;
  const int i0s = min(N, tid * per), i1s = min(N, i0s + per);
  // chunks of sequence i this kernel streams: its attended chunks (all of them without
  // a window), after its shared prefix when PRE (which takes no window)
  auto chunks_of = [&](int i) {
    if constexpr (PRE) return max(0, ((a.context_lens[i] + 15) >> 4) - (a.seq_begin[i] >> 4));
    return attended_chunk_count(a.context_lens[i], a.window, a.sinks);
  };
  // a thread's first few counts are kept in registers (their loads issued together) for
  // the second pass below; beyond that (thousands of sequences) they are read again
  constexpr int kKeep = 4;
  int kept[kKeep];
  int local = 0;
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    kept[k] = i0s + k < i1s ? chunks_of(i0s + k) : 0;
    local += kept[k];
  }
  for (int i = i0s + kKeep; i < i1s; ++i) local += chunks_of(i);
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wave_tot[wv] = incl;
  if (tid < NW) lds_count[tid] = 0;
  __syncthreads();
  int run_sum = incl - local;
  for (int w2 = 0; w2 < wv; ++w2) run_sum += wave_tot[w2];
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    if (i0s + k < i1s) sk_cum[i0s + k] = run_sum;
    run_sum += kept[k];
  }
  for (int i = i0s + kKeep; i < i1s; ++i) {
    sk_cum[i] = run_sum;
    run_sum += chunks_of(i);
  }
  if (tid == NTH - 1) sk_cum[N] = run_sum;
  __syncthreads();

  const long long C = __builtin_amdgcn_readfirstlane(sk_cum[N]);
  const long long U = C * a.num_kv_heads;
  const int G = a.num_q_heads / a.num_kv_heads;
  const float vnorm = KV == kFP8 ? a.v_scale : 1.0f;

  // Fold the prefix partials of (sequence s, KV head g) into rs (PRE, s has a prefix).
  // The slices' loads go out in batches (as many as 8 partial elements of registers
  // allow) so a fold waits for memory once per batch, not once per slice; a batch's
  // entries past the last slice re-read it and weigh nothing (m = -inf).
  auto add_prefix = [&](RS& rs, int s, int g) {
    if constexpr (PRE) {
      if (a.seq_begin[s] <= 0) return;
      constexpr int BATCH = RS::EPL >= 8 ? 1 : 8 / RS::EPL;
      const int T = a.pre_splits;
      const float* base = a.pre_part + ((size_t)s * a.num_q_heads + (size_t)g * G) * T * PSTRIDE;
      for (int t0 = 0; t0 < T; t0 += BATCH) {
        float pm[BATCH][RS::EPL], pl[BATCH][RS::EPL];
        float4 px[BATCH][RS::EPL];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
          const int t = min(t0 + b, T - 1);
#pragma unroll
          for (int k = 0; k < RS::EPL; ++k) {
            const float* pp = base + ((size_t)rs.hh[k] * T + t) * PSTRIDE;
            pm[b][k] = t0 + b < T ? pp[0] : kNegInf;
            pl[b][k] = pp[1];
            px[b][k] = *(const float4*)(pp + 4 + rs.dd[k]);
          }
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
#pragma unroll
          for (int k = 0; k < RS::EPL; ++k) rs.add(k, pm[b][k], pl[b][k], px[b][k]);
      }
    }
  };

  // Prefix partials in LDS (PRE_LDS, when a segment's G x pre_splits rows fit): issued
  // before the piece's first K/V loads, so they arrive with them.  Bytes past the
  // segment's rows read as zeros (the resource ends there) into the rest of the area.
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const bool pre_early = PRE_LDS && G * a.pre_splits <= kPreRows;
  auto prefetch_prefix = [&](int s, int g) {
    if constexpr (PRE_LDS) {
      const int T = a.pre_splits;
      const float* base = a.pre_part + ((size_t)s * a.num_q_heads + (size_t)g * G) * T * PSTRIDE;
      const __amdgpu_buffer_rsrc_t r = tile_rsrc((const uint8_t*)base, G * T * PSTRIDE * (int)sizeof(float));
#pragma unroll
      for (int i = 0; i < PRE_FLOATS / 256; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)&lds_pre[wvu][256 * i],
                                                 16, 16 * lane + 1024 * i, 0, 0, 0);
    }
  };
  // Fold the partials prefetched into this wave's LDS area into rs.
  auto add_prefix_lds = [&](RS& rs) {
    if constexpr (PRE_LDS) {
      __builtin_amdgcn_s_waitcnt(0);  // the loads into LDS are complete
      wave_lds_sync();
      const int T = a.pre_splits;
      for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int k = 0; k < RS::EPL; ++k) {
          const float* pp = &lds_pre[wvu][(rs.hh[k] * T + t) * PSTRIDE];
          rs.add(k, pp[0], pp[1], *(const float4*)(pp + 4 + rs.dd[k]));
        }
      }
    }
  };

  // Contexts with no chunk to stream own no unit: zeros, or (PRE) their prefix alone;
  // spread over all waves.
  {
    const long long Wl = (long long)gridDim.x * NW, w = (long long)blockIdx.x * NW + wv;
    for (long long s = w; s < N; s += Wl) {
      if (sk_cum[s + 1] != sk_cum[s]) continue;
      const size_t row0 = (size_t)s * a.num_q_heads * D;
      if (PRE && a.seq_begin[s] > 0) {
        for (int g = 0; g < a.num_kv_heads; ++g) {
          RS rs;
          rs.init(lane, G);
          add_prefix(rs, (int)s, g);
          rs.write_out(a, row0 + (size_t)g * G * D, vnorm);
        }
      } else {
        for (int i = lane; i < a.num_q_heads * D; i += 64) store_out(a.out, row0 + i, a.out_dtype, 0.0f);
      }
    }
  }

  // ---- this workgroup's and this wave's unit ranges (only non-empty parts exist) ----
  const long long NB = min((long long)gridDim.x, U);
  const long long b = blockIdx.x;
  if (b >= NB) return;  // whole workgroup: no barrier follows
  const long long ub = split_begin(U, NB, b), ue = split_begin(U, NB, b + 1);
  const long long Lb = ue - ub;
  const int NWn = (int)min((long long)NW, Lb);
  // the part of the workgroup's range this wave takes: with a full workgroup of 8 waves the
  // older wave of each SIMD pair (waves 0-3) takes the range's two ends
  const int pw = (NW == 8 && NWn == 8) ? ((wv < 4) ? ((wv < 2) ? wv : wv + 4) : wv - 2) : wv;
  const long long wb = pw < NWn ? ub + split_begin(Lb, NWn, pw) : ub;
  const long long we = pw < NWn ? ub + split_begin(Lb, NWn, pw + 1) : ub;

  const __amdgpu_buffer_rsrc_t parts = __builtin_amdgcn_make_buffer_rsrc(
      a.sk_part, (short)0, (int)(2 * NB * L_::STRIDE * sizeof(float)), kRsrcWord3);

  auto seg_of = [&](long long u) {
    Seg x;
    x.g = (int)udiv(u, C);
    const int r = (int)(u - (long long)x.g * C);
    // Values read from LDS are wave-uniform; say so, so that what derives from them
    // (block-table addresses in particular) stays on the scalar path.
    x.s = __builtin_amdgcn_readfirstlane(find_seq(sk_cum, N, r));
    const int cs = __builtin_amdgcn_readfirstlane(sk_cum[x.s]);
    x.n = __builtin_amdgcn_readfirstlane(sk_cum[x.s + 1]) - cs;
    x.xs = (long long)x.g * C + cs;
    x.xe = x.xs + x.n;
    return x;
  };

  W wd;
  wd.init(a, lds_p[wv], lds_alpha[wv]);

  // Units [u0, u1) of segment X.
  auto do_piece = [&](const Seg& X, long long u0, long long u1) {
    const int cb = (int)(u0 - X.xs), ce = (int)(u1 - X.xs);
    const int ctx = a.context_lens[X.s];
    // PRE: the piece starting a segment with a shared prefix takes the prefix in
    const bool fold_here = pre_early && cb == 0 && a.seq_begin[X.s] > 0;
    if (fold_here) prefetch_prefix(X.s, X.g);
    wd.begin(a, X.s, X.g, ctx);
    if constexpr (PRE) {
      const int cb0 = a.seq_begin[X.s] >> 4;  // first streamed chunk of the context
      run_chunks(wd, cb0 + cb, cb0 + ce, 1);
    } else {
      int ca, cw;  // attended chunks [0, ca) and [cw, ...): units count them without the gap
      attended_chunks(ctx, a.window, a.sinks, ca, cw);
      run_chunks(wd, cb, ce, 1, __builtin_amdgcn_readfirstlane(ca), __builtin_amdgcn_readfirstlane(cw - ca));
    }
    wd.finish();
    float Mh[GP], Lh[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      Mh[h] = wd.head_m(h);
      Lh[h] = wd.head_l(h);
    }
    const size_t row0 = ((size_t)X.s * a.num_q_heads + (size_t)X.g * G) * D;
    const bool full = cb == 0 && ce == X.n;
    if (!PRE && full) {  // the whole context: final output
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) lds_inv[wv][h] = Lh[h] != 0.0f ? vnorm / Lh[h] : 0.0f;
      }
      wave_lds_sync();
      wd.visit([&](int h, int d, float v) {
        store_out(a.out, row0 + (size_t)h * D + d, a.out_dtype, v * lds_inv[wv][h]);
      });
      wave_lds_sync();
      return;
    }
    // Partial: slot 1 if the piece starts the segment and continues past this wave,
    // slot 0 if it continues one that started before this wave's range, slot 2 (PRE)
    // if it is the whole segment.
    float* lp = lds_part[NSLOT * pw + (full ? 2 : (cb == 0 ? 1 : 0))];
    wd.visit([&](int h, int d, float v) { lp[L_::ACC + h * D + d] = v; });
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        lp[h] = Mh[h];
        lp[GP + h] = Lh[h];
      }
    }
    // The waves of this workgroup that cover X: i0 .. i1.
    const int i0 = (int)split_owner(Lb, NWn, max(X.xs, ub) - ub);
    const int i1 = (int)split_owner(Lb, NWn, min(X.xe, ue) - 1 - ub);
    if (fold_here) {  // the segment's first piece: fold in the prefix from LDS
      wave_lds_sync();
      RS rs;
      rs.init(lane, G);
#pragma unroll
      for (int k = 0; k < RS::EPL; ++k)
        rs.add(k, lp[rs.hh[k]], lp[GP + rs.hh[k]], *(const float4*)(lp + L_::ACC + rs.hh[k] * D + rs.dd[k]));
      add_prefix_lds(rs);
      if (full) {  // the whole segment: write
        rs.write_out(a, row0, vnorm);
        wave_lds_sync();  // the slot is reused by this wave's next whole segment
        return;
      }
      // else the piece's partial, now with the prefix, goes back to its slot
#pragma unroll
      for (int k = 0; k < RS::EPL; ++k) {
        if (!rs.ok[k]) continue;
        *(float4*)(lp + L_::ACC + rs.hh[k] * D + rs.dd[k]) = rs.A[k];
        if (rs.dd[k] == 0) {
          lp[rs.hh[k]] = rs.M[k];
          lp[GP + rs.hh[k]] = rs.L[k];
        }
      }
    }
    if (PRE && full) {  // this wave holds the whole segment: fold in the prefix, write
      wave_lds_sync();
      RS rs;
      rs.init(lane, G);
#pragma unroll
      for (int k = 0; k < RS::EPL; ++k)
        rs.add(k, lp[rs.hh[k]], lp[GP + rs.hh[k]], *(const float4*)(lp + L_::ACC + rs.hh[k] * D + rs.dd[k]));
      add_prefix(rs, X.s, X.g);
      rs.write_out(a, row0, vnorm);
      wave_lds_sync();  // the slot is reused by this wave's next whole segment
      return;
    }
    if (i1 > i0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      int prev = 0;
      if (lane == 0)
        prev = __hip_atomic_fetch_add(&lds_count[i0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      prev = __builtin_amdgcn_readfirstlane(prev);
      if (prev != i1 - i0) return;  // another wave of this workgroup combines
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    } else {
      wave_lds_sync();
    }
    // This wave arrived last in the workgroup: combine the workgroup's pieces.  Wave
    // i0's piece is in its slot 1 if X starts inside i0's range, else in slot 0; the
    // later waves' pieces continue X, slot 0.
    RS rs;
    rs.init(lane, G);
    for (int i = i0; i <= i1; ++i) {
      const int sl = (i == i0 && X.xs >= ub + split_begin(Lb, NWn, i0)) ? 1 : 0;
      const float* q = lds_part[NSLOT * i + sl];
#pragma unroll
      for (int k = 0; k < RS::EPL; ++k)
        rs.add(k, q[rs.hh[k]], q[GP + rs.hh[k]], *(const float4*)(q + L_::ACC + rs.hh[k] * D + rs.dd[k]));
    }
    if (X.xs >= ub && X.xe <= ue) {  // X lies inside this workgroup's range
      if (!pre_early) add_prefix(rs, X.s, X.g);
      rs.write_out(a, row0, vnorm);
      return;
    }
    // Publish this workgroup's partial of X: slot 1 if X starts in this workgroup's
    // range, else slot 0 (the same rule one level up).
    const int gbase = (int)((2 * b + (X.xs >= ub ? 1 : 0)) * L_::STRIDE * sizeof(float));
#pragma unroll
    for (int k = 0; k < RS::EPL; ++k) {
      if (!rs.ok[k]) continue;
      const u32x4_t v = {f32_bits(rs.A[k].x), f32_bits(rs.A[k].y), f32_bits(rs.A[k].z), f32_bits(rs.A[k].w)};
      __builtin_amdgcn_raw_buffer_store_b128(v, parts, gbase + (L_::ACC + rs.hh[k] * D + rs.dd[k]) * 4, 0,
                                             kAuxDevice);
      if (rs.dd[k] == 0) {  // one lane per head row also stores its (m, l)
        __builtin_amdgcn_raw_buffer_store_b32(f32_bits(rs.M[k]), parts, gbase + rs.hh[k] * 4, 0, kAuxDevice);
        __builtin_amdgcn_raw_buffer_store_b32(f32_bits(rs.L[k]), parts, gbase + (GP + rs.hh[k]) * 4, 0,
                                              kAuxDevice);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the stores above are complete, device-wide
    const long long b0 = split_owner(U, NB, X.xs), b1 = split_owner(U, NB, X.xe - 1);
    int prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(a.sk_count + b0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (int)(b1 - b0)) return;  // another workgroup combines
    // Last workgroup at X: combine the partials of workgroups b0 (slot 1: X starts in
    // its range) .. b1 (slot 0), read at device scope, and write the output.
    RS fin;
    fin.init(lane, G);
    for (long long bb = b0; bb <= b1; ++bb) {
      const int base = (int)((2 * bb + (bb == b0 ? 1 : 0)) * L_::STRIDE * sizeof(float));
#pragma unroll
      for (int k = 0; k < RS::EPL; ++k) {
        const float m = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(parts, base + fin.hh[k] * 4, 0, kAuxDevice));
        const float l = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(parts, base + (GP + fin.hh[k]) * 4, 0, kAuxDevice));
        const u32x4_t x = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
            parts, base + (L_::ACC + fin.hh[k] * D + fin.dd[k]) * 4, 0, kAuxDevice));
        fin.add(k, m, l, make_float4(bits_f32(x.x), bits_f32(x.y), bits_f32(x.z), bits_f32(x.w)));
      }
    }
    if (!pre_early) add_prefix(fin, X.s, X.g);
    fin.write_out(a, row0, vnorm);
    if (lane == 0) __hip_atomic_store(a.sk_count + b0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  if (wb >= we) return;
  // Piece order: the last piece first when it continues past this wave's range, then
  // the rest in order.  One call site keeps one copy of the pipeline in the code.
  const Seg last = seg_of(we - 1);
  const long long split = max(wb, last.xs);
  bool pending_last = we < last.xe;
  const long long stop = pending_last ? split : we;
  long long u = wb;
  while (true) {
    Seg X;
    long long p0, p1;
    if (pending_last) {
      X = last;
      p0 = split;
      p1 = we;
      pending_last = false;
    } else {
      if (u >= stop) break;
      X = seg_of(u);
      p0 = u;
      p1 = min(stop, X.xe);
      u = p1;
    }
    do_piece(X, p0, p1);
  }
}

// Launcher of one instantiation; explicitly instantiated per cache dtype in
// decode_sk_<dtype>.hip.
template <int KV, int Q, int D, int GP, bool NT, bool PRE = false>
struct SkKernels {
  static constexpr int NW = SkShape<KV, GP>::NW;
  static constexpr int STRIDE = SkLayout<GP, D>::STRIDE;
  static const void* decode();
  static hipError_t launch(const DecodeArgs& a, hipStream_t stream);
};

#ifdef PKV_SK_DEFINE
template <int KV, int Q, int D, int GP, bool NT, bool PRE>
const void* SkKernels<KV, Q, D, GP, NT, PRE>::decode() {
  return (const void*)&decode_sk_kernel<KV, Q, D, GP, NW, NT, PRE>;
}
template <int KV, int Q, int D, int GP, bool NT, bool PRE>
hipError_t SkKernels<KV, Q, D, GP, NT, PRE>::launch(const DecodeArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int);
  hipLaunchKernelGGL((decode_sk_kernel<KV, Q, D, GP, NW, NT, PRE>), dim3(a.sk_workers / NW), dim3(64 * NW),
                     lds, stream, a);
  return hipGetLastError();
}
#endif

// Every (head dim, padded group, load policy) of one (cache, query) dtype pair.
#define PKV_SK_FOR_DTYPES(X, KV, Q)                                              \
  X(KV, Q, 64, 1) X(KV, Q, 64, 2) X(KV, Q, 64, 4) X(KV, Q, 64, 8) X(KV, Q, 64, 16) \
  X(KV, Q, 128, 1) X(KV, Q, 128, 2) X(KV, Q, 128, 4) X(KV, Q, 128, 8) X(KV, Q, 128, 16)
#define PKV_SK_INSTANTIATE(KV, Q, D, GP)          \
  template struct SkKernels<KV, Q, D, GP, true>;  \
  template struct SkKernels<KV, Q, D, GP, false>;
#define PKV_SK_EXTERN(KV, Q, D, GP)                      \
  extern template struct SkKernels<KV, Q, D, GP, true>;  \
  extern template struct SkKernels<KV, Q, D, GP, false>;
// the suffix pass of the shared-prefix decode: private blocks, streaming loads
#define PKV_SK_INSTANTIATE_PRE(KV, Q, D, GP) template struct SkKernels<KV, Q, D, GP, true, true>;
#define PKV_SK_EXTERN_PRE(KV, Q, D, GP) extern template struct SkKernels<KV, Q, D, GP, true, true>;

}  // namespace pkv
