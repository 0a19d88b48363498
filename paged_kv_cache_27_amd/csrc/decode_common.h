// Per-wave building blocks of the gfx950 paged decode kernels.
//
// One wave processes 16-token chunks of one (sequence, KV head) context and keeps
// the online-softmax state of all G query heads of that KV head, accumulating with
// the rescaling of "Optimizacion de Inferencia LLM", sections "PagedAttention:
// Conceptos de SO..." (per-block loads, online softmax) and "FlashAttention-3..."
// (accumulate with rescaling, write O once).  Two variants:
//
// MfmaDecoder (bf16, f16 and fp8 caches) -- both products on the matrix cores:
//   * Q.K^T: one 16x16x32 MFMA tile per 4 query heads, K as the A operand.  Tile
//     row i is token 4(i%4) + i/4 of the chunk and tile column j is query head j/4
//     (each head repeated over 4 columns), so lane l ends up holding, in register
//     k, the score of head (l%16)/4 against token 4k + l/16.  Each lane's 16-byte K
//     load is directly its A fragment (row 4(l%4) + (l%16)/4, bytes 64c + 16(l/16)).
//   * softmax: per lane over its 4 registers, then across the 4 lane groups with
//     two permlane swaps; no LDS round trip.
//   * P.V: block-diagonal 16x16x16 MFMAs.  With k = 4 t + e (token t of the 4-token
//     step, sub-dim e) and output row i = 4 h + e', A holds p[h][t] where e == e',
//     zero elsewhere, so each lane contributes the one probability it already holds;
//     B is the lane's own V load (token 4k + l/16, D/16 consecutive dims); the
//     accumulator gives lane l head l/16 and D/16 consecutive output dims.  P is
//     split into two bf16 (or f16) terms hi + lo so the product keeps ~16 bits of
//     the probability; for fp8 V a single f16 P is used (the fp8 values are exact
//     in f16).
// ValuDecoder (fp32 caches) -- Q.K^T on the 16x16x4 fp32 MFMA (rows = heads,
//   columns = tokens), P.V on the VALU in fp32 with probabilities through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// ---- Q.K^T MFMA flavours per (cache dtype, query dtype) -------------------------
template <int KV, int Q> struct Qk;

template <> struct Qk<kBF16, kBF16> {
  static constexpr int SUB = 1;  // MFMAs per 16-byte K load
  using frag = bf16x8_t;
  __device__ __forceinline__ static frag kfrag(const uint4& w, int) {
    return __builtin_bit_cast(frag, w);
  }
  __device__ __forceinline__ static int qdim(int c, int grp, int) { return 32 * c + 8 * grp; }
  __device__ __forceinline__ static frag qload(const uint8_t* qrow, int dim) {
    return __builtin_bit_cast(frag, *(const uint4*)(qrow + 2 * dim));
  }
  __device__ __forceinline__ static frag zero() { return __builtin_bit_cast(frag, make_uint4(0, 0, 0, 0)); }
  __device__ __forceinline__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Qk<kF16, kF16> {
  static constexpr int SUB = 1;
  using frag = f16x8_t;
  __device__ __forceinline__ static frag kfrag(const uint4& w, int) {
    return __builtin_bit_cast(frag, w);
  }
  __device__ __forceinline__ static int qdim(int c, int grp, int) { return 32 * c + 8 * grp; }
  __device__ __forceinline__ static frag qload(const uint8_t* qrow, int dim) {
    return __builtin_bit_cast(frag, *(const uint4*)(qrow + 2 * dim));
  }
  __device__ __forceinline__ static frag zero() { return __builtin_bit_cast(frag, make_uint4(0, 0, 0, 0)); }
  __device__ __forceinline__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// fp8 cache, bf16 queries: a 16-byte load holds 16 codes = two bf16x8 fragments;
// e4m3fn -> bf16 is exact.
template <> struct Qk<kFP8, kBF16> {
  static constexpr int SUB = 2;
  using frag = bf16x8_t;
  __device__ __forceinline__ static frag kfrag(const uint4& w, int j) {
    const int lo = (int)(j ? w.z : w.x), hi = (int)(j ? w.w : w.y);
    bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    frag r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
  }
  __device__ __forceinline__ static int qdim(int c, int grp, int j) { return 64 * c + 16 * grp + 8 * j; }
  __device__ __forceinline__ static frag qload(const uint8_t* qrow, int dim) {
    return __builtin_bit_cast(frag, *(const uint4*)(qrow + 2 * dim));
  }
  __device__ __forceinline__ static frag zero() { return __builtin_bit_cast(frag, make_uint4(0, 0, 0, 0)); }
  __device__ __forceinline__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// fp8 cache, f16 queries: e4m3fn -> f16 is exact as well.
template <> struct Qk<kFP8, kF16> {
  static constexpr int SUB = 2;
  using frag = f16x8_t;
  __device__ __forceinline__ static frag kfrag(const uint4& w, int j) {
    const int lo = (int)(j ? w.z : w.x), hi = (int)(j ? w.w : w.y);
    f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    f16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    frag r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
  }
  __device__ __forceinline__ static int qdim(int c, int grp, int j) { return 64 * c + 16 * grp + 8 * j; }
  __device__ __forceinline__ static frag qload(const uint8_t* qrow, int dim) {
    return __builtin_bit_cast(frag, *(const uint4*)(qrow + 2 * dim));
  }
  __device__ __forceinline__ static frag zero() { return __builtin_bit_cast(frag, make_uint4(0, 0, 0, 0)); }
  __device__ __forceinline__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// fp32 cache and queries: 16x16x4 fp32 MFMA; one 16-byte load = four MFMAs.
template <> struct Qk<kF32, kF32> {
  static constexpr int SUB = 4;
  using frag = float;
  __device__ __forceinline__ static frag kfrag(const uint4& w, int j) {
    return bits_f32(j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w);
  }
  __device__ __forceinline__ static int qdim(int c, int grp, int j) { return 16 * c + 4 * grp + j; }
  __device__ __forceinline__ static frag qload(const uint8_t* qrow, int dim) {
    return *(const float*)(qrow + 4 * dim);
  }
  __device__ __forceinline__ static frag zero() { return 0.0f; }
  __device__ __forceinline__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <int Q> struct QBytes { static constexpr int v = DtInfo<Q>::bytes; };

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// V row fragment: 8 consecutive elements (8 * bytes) of one token row.
template <int KV> struct VFrag {
  static constexpr int W = 2 * DtInfo<KV>::bytes;  // 32-bit words
  uint32_t w[W];
  template <bool NT>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int off) {
    if constexpr (W == 8) {
      uint4 a = load_kv16<NT>(r, off), b = load_kv16<NT>(r, off + 16);
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
      w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (W == 4) {
      uint4 a = load_kv16<NT>(r, off);
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else {
      uint2 a = load_kv8<NT>(r, off);
      w[0] = a.x; w[1] = a.y;
    }
  }
};

template <int KV, int D> struct ChunkRegs {
  static constexpr int ROW = D * DtInfo<KV>::bytes;
  static constexpr int NC = ROW / 64;           // 16-byte K loads per lane
  static constexpr int LPR = D / 8;             // lanes per V row
  static constexpr int RPI = 64 / LPR;          // V rows per load
  static constexpr int NV = 16 / RPI;           // V loads per lane
  uint4 k[NC];
  VFrag<KV> v[NV];
};



// ============================ fp32: VALU P.V ======================================
template <int KV, int Q, int D, int GP, bool NT>
struct ValuDecoder {
  using T = Qk<KV, Q>;
  using R = ChunkRegs<KV, D>;
  static constexpr int kDepth = 1;  // chunks whose loads are in flight ahead of the one computed
  static constexpr int EB = DtInfo<KV>::bytes;
  static constexpr int ROW = R::ROW, NC = R::NC, LPR = R::LPR, RPI = R::RPI, NV = R::NV;
  static constexpr int QB = DtInfo<Q>::bytes;
  static constexpr int NR = GP < 4 ? GP : 4;  // accumulator rows holding real heads per lane group
  using Buf = R;

  int lane, grp;
  float* lds_p;      // this wave's [16][GP] probability tile
  float* lds_alpha;  // this wave's [GP] rescale factors
  typename T::frag qf[NC * T::SUB];
  float m[NR], l[NR], lsum[NR];
  float acc[GP][8];
  float scale_l2;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* bt;
  int BS, bs_shift, Hkv, G, g, tok_end;
  int win_lo, sink_hi;  // attended: tokens >= win_lo or < sink_hi (and < tok_end)

  __device__ __forceinline__ void init(const DecodeArgs& a, float* p_tile, float* alpha_tile) {
    lane = threadIdx.x & 63;
    grp = lane >> 4;
    lds_p = p_tile;
    lds_alpha = alpha_tile;
    scale_l2 = a.scale * kLog2e;
    if constexpr (KV == kFP8) scale_l2 *= a.k_scale;
    kc = (const uint8_t*)a.k_cache;
    vc = (const uint8_t*)a.v_cache;
    BS = a.block_size;
    bs_shift = BS == 32 ? 5 : 4;  // the host admits block sizes 16 and 32
    Hkv = a.num_kv_heads;
    G = a.num_q_heads / a.num_kv_heads;
  }

  __device__ __forceinline__ void begin(const DecodeArgs& a, int s, int g_, int ctx) {
    g = g_;
    tok_end = ctx;
    win_lo = a.window > 0 ? ctx - a.window : 0;
    sink_hi = a.window > 0 ? min(a.sinks, ctx) : 0;
    bt = a.block_tables + (size_t)s * a.max_blocks_per_seq;
    const int hrow = lane & 15;
    const bool qvalid = hrow < G;
    const uint8_t* qrow = (const uint8_t*)a.q +
                          ((size_t)s * a.num_q_heads + (size_t)g * G + (qvalid ? hrow : 0)) * D * QB;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int j = 0; j < T::SUB; ++j)
        qf[c * T::SUB + j] = qvalid ? T::qload(qrow, T::qdim(c, grp, j)) : T::zero();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      m[r] = kNegInf;
      l[r] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  }

  __device__ __forceinline__ bool keep(int t) const { return t < tok_end && (t >= win_lo || t < sink_hi); }

  // Physical block of chunk c (tokens 16c ..), a scalar load: the index is uniform,
  // and the scalar path keeps table reads out of the vector-memory counter.
  __device__ __forceinline__ int table_entry(int c) const {
    const int idx = __builtin_amdgcn_readfirstlane(16 * c) >> bs_shift;
    const uint64_t p = (uint64_t)(uintptr_t)bt;
    const uint64_t pu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    return ((const __attribute__((address_space(4))) int32_t*)pu)[idx];
  }

  // live == false: a padding step past the range's end; its loads read nothing.
  __device__ __forceinline__ void load_chunk(int ct, int blk, R& buf, bool live) {
    // scalar: the chunk, its block and the head are wave-uniform (block size 16 or 32)
    const uint32_t row = (uint32_t)(__builtin_amdgcn_readfirstlane(ct) & (BS - 1));
    const size_t tile = (((size_t)(uint32_t)__builtin_amdgcn_readfirstlane(blk) * (uint32_t)Hkv +
                          (uint32_t)__builtin_amdgcn_readfirstlane(g)) * (uint32_t)BS + row) * ROW;
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kc + tile, live ? 16 * ROW : 0);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vc + tile, live ? 16 * ROW : 0);
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2)
      buf.k[c2] = load_kv16<NT>(kr, (lane & 15) * ROW + 64 * c2 + 16 * grp);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      buf.v[i].template load<NT>(vr, (i * RPI + lane / LPR) * ROW + (lane % LPR) * 8 * EB);
  }

  __device__ __forceinline__ void process_chunk(int ct, const R& buf) {
    f32x4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2)
#pragma unroll
      for (int j = 0; j < T::SUB; ++j) S = T::mma(qf[c2 * T::SUB + j], T::kfrag(buf.k[c2], j), S);
    // S[r] = score of head 4*grp + r against token ct + lane%16.
    const bool tok_ok = keep(ct + (lane & 15));
    float pr[NR], alpha[NR];
    bool changed = false;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float sc = tok_ok ? S[r] * scale_l2 : kNegInf;
      const float mn = fmaxf(m[r], row16_max(sc));
      changed |= mn > m[r];
      const float base = mn == kNegInf ? 0.0f : mn;
      alpha[r] = fast_exp2(m[r] - base);
      pr[r] = fast_exp2(sc - base);
      l[r] = l[r] * alpha[r] + pr[r];
      m[r] = mn;
    }
    const bool any_changed = __ballot(changed) != 0;
    if (4 * grp < GP) {
      float* dst = &lds_p[(lane & 15) * GP + 4 * grp];
#pragma unroll
      for (int r = 0; r < NR; ++r) dst[r] = pr[r];
      if (any_changed && (lane & 15) == 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) lds_alpha[4 * grp + r] = alpha[r];
      }
    }
    wave_lds_sync();
    if (any_changed) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float al = lds_alpha[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al;
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int t = i * RPI + lane / LPR;
      float vf[8];
      Unpack8<KV>::run(buf.v[i].w, vf);
      if (!keep(ct + t)) {  // past the context or outside the window: never let its bytes in
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = 0.0f;
      }
      const float* pp = &lds_p[t * GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float ph = pp[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(ph, vf[e], acc[h][e]);
      }
    }
    wave_lds_sync();
  }

  // Per-head denominators (uniform in each 16-lane row) and the accumulator summed
  // over the RPI row groups.
  __device__ __forceinline__ void finish() {
#pragma unroll
    for (int r = 0; r < NR; ++r) lsum[r] = row16_sum(l[r]);
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[h][e];
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
        acc[h][e] = x;
      }
  }

  __device__ __forceinline__ static float pick(const float (&x)[NR], int h) {
    float v = x[0];
#pragma unroll
    for (int r = 1; r < NR; ++r)
      if ((h & 3) == r) v = x[r];
    return bits_f32((uint32_t)__builtin_amdgcn_readlane((int)f32_bits(v), 16 * (h >> 2)));
  }
  __device__ __forceinline__ float head_m(int h) const { return pick(m, h); }
  __device__ __forceinline__ float head_l(int h) const { return pick(lsum, h); }

  // f(h, d, value) for every output element this lane owns (after finish()).
  template <class F>
  __device__ __forceinline__ void visit(F&& f) const {
    if (lane < LPR) {
#pragma unroll
      for (int h = 0; h < GP; ++h)
        if (h < G) {
#pragma unroll
          for (int e = 0; e < 8; ++e) f(h, 8 * lane + e, acc[h][e]);
        }
    }
  }
};

// ================= bf16 / f16 / fp8: MFMA Q.K^T and MFMA P.V ======================
typedef __bf16 bf16x4_t __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef _Float16 f16x4_t __attribute__((__vector_size__(4 * sizeof(_Float16))));

__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(f32_bits(x), f32_bits(x), false, false);
  return fmaxf(bits_f32(r[0]), bits_f32(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(f32_bits(x), f32_bits(x), false, false);
  return fmaxf(bits_f32(r[0]), bits_f32(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(f32_bits(x), f32_bits(x), false, false);
  return bits_f32(r[0]) + bits_f32(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(f32_bits(x), f32_bits(x), false, false);
  return bits_f32(r[0]) + bits_f32(r[1]);
}

// P.V operand handling per cache dtype.  A fragment: 4 16-bit elements (two words),
// element (lane & 3) holds the probability, the others zero.  The element is placed by
// two byte permutes whose selectors (s0, s1: one per word, fixed per lane) take the
// 16-bit value from bytes kSrc of a 32-bit source and zero the rest.
template <int KV> struct Pv;
template <> struct Pv<kBF16> {
  static constexpr bool kSplit = true;
  static constexpr uint32_t kSrc = 0x0302u;  // the upper half of fp32 bits
  using frag = bf16x4_t;
  // V: two 32-bit words = 4 bf16
  __device__ __forceinline__ static frag vfrag(const uint32_t* w, int half) {
    return __builtin_bit_cast(frag, make_uint2(w[2 * half], w[2 * half + 1]));
  }
  // p = hi + lo, hi the upper half of p's fp32 bits, lo the bf16 truncation of the rest.
  __device__ __forceinline__ static void pfrag(float p, uint32_t s0, uint32_t s1, frag& hi, frag& lo) {
    const uint32_t pb = f32_bits(p);
    const uint32_t rb = f32_bits(p - bits_f32(pb & 0xffff0000u));
    hi = __builtin_bit_cast(frag, make_uint2(__builtin_amdgcn_perm(0u, pb, s0), __builtin_amdgcn_perm(0u, pb, s1)));
    lo = __builtin_bit_cast(frag, make_uint2(__builtin_amdgcn_perm(0u, rb, s0), __builtin_amdgcn_perm(0u, rb, s1)));
  }
  __device__ __forceinline__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};
template <> struct Pv<kF16> {
  static constexpr bool kSplit = true;
  static constexpr uint32_t kSrc = 0x0100u;  // an f16 value in the low half
  using frag = f16x4_t;
  __device__ __forceinline__ static frag vfrag(const uint32_t* w, int half) {
    return __builtin_bit_cast(frag, make_uint2(w[2 * half], w[2 * half + 1]));
  }
  __device__ __forceinline__ static void pfrag(float p, uint32_t s0, uint32_t s1, frag& hi, frag& lo) {
    const _Float16 h = (_Float16)p;
    const _Float16 r = (_Float16)(p - (float)h);
    const uint32_t hb = __builtin_bit_cast(uint16_t, h), rb = __builtin_bit_cast(uint16_t, r);
    hi = __builtin_bit_cast(frag, make_uint2(__builtin_amdgcn_perm(0u, hb, s0), __builtin_amdgcn_perm(0u, hb, s1)));
    lo = __builtin_bit_cast(frag, make_uint2(__builtin_amdgcn_perm(0u, rb, s0), __builtin_amdgcn_perm(0u, rb, s1)));
  }
  __device__ __forceinline__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Pv<kFP8> {
  static constexpr bool kSplit = false;
  static constexpr uint32_t kSrc = 0x0100u;
  using frag = f16x4_t;
  // V: one 32-bit word = 4 e4m3fn codes, converted exactly to f16.
  __device__ __forceinline__ static frag vfrag(const uint32_t* w, int half) {
    const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[half], 1.0f, false);
    const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[half], 1.0f, true);
    frag r = {a[0], a[1], b[0], b[1]};
    return r;
  }
  __device__ __forceinline__ static void pfrag(float p, uint32_t s0, uint32_t s1, frag& hi, frag&) {
    const uint32_t hb = __builtin_bit_cast(uint16_t, (_Float16)p);
    hi = __builtin_bit_cast(frag, make_uint2(__builtin_amdgcn_perm(0u, hb, s0), __builtin_amdgcn_perm(0u, hb, s1)));
  }
  __device__ __forceinline__ static f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};

constexpr float kDecodeSlack = 8.0f;  // log2 units: decode weights stay <= 2^8 between rescales

template <int KV, int D> struct MfmaChunk {
  static constexpr int EB = DtInfo<KV>::bytes;
  static constexpr int ROW = D * EB;
  static constexpr int NC = ROW / 64;               // 16-byte K loads per lane
  static constexpr int VBYTES = (D / 16) * EB;       // bytes of one V row per lane
  static constexpr int VW = VBYTES / 4;             // 32-bit words of it
  uint4 k[NC];
  uint32_t v[4][VW];
};

template <int KV, int Q, int D, int GP, bool NT>
struct MfmaDecoder {
  using T = Qk<KV, Q>;
  using P = Pv<KV>;
  using Buf = MfmaChunk<KV, D>;
  // Chunks whose loads are in flight ahead of the one computed: one for 16-bit caches,
  // two for fp8 (half the bytes per chunk).  (Three for fp8 -- as many bytes in flight as
  // the 16-bit decoder -- measured 12 % slower on the 70B-shaped workload, and
  // pushed its 8-head decoder past 256 VGPRs.)
  static constexpr int kDepth = KV == kFP8 ? 2 : 1;
  static constexpr int EB = DtInfo<KV>::bytes;
  static constexpr int ROW = Buf::ROW, NC = Buf::NC, VW = Buf::VW, VBYTES = Buf::VBYTES;
  static constexpr int QB = DtInfo<Q>::bytes;
  static constexpr int HS = GP < 4 ? 1 : GP / 4;  // head sets of 4
  static constexpr int HALVES = D / 64;           // 16x16x16 P.V tiles per 4-token step

  int lane;
  typename T::frag qf[HS][NC * T::SUB];
  float m[HS], l[HS], lfin[HS];
  f32x4_t acc[HS][HALVES];
  // Scores are taken raw (S = K Q^T) and scaled inside the exponent, 2^(c s - m) with
  // c = |scale| log2(e) (x |k_scale| for fp8) > 0, so that the maximum can be taken on
  // raw scores: a negative scale flips the sign of Q instead (exact), a zero one zeroes
  // Q (all scores 0: uniform weights).
  float c_l2;
  uint32_t qflip;
  bool qzero;
  uint32_t psel0, psel1;  // P fragment placement (Pv::pfrag)
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* bt;
  int BS, bs_shift, Hkv, G, g, tok_end;
  int win_lo, sink_hi;  // attended: tokens >= win_lo or < sink_hi (and < tok_end)

  __device__ __forceinline__ void init(const DecodeArgs& a, float*, float*) {
    lane = threadIdx.x & 63;
    float ks = 1.0f;
    if constexpr (KV == kFP8) ks = a.k_scale;
    qflip = (a.scale < 0.0f) != (ks < 0.0f) ? 0x80008000u : 0u;
    qzero = a.scale == 0.0f || ks == 0.0f;
    c_l2 = (a.scale != 0.0f ? __builtin_fabsf(a.scale) : 1.0f) * kLog2e * (ks != 0.0f ? __builtin_fabsf(ks) : 1.0f);
    // element lane & 3 of the P fragment: word (lane & 3) / 2, half (lane & 1)
    const uint32_t pat = (lane & 1) ? ((P::kSrc << 16) | 0x0c0cu) : (0x0c0c0000u | P::kSrc);
    psel0 = (lane & 2) ? 0x0c0c0c0cu : pat;
    psel1 = (lane & 2) ? pat : 0x0c0c0c0cu;
    kc = (const uint8_t*)a.k_cache;
    vc = (const uint8_t*)a.v_cache;
    BS = a.block_size;
    bs_shift = BS == 32 ? 5 : 4;  // the host admits block sizes 16 and 32
    Hkv = a.num_kv_heads;
    G = a.num_q_heads / a.num_kv_heads;
  }

  __device__ __forceinline__ void begin(const DecodeArgs& a, int s, int g_, int ctx) {
    g = g_;
    tok_end = ctx;
    win_lo = a.window > 0 ? ctx - a.window : 0;
    sink_hi = a.window > 0 ? min(a.sinks, ctx) : 0;
    bt = a.block_tables + (size_t)s * a.max_blocks_per_seq;
    const int grp = lane >> 4;
    const uint8_t* qbase = (const uint8_t*)a.q + ((size_t)s * a.num_q_heads + (size_t)g * G) * D * QB;
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
      const int h = 4 * hs + ((lane & 15) >> 2);  // B-operand column l%16 -> head (l%16)/4
      const bool qvalid = h < G;
      const uint8_t* qrow = qbase + (size_t)(qvalid ? h : 0) * D * QB;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < T::SUB; ++j) {
          typename T::frag f = T::zero();
          if (qvalid && !qzero) {
            const uint4 w = __builtin_bit_cast(uint4, T::qload(qrow, T::qdim(c, grp, j)));
            f = __builtin_bit_cast(typename T::frag, make_uint4(w.x ^ qflip, w.y ^ qflip, w.z ^ qflip, w.w ^ qflip));
          }
          qf[hs][c * T::SUB + j] = f;
        }
      m[hs] = kNegInf;
      l[hs] = 0.0f;
#pragma unroll
      for (int hf = 0; hf < HALVES; ++hf) acc[hs][hf] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  __device__ __forceinline__ bool keep(int t) const { return t < tok_end && (t >= win_lo || t < sink_hi); }

  __device__ __forceinline__ int table_entry(int c) const {
    const int idx = __builtin_amdgcn_readfirstlane(16 * c) >> bs_shift;
    const uint64_t p = (uint64_t)(uintptr_t)bt;
    const uint64_t pu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    return ((const __attribute__((address_space(4))) int32_t*)pu)[idx];
  }

  // live == false: a padding step past the range's end; its loads read nothing.  The
  // resources cover only the chunk's rows before the context's end, so the rows past it
  // (the tail of the last block: any bytes, NaN included) load as zeros: their scores
  // are masked and their zero V rows cannot spoil the P.V products.  Rows outside a
  // window but inside a chunk that holds attended tokens are tokens written earlier,
  // in a block that is still live: only their scores need masking.
  __device__ __forceinline__ void load_chunk(int ct, int blk, Buf& buf, bool live) {
    // scalar: the chunk, its block and the head are wave-uniform (block size 16 or 32)
    const int ctu = __builtin_amdgcn_readfirstlane(ct);
    const uint32_t row = (uint32_t)(ctu & (BS - 1));
    const size_t tile = (((size_t)(uint32_t)__builtin_amdgcn_readfirstlane(blk) * (uint32_t)Hkv +
                          (uint32_t)__builtin_amdgcn_readfirstlane(g)) * (uint32_t)BS + row) * ROW;
    const int rows = live ? min(16, __builtin_amdgcn_readfirstlane(tok_end) - ctu) : 0;
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kc + tile, rows * ROW);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vc + tile, rows * ROW);
    const int krow = 4 * (lane & 3) + ((lane & 15) >> 2);  // A-operand row l%16 -> token
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2)
      buf.k[c2] = load_kv16<NT>(kr, krow * ROW + 64 * c2 + 16 * (lane >> 4));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int off = (4 * k + (lane >> 4)) * ROW + (lane & 15) * VBYTES;
      if constexpr (VW == 4) {
        const uint4 x = load_kv16<NT>(vr, off);
        buf.v[k][0] = x.x; buf.v[k][1] = x.y; buf.v[k][2] = x.z; buf.v[k][3] = x.w;
      } else if constexpr (VW == 2) {
        const uint2 x = load_kv8<NT>(vr, off);
        buf.v[k][0] = x.x; buf.v[k][1] = x.y;
      } else {
        buf.v[k][0] = load_kv4<NT>(vr, off);
      }
    }
  }

  __device__ __forceinline__ void process_chunk(int ct, Buf& buf) {
    // ---- Q.K^T: S[hs][k] = score(head 4hs + (l%16)/4, token ct + 4k + l/16)
    f32x4_t S[HS];
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) S[hs] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2)
#pragma unroll
      for (int j = 0; j < T::SUB; ++j) {
        const auto kf = T::kfrag(buf.k[c2], j);
#pragma unroll
        for (int hs = 0; hs < HS; ++hs) S[hs] = T::mma(kf, qf[hs][c2 * T::SUB + j], S[hs]);
      }
    const int tb = ct + (lane >> 4);
    // ---- online softmax, one head per lane (duplicated over lane & 3).  Lazy
    // rescaling: the reference max m moves only when a score exceeds it by more than
    // kDecodeSlack (or on the first attended token), so weights 2^(c s - m) stay <= 2^8
    // and the rescale of l and acc is rare; (m, l, acc) stay one consistent partial.
    float p[HS][4], alpha[HS];
    bool moved = false;
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
      float s[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) s[k] = keep(tb + 4 * k) ? S[hs][k] : kNegInf;
      float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      bm = xor32_max(xor16_max(bm)) * c_l2;
      const bool mv = bm > m[hs] + kDecodeSlack;
      moved |= mv;
      const float mn = mv ? bm : m[hs];
      const float base = mn == kNegInf ? 0.0f : mn;
      alpha[hs] = fast_exp2(m[hs] - base);  // 1 unless m moved (0 from -inf)
#pragma unroll
      for (int k = 0; k < 4; ++k) p[hs][k] = fast_exp2(__builtin_fmaf(s[k], c_l2, -base));
      l[hs] = l[hs] * alpha[hs] + ((p[hs][0] + p[hs][1]) + (p[hs][2] + p[hs][3]));
      m[hs] = mn;
    }
    if (__ballot(moved) != 0) {
      // the accumulator of lane l belongs to head 4hs + l/16, whose factor lane 4(l/16) holds
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) {
        const float al = __shfl(alpha[hs], 4 * (lane >> 4));
#pragma unroll
        for (int hf = 0; hf < HALVES; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[hs][hf][r] *= al;
      }
    }
    // ---- P.V
    // A chunk holding tokens between the sinks and the window start (wave-uniform test:
    // only the chunks at those two edges): their weights are zero, but a zero weight
    // times a non-finite V element is NaN on the matrix cores, and the definition leaves
    // those tokens out entirely, so their V fragments are replaced by zeros.
    const bool gap = win_lo > sink_hi && ct < win_lo && ct + 16 > sink_hi;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      typename P::frag vf[HALVES];
#pragma unroll
      for (int hf = 0; hf < HALVES; ++hf) vf[hf] = P::vfrag(buf.v[k], hf);
      if (gap) {
        const int t = tb + 4 * k;
        if (t >= sink_hi && t < win_lo) {
#pragma unroll
          for (int hf = 0; hf < HALVES; ++hf) vf[hf] = typename P::frag{};
        }
      }
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) {
        typename P::frag ahi, alo;
        P::pfrag(p[hs][k], psel0, psel1, ahi, alo);
#pragma unroll
        for (int hf = 0; hf < HALVES; ++hf) {
          acc[hs][hf] = P::mma(ahi, vf[hf], acc[hs][hf]);
          if constexpr (P::kSplit) acc[hs][hf] = P::mma(alo, vf[hf], acc[hs][hf]);
        }
      }
    }
  }

  __device__ __forceinline__ void finish() {
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) lfin[hs] = xor32_sum(xor16_sum(l[hs]));
  }
  // head h's values live in the lanes with (l%16)/4 == h%4
  __device__ __forceinline__ float head_m(int h) const {
    float v = m[0];
#pragma unroll
    for (int hs = 1; hs < HS; ++hs)
      if ((h >> 2) == hs) v = m[hs];
    return bits_f32((uint32_t)__builtin_amdgcn_readlane((int)f32_bits(v), 4 * (h & 3)));
  }
  __device__ __forceinline__ float head_l(int h) const {
    float v = lfin[0];
#pragma unroll
    for (int hs = 1; hs < HS; ++hs)
      if ((h >> 2) == hs) v = lfin[hs];
    return bits_f32((uint32_t)__builtin_amdgcn_readlane((int)f32_bits(v), 4 * (h & 3)));
  }
  template <class F>
  __device__ __forceinline__ void visit(F&& f) const {
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
      const int h = 4 * hs + (lane >> 4);
      if (h < G) {
#pragma unroll
        for (int hf = 0; hf < HALVES; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r) f(h, (D / 16) * (lane & 15) + 4 * hf + r, acc[hs][hf][r]);
      }
    }
  }
};

template <int KV, int Q, int D, int GP, bool NT>
using Decoder = typename std::conditional<KV == kF32, ValuDecoder<KV, Q, D, GP, NT>,
                                          MfmaDecoder<KV, Q, D, GP, NT>>::type;

// The 16-token chunks of a ctx-token context that hold attended tokens: [0, a) and
// [b, nc) with a <= b, nc = ceil(ctx / 16).  Without a window (window == 0) or when the
// window reaches back to the sink tokens, one range: a = b = nc.  With a window, the
// sink chunks [0, ceil(min(sinks, ctx) / 16)) and the window chunks from
// floor((ctx - window) / 16) ("PagedAttention por dentro...", sections "Sliding window
// attention" and "StreamingLLM...: los attention sinks": the last K tokens plus the
// first few).  Chunks in the gap are never read: their blocks may have been freed.
__device__ __forceinline__ void attended_chunks(int ctx, int window, int sinks, int& a, int& b) {
  const int nc = (ctx + 15) >> 4;
  a = nc;
  b = nc;
  if (window > 0 && ctx - window > 0) {
    const int sa = (min(sinks, ctx) + 15) >> 4;
    const int wb = (ctx - window) >> 4;
    if (sa < wb) {
      a = sa;
      b = wb;
    }
  }
}
// Attended chunks of a context, counted without the gap.
__device__ __forceinline__ int attended_chunk_count(int ctx, int window, int sinks) {
  int a, b;
  attended_chunks(ctx, window, sinks, a, b);
  return a + ((ctx + 15) >> 4) - b;
}

// Chunks c_begin, c_begin + step, ... < c_end (chunk c covers tokens 16c .. 16c+15),
// with the loads of the next W::kDepth chunks in flight while one is computed
// (kDepth + 1 register buffers, rotated by a fully unrolled inner loop).  Every step
// issues its loads unconditionally -- past the end as padding loads through an empty
// buffer resource, which read nothing -- so the vector-memory wait before a chunk's
// use only covers that chunk's own loads, never the ones issued after it.
// Block-table entries come one chunk ahead through the scalar path.
//
// The range is in gap-free chunk numbers v (see attended_chunks): chunk v + shift is
// read when v >= split, chunk v otherwise.
template <class W>
__device__ __forceinline__ void run_chunks(W& wd, int c_begin, int c_end, int step, int split = 0x7fffffff,
                                           int shift = 0) {
  constexpr int DEPTH = W::kDepth;
  // wave-uniform by construction; said so, so that the chunk and address arithmetic stays
  // scalar (in vector registers it had competed with the in-flight loads for registers,
  // and the compiler then drained every load at the top of the loop)
  c_begin = __builtin_amdgcn_readfirstlane(c_begin);
  c_end = __builtin_amdgcn_readfirstlane(c_end);
  step = __builtin_amdgcn_readfirstlane(step);
  split = __builtin_amdgcn_readfirstlane(split);
  shift = __builtin_amdgcn_readfirstlane(shift);
  if (c_begin >= c_end) return;
  const int n = (c_end - c_begin + step - 1) / step;  // chunks of this wave
  auto chunk = [&](int i) {
    const int v = c_begin + (i < n ? i : n - 1) * step;
    return v >= split ? v + shift : v;
  };
  typename W::Buf buf[DEPTH + 1];
  int blk = wd.table_entry(chunk(0));
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) {
    wd.load_chunk(16 * chunk(j), blk, buf[j], j < n);
    blk = wd.table_entry(chunk(j + 1));
  }
  // Whole rounds of DEPTH + 1 chunks, with no exit inside a round (an exit there made
  // the compiler copy the in-flight buffers at the loop edge and wait for their loads),
  // then the last n mod (DEPTH + 1) chunks, already loaded in buf[0 ..].
  const int full = n - n % (DEPTH + 1);
  for (int i = 0; i < full; i += DEPTH + 1) {
#pragma unroll
    for (int u = 0; u <= DEPTH; ++u) {
      const int ii = i + u;
      wd.load_chunk(16 * chunk(ii + DEPTH), blk, buf[(u + DEPTH) % (DEPTH + 1)], ii + DEPTH < n);
      blk = wd.table_entry(chunk(ii + DEPTH + 1));
      wd.process_chunk(16 * chunk(ii), buf[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < DEPTH; ++u)
    if (full + u < n) wd.process_chunk(16 * chunk(full + u), buf[u]);
}

// Log-sum-exp merge of P partial results of one query head (the online-softmax
// algebra: M = max_p m_p, out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p),
// by one workgroup of kMergeThreads threads: thread t handles output dim t % D for
// the partials p = t / D, t / D + PG, ...; the PG groups are combined in LDS.  One
// pass with a running maximum (each partial rescales the running sums when it raises
// it); a thread's partials are read in batches of kMergeBatch, so it waits for memory
// once per batch.  part(p) returns the partial's (m, l, acc-row) pointers.  vnorm
// scales the result (the fp8 V scale).  Writes out[row + d].
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 32;  // 64 partitions of 128 dims: one batch per thread
__device__ __forceinline__ void lse_add(float& M, float& L, float& A, float m, float l, float x) {
  const float Mn = fmaxf(M, m);
  const float base = Mn == kNegInf ? 0.0f : Mn;
  const float fo = fast_exp2(M - base), fn = fast_exp2(m - base);
  L = L * fo + l * fn;
  A = A * fo + x * fn;
  M = Mn;
}
template <int D, class PartFn>
__device__ __forceinline__ void merge_head(int P, PartFn part, void* out, size_t row, int out_dtype,
                                           float vnorm) {
  constexpr int PG = kMergeThreads / D;
  __shared__ float red_m[PG], red_l[PG], red_a[PG][D];
  const int t = threadIdx.x, d = t % D, pg = t / D;
  float M = kNegInf, L = 0.0f, A = 0.0f;
  for (int p0 = pg; p0 < P; p0 += PG * kMergeBatch) {
    float pm[kMergeBatch], pl[kMergeBatch], pa[kMergeBatch];
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      const int p = p0 + b * PG;
      const auto q = part(p < P ? p : p0);
      pm[b] = p < P ? *q.m : kNegInf;  // past the last partial: weighs nothing
      pl[b] = *q.l;
      pa[b] = q.acc[d];
    }
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) lse_add(M, L, A, pm[b], pl[b], pa[b]);
  }
  red_a[pg][d] = A;
  if (d == 0) {
    red_m[pg] = M;
    red_l[pg] = L;
  }
  __syncthreads();
  if (pg == 0) {
    float MM = kNegInf, LL = 0.0f, AA = 0.0f;
#pragma unroll
    for (int j = 0; j < PG; ++j) lse_add(MM, LL, AA, red_m[j], red_l[j], red_a[j][d]);
    store_out(out, row + d, out_dtype, LL != 0.0f ? AA / LL * vnorm : 0.0f);
  }
}

struct PartialRef {
  const float* m;
  const float* l;
  const float* acc;
};

}  // namespace pkv
