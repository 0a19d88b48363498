// Paged decode attention for gfx950, with the split-context log-sum-exp merge.
//
// What is computed: for each sequence s and query head h,
//   out[s][h] = softmax_t(scale * q[s][h] . K_t) V_t,  t = 0 .. ctx[s]-1,
// K_t / V_t of KV head h / G, found through the block table ("Capitulo 2", section
// "Que guarda realmente el KV cache"; "Optimizacion de Inferencia LLM", section
// "El Cuello de Botella..."), accumulated block by block with the online-softmax
// rescaling of "Optimizacion de Inferencia LLM", sections "PagedAttention:
// Conceptos de SO..." (kernel pseudocode) and "FlashAttention-3..." (accumulate
// with rescaling, write O once).
//
// Work decomposition (gfx950, wave64):
//   * one workgroup of NW waves per (partition, KV head, sequence); the workgroup
//     serves all G query heads of its KV head from one pass over the blocks;
//   * the partition is cut into 16-token chunks (a 16-token block, or half of a
//     32-token block) dealt round-robin to the waves;
//   * per chunk, Q.K^T is one 16x16 MFMA tile (rows = the G query heads, padded
//     to 16; columns = the 16 tokens).  Each lane's 16-byte K load is directly an
//     MFMA B-operand fragment: lane l reads token l%16, bytes 64c + 16(l/16) of the
//     row, so the four lane groups cover 64 contiguous bytes of every row per load;
//   * the online softmax runs on the MFMA accumulator layout (lane l holds heads
//     4(l/16)+r of token l%16): a 16-lane DPP reduction gives each head's chunk max;
//   * P.V runs on the VALU in fp32: lane l owns 8 consecutive dims of one token row
//     per load (D/8 lanes per row), probabilities come from LDS;
//   * the next chunk's K and V are in flight while the current one is computed;
//   * at the end the waves are merged through LDS; in split mode the workgroup
//     stores (max, denominator, unnormalised output) and merge_kernel combines the
//     partitions of each (sequence, query head).
#include <hip/hip_runtime.h>
#include <stdint.h>

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

__device__ __forceinline__ void store_out(void* out, size_t idx, int out_dtype, float x) {
  if (out_dtype == kF32)
    ((float*)out)[idx] = x;
  else if (out_dtype == kBF16)
    ((uint16_t*)out)[idx] = f32_to_bf16_rne(x);
  else
    ((uint16_t*)out)[idx] = f32_to_f16_rne(x);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// V row fragment: 8 consecutive elements (8 * bytes) of one token row.
template <int KV> struct VFrag {
  static constexpr int W = 2 * DtInfo<KV>::bytes;  // 32-bit words
  uint32_t w[W];
  __device__ __forceinline__ void load(const uint8_t* p) {
    if constexpr (W == 8) {
      uint4 a = *(const uint4*)p, b = *(const uint4*)(p + 16);
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
      w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (W == 4) {
      uint4 a = *(const uint4*)p;
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else {
      uint2 a = *(const uint2*)p;
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

template <int KV, int Q, int D, int GP, int NW>
__global__ void __launch_bounds__(64 * NW)
decode_kernel(const DecodeArgs a) {
  using T = Qk<KV, Q>;
  using R = ChunkRegs<KV, D>;
  constexpr int EB = DtInfo<KV>::bytes;
  constexpr int ROW = R::ROW, NC = R::NC, LPR = R::LPR, RPI = R::RPI, NV = R::NV;
  constexpr int QB = QBytes<Q>::v;
  constexpr int NR = GP < 4 ? GP : 4;  // accumulator rows holding real heads per lane group

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
  const int nchunks = tok_end > tok_begin ? (tok_end - tok_begin + 15) >> 4 : 0;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int BS = a.block_size;
  const int Hkv = a.num_kv_heads;

  // Query fragments (MFMA A operand): row = head lane%16, dims matching the K loads.
  const int hrow = lane & 15, grp = lane >> 4;
  const bool qvalid = hrow < G;
  const uint8_t* qrow = (const uint8_t*)a.q +
                        ((size_t)s * a.num_q_heads + (size_t)g * G + (qvalid ? hrow : 0)) * D * QB;
  typename T::frag qf[NC * T::SUB];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int j = 0; j < T::SUB; ++j)
      qf[c * T::SUB + j] = qvalid ? T::qload(qrow, T::qdim(c, grp, j)) : T::zero();

  float scale_l2 = a.scale * kLog2e;
  float vnorm = 1.0f;
  if constexpr (KV == kFP8) {
    scale_l2 *= a.k_scale;
    vnorm = a.v_scale;
  }

  float m[NR], l[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    m[r] = kNegInf;
    l[r] = 0.0f;
  }
  float acc[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;

  // Block-table window: lane j holds entry win_base + j (uniform base).
  const int32_t* bt = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const int nblk_end = (tok_end + BS - 1) / BS;  // entries past this are never read
  int win_base = -(1 << 30);
  int win_reg = 0;
  const uint8_t* kc = (const uint8_t*)a.k_cache;
  const uint8_t* vc = (const uint8_t*)a.v_cache;

  auto load_chunk = [&](int c, R& buf) {
    const int ct = tok_begin + 16 * c;
    const int lb = ct / BS;
    const int off0 = ct - lb * BS;
    if (lb >= win_base + 64 || lb < win_base) {
      win_base = lb;
      const int idx = lb + lane;
      win_reg = idx < nblk_end ? bt[idx] : 0;
    }
    const int blk = __builtin_amdgcn_readlane(win_reg, lb - win_base);
    const size_t tile = (((size_t)blk * Hkv + g) * BS + off0) * ROW;
    const uint8_t* kt = kc + tile;
    const uint8_t* vt = vc + tile;
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2)
      buf.k[c2] = *(const uint4*)(kt + (lane & 15) * ROW + 64 * c2 + 16 * grp);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      buf.v[i].load(vt + (i * RPI + lane / LPR) * ROW + (lane % LPR) * 8 * EB);
  };

  auto process_chunk = [&](int c, const R& buf) {
    const int ct = tok_begin + 16 * c;
    f32x4_t S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2)
#pragma unroll
      for (int j = 0; j < T::SUB; ++j) S = T::mma(qf[c2 * T::SUB + j], T::kfrag(buf.k[c2], j), S);

    // S[r] = score of head 4*grp + r against token ct + lane%16.
    const bool tok_ok = ct + (lane & 15) < tok_end;
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

    // Publish this chunk's probabilities [token][head] (and the rescale factors).
    if (4 * grp < GP) {
      float* dst = &lds_p[wv][(lane & 15) * GP + 4 * grp];
#pragma unroll
      for (int r = 0; r < NR; ++r) dst[r] = pr[r];
      if (any_changed && (lane & 15) == 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) lds_alpha[wv][4 * grp + r] = alpha[r];
      }
    }
    wave_lds_sync();

    if (any_changed) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float al = lds_alpha[wv][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al;
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int t = i * RPI + lane / LPR;
      float vf[8];
      Unpack8<KV>::run(buf.v[i].w, vf);
      if (ct + t >= tok_end) {  // tail of the last block: never let its bytes in
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = 0.0f;
      }
      const float* pp = &lds_p[wv][t * GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        const float ph = pp[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(ph, vf[e], acc[h][e]);
      }
    }
    wave_lds_sync();
  };

  // Software pipeline: the next chunk of this wave is loading while one computes.
  R buf0, buf1;
  int c = wv;
  if (c < nchunks) load_chunk(c, buf0);
  for (; c < nchunks; c += 2 * NW) {
    if (c + NW < nchunks) load_chunk(c + NW, buf1);
    process_chunk(c, buf0);
    if (c + NW >= nchunks) break;
    if (c + 2 * NW < nchunks) load_chunk(c + 2 * NW, buf0);
    process_chunk(c + NW, buf1);
  }

  // ---- wave results -> LDS ----
  float lsum[NR];
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
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float* dst = &lds_acc[wv][h * D + 8 * lane];
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = acc[h][e];
    }
  }
  if ((lane & 15) == 0 && 4 * grp < GP) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      lds_m[wv][4 * grp + r] = m[r];
      lds_l[wv][4 * grp + r] = lsum[r];
    }
  }
  __syncthreads();

  // ---- merge the waves; write the output (single pass) or the partition's partials ----
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
      store_out(a.out, hq * D + d, a.out_dtype, L > 0.0f ? A / L * vnorm : 0.0f);
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

// Log-sum-exp merge of the partitions of one (sequence, query head):
//   M = max_p m_p;  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// (the same rescaling algebra as the online softmax).  Partitions at or past the
// sequence's context were never written and are not read.
template <int D, int KV>
__global__ void __launch_bounds__(D) merge_kernel(const DecodeArgs a) {
  const int hq = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int ctx = a.context_lens[s];
  const int np = (ctx + a.partition - 1) / a.partition;
  const size_t base = ((size_t)s * a.num_q_heads + hq) * a.num_partitions;
  float M = kNegInf;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.ws_m[base + p]);
  float L = 0.0f, A = 0.0f;
  if (M != kNegInf) {
    for (int p = 0; p < np; ++p) {
      const float f = fast_exp2(a.ws_m[base + p] - M);
      L += f * a.ws_l[base + p];
      A += f * a.ws_acc[(base + p) * D + d];
    }
  }
  const float vnorm = KV == kFP8 ? a.v_scale : 1.0f;
  store_out(a.out, ((size_t)s * a.num_q_heads + hq) * D + d, a.out_dtype,
            L > 0.0f ? A / L * vnorm : 0.0f);
}

// ---- dispatch --------------------------------------------------------------------
constexpr int kWaves = 4;

template <int KV, int Q, int D, int GP>
static hipError_t launch_gp(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.num_partitions, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_kernel<KV, Q, D, GP, kWaves>), grid, dim3(64 * kWaves), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions == 1) return e;
  hipLaunchKernelGGL((merge_kernel<D, KV>), dim3(a.num_q_heads, a.num_seqs), dim3(D), 0, stream, a);
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
