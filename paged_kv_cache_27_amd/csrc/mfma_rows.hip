// Attention of many query rows against one paged token range, on the matrix cores
// (gfx950).  Two uses:
//
// Shared-prefix decode (the prefix half of cascade attention).  With prefix caching
// several sequences map their first blocks to the same physical blocks ("La despensa
// por casilleros", section "Prefix caching: compartir casilleros con copy-on-write";
// "PagedAttention por dentro...", section "Prefix caching cross-session").  Attention over those
// shared tokens is the same matrix product for every sequence of the group, so it is
// computed once for all of them: the queries of the group's sequences (for one KV head:
// n_seqs x G rows) are the rows of S = Q K^T, P = online-softmax(S), O = P V over the
// prefix tokens, and each row leaves a partial result (running max m in the log2
// domain, denominator l, unnormalised output acc) that the suffix pass merges with the
// sequence's own tokens by the log-sum-exp algebra of the online softmax ("Optimizacion
// de Inferencia LLM", sections "PagedAttention: Conceptos de SO..." and
// "FlashAttention-3...").
//
// Chunked prefill.  A sequence brings a chunk of n query tokens, the last n of its
// context (their K/V already written); query i, at position ctx - n + i, attends to
// tokens 0 .. ctx - n + i of the paged cache ("PagedAttention por dentro...", section
// "Chunked prefill integrado con paged KV"; "Componentes Internos de Servicio de vLLM",
// section "Chunked prefill protege la cola del TTFT").  The rows are (query token,
// query head) of one sequence and KV head, each with its own causal limit, and the
// workgroup writes the normalised output.
//
// One workgroup = 4 waves x 2 sets of 16 query rows, over a range of the 16-token
// chunks, taken two at a time (32-token steps).  Per step, wave and row set, on the
// matrix cores:
//   * S^T = K Q^T per chunk: 16x16x32 MFMAs, A = the chunk's K rows as staged (lane l:
//     token l%16, 8 dims; one LDS read serves both sets), B = the set's 16 query rows;
//     lane l gets row l%16 against tokens 4(l/16) .. 4(l/16)+3 of each chunk;
//   * those 8 probabilities are exactly lane l's A operand of a 16x16x32 P.V MFMA (row
//     l%16, k-slots 8(l/16) .. +7 standing for tokens 4(l/16)+i of both chunks), so P
//     never leaves registers (split hi + lo in 16 bits, ~16 bits of each probability
//     kept);
//   * V's B operand needs those 8 tokens of one dim per lane: the workgroup stages each
//     step's V once in LDS as [lane group][dim][8 tokens], so a lane's fragment is one
//     conflict-free 16-byte LDS read (again serving both sets);
//   * the row sums come from the same weights in fp32, on the VALU: each lane adds its 8
//     weights of row l%16 into a running share (rescaled with the row), and the four lane
//     groups' shares are summed once at the end.  (As P times a tile of ones on the
//     matrix cores -- two more MFMAs per row set and step -- prefill over a 16-bit cache
//     measured ~1-2 % slower.)  Prefill over an fp8 cache keeps the ones tile: there the
//     VALU sums cost the registers of a third wave per SIMD (174 against 167 VGPRs), and
//     it measured 4 % slower with them.
// Two row sets per wave halve the LDS reads, staging and barriers per MFMA against one
// set, and give each wave two independent softmax chains (measured 9% faster on the
// chunked-prefill workload at ~170 VGPRs, two waves per SIMD, than one set at ~110 VGPRs
// and four waves per SIMD).
// K is staged in LDS as [32 tokens][d_h + 8] (the padding puts a wave's 16-byte
// A-fragment reads in distinct banks); the next step's loads are in flight in registers
// while one is computed.  Workgroups of one KV head are numbered so that they share an
// XCD (workgroup i runs on XCD i mod 8 when the KV head count is a multiple of 8),
// keeping the head's K/V tiles in that L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

template <int KV> struct PfxOps;
// split2(p0, p1, hi, lo): two probabilities as 16-bit pairs (p0 in the low half) with
// p = hi + lo to ~16 significant bits; kOne: 1.0 in both halves.
template <> struct PfxOps<kBF16> {
  using frag8 = bf16x8_t;
  static constexpr uint32_t kOne = 0x3f803f80u;
  // four e4m3fn codes -> four bf16 (exact), as two words of two
  __device__ __forceinline__ static uint2 from_fp8(uint32_t w) {
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true)));
  }
  __device__ __forceinline__ static f32x4_t qk(frag8 a, frag8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // hi: the upper halves of the fp32 bits; lo: the upper half of what remains
  __device__ __forceinline__ static void split2(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    const uint32_t b0 = f32_bits(p0), b1 = f32_bits(p1);
    hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
    const float r0 = p0 - bits_f32(b0 & 0xffff0000u), r1 = p1 - bits_f32(b1 & 0xffff0000u);
    lo = __builtin_amdgcn_perm(f32_bits(r1), f32_bits(r0), 0x07060302u);
  }
};
template <> struct PfxOps<kF16> {
  using frag8 = f16x8_t;
  static constexpr uint32_t kOne = 0x3c003c00u;
  __device__ __forceinline__ static uint2 from_fp8(uint32_t w) {  // e4m3fn -> f16 is exact too
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true)));
  }
  __device__ __forceinline__ static f32x4_t qk(frag8 a, frag8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // hi rounded toward zero to f16, lo the rest (also f16)
  __device__ __forceinline__ static void split2(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    const auto h = __builtin_amdgcn_cvt_pkrtz(p0, p1);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0 - (float)h[0], p1 - (float)h[1]));
  }
};

// NaN-propagating maximum (v_maximum3_f32 on gfx950: no operand canonicalisation, and
// three inputs per instruction); scores here are finite or -inf.
__device__ __forceinline__ float pf_max(float x, float y) { return __builtin_elementwise_maximum(x, y); }
__device__ __forceinline__ float pf_xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(f32_bits(x), f32_bits(x), false, false);
  return pf_max(bits_f32(r[0]), bits_f32(r[1]));
}
__device__ __forceinline__ float pf_xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(f32_bits(x), f32_bits(x), false, false);
  return pf_max(bits_f32(r[0]), bits_f32(r[1]));
}

constexpr int kRowsWaves = 4;
// Each wave owns RowSets<PREFILL> sets of 16 query rows: one step's K and V fragments,
// read once from LDS, feed the MFMAs of every set, and the sets' softmax chains are
// independent.  Chunked prefill (long ranges, many rows) takes two sets: ~170 VGPRs, two
// waves per SIMD.  The shared-prefix pass (a few 64-row tiles per KV head, short slices)
// keeps one set at <= 128 VGPRs and four waves per SIMD, which measured ~3 us faster on
// the 256-sequence workload than two sets.
template <bool PREFILL> struct RowSets {
  static constexpr int n = PREFILL ? 2 : 1;
  static constexpr int rows = 16 * kRowsWaves * n;  // query rows per workgroup
  static constexpr int waves_per_simd = PREFILL ? 2 : 4;
};
static_assert(RowSets<true>::rows == kPrefillRows && RowSets<false>::rows == kPrefixRows,
              "row tiles agree with the host plan");
constexpr float kRescaleSlack = 8.0f;  // log2 units: weights stay <= 2^8 between rescales
constexpr int kRowsDepth = 1;  // steps (32 tokens each) whose loads are in flight

// PREFILL = false: shared-prefix partials; true: causal chunked prefill.
//
// A step is two 16-token chunks A and B (B may be padding past the range).  Lane l of a
// wave holds the scores of its row l%16 against tokens 4(l/16) + i of A and of B
// (i < 4), and those 8 probabilities are its k-slots 8(l/16) .. 8(l/16)+7 of the
// 16x16x32 P.V MFMA (the contraction order is free as long as V uses the same one), so
// V is staged as [lane group g][dim][tokens 4g..4g+3 of A, 4g..4g+3 of B].
// KV: cache dtype (bf16, f16, or fp8 e4m3fn with 16-bit queries); QT: query dtype, the
// 16-bit type the tiles are staged in (fp8 codes convert to it exactly) and the MFMAs
// run in.
template <int KV, int QT, int D, bool PREFILL>
__global__ void __launch_bounds__(64 * kRowsWaves)
    __attribute__((amdgpu_waves_per_eu(RowSets<PREFILL>::waves_per_simd)))
rows_kernel(const RowsArgs a) {
  using O_ = PfxOps<QT>;
  using frag8 = typename O_::frag8;
  // P.V over an fp8 cache runs on the f16 MFMA with one f16 P (rounded toward zero,
  // < 2^-10 relative): its V codes convert to f16 exactly, and the fp8 tolerance leaves
  // room for that rounding.  Over 16-bit caches P keeps ~16 bits (hi + lo, two MFMAs):
  // a bf16 output's own rounding leaves too little of the tolerance for more.
  constexpr bool SINGLE_P = KV == kFP8;
  using PV_ = PfxOps<SINGLE_P ? kF16 : QT>;
  using pfrag8 = typename PV_::frag8;
  constexpr int EB = KV == kFP8 ? 1 : 2;  // cache element bytes
  constexpr int ROW = EB * D;          // bytes of one cache K/V row
  constexpr int QROW = 2 * D;          // bytes of one query row
  constexpr int NKC = D / 32;          // 16x16x32 MFMAs per 16 tokens of Q.K (K dims)
  constexpr int NJ = D / 16;           // 16-dim output tiles
  constexpr int NT = 64 * kRowsWaves;   // threads of the workgroup
  constexpr int PE = 16 / EB;           // elements of a 16-byte cache piece
  constexpr int KPIECES = 32 * (D / PE); // 16-byte pieces of a step's 32 K rows
  constexpr int KP = (KPIECES + NT - 1) / NT;  // K pieces per thread (the last round may be partial)
  constexpr bool KFULL = KPIECES % NT == 0;     // every thread has a piece in every round
  constexpr int DPT = 4 / EB;           // V dims per stager (one 32-bit word of each token row)
  constexpr int VSTAGE = 4 * (D / DPT); // V stagers: 4 lane groups x D/DPT dim groups
  constexpr int KROW = D + 8;           // K row stride in LDS (elements): conflict-free A reads
  constexpr int STRIDE = 4 + D;         // floats per partial: m, l, pad, pad, acc[D]
  static_assert(KPIECES % 64 == 0 && VSTAGE <= NT && VSTAGE % 64 == 0 && (16 * (D / PE)) % 64 == 0,
                "staging by whole waves of the workgroup");
  // K as [32 tokens][KROW]; V as [lane group g][dim][8 tokens: 4g..4g+3 of A, of B], 16-bit.
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][32 * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][4 * D * 8];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int Hkv = a.num_kv_heads, G = a.num_q_heads / Hkv;
  int bid = blockIdx.x;
  const int g = bid % Hkv;
  bid /= Hkv;
  // ---- this workgroup's rows, their sequence and the chunk range [c0, c1)
  int T = 1, t = 0, s, nrows, c0, c1, qbase, row0, base_pos = 0, ctx = 0;
  if constexpr (PREFILL) {
    // rows (query token i, head) of sequence s: row r -> token r / G, head g G + r % G
    row0 = (bid % a.tiles) * kPrefillRows;
    s = bid / a.tiles;
    const int n = a.cu_q[s + 1] - a.cu_q[s];
    nrows = n * G;
    if (row0 >= nrows) return;  // whole workgroup: no barrier reached
    ctx = a.context_lens[s];
    base_pos = ctx - n;         // position of query token 0
    qbase = a.cu_q[s];
    const int last = min(nrows, row0 + kPrefillRows) - 1;
    c0 = 0;
    c1 = (base_pos + last / G + 1 + 15) / 16;  // through the last row's own token
  } else {
    // rows (sequence, head) of group j: row r -> sequence s0 + r / G, head g G + r % G
    T = a.splits;
    t = bid % T;
    bid /= T;
    row0 = (bid % a.tiles) * kPrefixRows;
    const int j = bid / a.tiles;
    s = a.group_starts[j];
    nrows = (a.group_starts[j + 1] - s) * G;
    if (row0 >= nrows) return;  // whole workgroup: no barrier reached
    const int P = a.prefix_lens[s];
    if (P <= 0) return;         // nothing shared: the suffix pass reads no partial
    const int nch = P / 16;
    c0 = nch * t / T;
    c1 = nch * (t + 1) / T;
    qbase = s;
  }
  const int32_t* bt = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const int BS = a.block_size;
  // this KV head's rows of block 0; a block's rows for all heads span blk_bytes
  const size_t head_off = (size_t)g * BS * ROW;
  const uint8_t* kc = (const uint8_t*)a.k_cache + head_off;
  const uint8_t* vc = (const uint8_t*)a.v_cache + head_off;
  const uint32_t blk_bytes = (uint32_t)Hkv * (uint32_t)(BS * ROW);
  // Scores are taken raw (S = K Q^T) and scaled inside the exponent, 2^(c s - m) with
  // c = |scale| log2(e) > 0, so the running max can be taken on raw scores: a negative
  // scale flips the sign of Q instead (exact in 16 bits) and a zero scale zeroes Q (all
  // scores 0: the same uniform weights).
  const float c_l2 = (a.scale != 0.0f ? __builtin_fabsf(a.scale) : 1.0f) * kLog2e * a.k_scale;
  const uint32_t qflip = a.scale < 0.0f ? 0x80008000u : 0u;
  const bool qzero = a.scale == 0.0f;

  // ---- this lane's query row in each set rs (B operand of S^T = K Q^T: row l%16 of the
  // set, dims 8(l/16) + 32c); the wave's rows are row0 + 16 (RS wv + rs) + 0..15
  constexpr int RS = RowSets<PREFILL>::n;
  const int wrow0 = row0 + 16 * RS * wv;
  int rq[RS], lim[RS];
  bool qvalid[RS];
  frag8 qf[RS][NKC];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    rq[rs] = wrow0 + 16 * rs + (lane & 15);
    qvalid[rs] = rq[rs] < nrows;
    const uint8_t* qrow = (const uint8_t*)a.q +
        ((size_t)(qbase + (qvalid[rs] ? rq[rs] / G : 0)) * a.num_q_heads + g * G + (qvalid[rs] ? rq[rs] % G : 0)) * QROW;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (qvalid[rs] && !qzero) {
        w = *(const uint4*)(qrow + 2 * (32 * c + 8 * (lane >> 4)));
        w = make_uint4(w.x ^ qflip, w.y ^ qflip, w.z ^ qflip, w.w ^ qflip);
      }
      qf[rs][c] = __builtin_bit_cast(frag8, w);
    }
    // this row attends to tokens < lim (prefill: its own position included; prefix: the
    // range's end, so a padding chunk B past it is masked)
    lim[rs] = PREFILL ? base_pos + (qvalid[rs] ? rq[rs] / G : 0) + 1 : 16 * c1;
  }
  // the smallest limit of the wave's rows (rows grow with the query token): steps below
  // it need no mask
  const int lim_lo = PREFILL ? __builtin_amdgcn_readfirstlane(base_pos + min(wrow0, nrows - 1) / G + 1)
                             : 16 * c1;

  // per set: m, the row's reference max (log2 domain, scaled); O, unnormalised output
  // rows 4(l/16) + i, dims 16jj + l%16; lrow, this lane's share of row l%16's denominator
  // (VSUM), or Om, the denominators of rows 4(l/16) + i summed on the matrix cores as P
  // times a ones tile (every column holds the row sum)
  constexpr bool VSUM = !(PREFILL && KV == kFP8);
  float m[RS];
  f32x4_t O[RS][NJ];
  float lrow[RS];
  f32x4_t Om[RS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    m[rs] = kNegInf;
    lrow[rs] = 0.0f;
    Om[rs] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) O[rs][jj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int bs_shift = BS == 32 ? 5 : 4;  // block size 16 or 32
  // A step's two chunks (clamped to the range's last one): their physical blocks, read
  // from the table one step before the step's loads are issued (scalar loads, so that
  // the issue does not wait for them), and their rows' byte offsets from kc / vc.
  struct Blk {
    uint32_t a, b;
  };
  auto blk_pair = [&](int cA) {
    return Blk{(uint32_t)bt[(16 * min(cA, c1 - 1)) >> bs_shift], (uint32_t)bt[(16 * min(cA + 1, c1 - 1)) >> bs_shift]};
  };
  auto tile_off = [&](int c, uint32_t blk) {
    return (size_t)blk * blk_bytes + (uint32_t)(((16 * min(c, c1 - 1)) & (BS - 1)) * ROW);
  };
  // Staging: K piece q = tid + NT k (k < KP, q < KPIECES) is row q / (D/PE) (chunk A for
  // rows < 16, B after), 16-byte piece q % (D/PE); V stager (gg, dp) = (tid / (D/DPT),
  // tid % (D/DPT)) loads tokens 4gg .. 4gg+3 of A and of B, dims DPT dp .. DPT dp + DPT-1
  // (one 32-bit word of each row).  Every thread issues all its loads, the ones it has no
  // part in through an empty resource.  fp8 codes become the query's 16-bit type on the
  // way into LDS.
  const int gg = (tid / (D / DPT)) & 3, dp = tid % (D / DPT);
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const bool vstage = tid < VSTAGE;
  struct Stage {
    uint4 k[KP];
    uint32_t v[8];
  };
  // Step at chunk cA (chunks cA, cA + 1): live halves read, padding ones read nothing.
  auto issue = [&](int cA, Blk bk, Stage& st) {
    const bool la = cA < c1, lb = cA + 1 < c1;
    const size_t oa = tile_off(cA, bk.a), ob = tile_off(cA + 1, bk.b);
    const __amdgpu_buffer_rsrc_t ka = tile_rsrc(kc + oa, la ? 16 * ROW : 0);
    const __amdgpu_buffer_rsrc_t kb = tile_rsrc(kc + ob, lb ? 16 * ROW : 0);
    const __amdgpu_buffer_rsrc_t none = tile_rsrc(kc, 0);
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int q = tid + NT * k, r = q / (D / PE), pc = q % (D / PE);
      // rows < 16 (pieces q < 16 D/PE, a multiple of 64) are chunk A, so a whole wave's
      // pieces fall in one chunk (a scalar select of the resources), and so does the
      // bound q < KPIECES of a partial last round
      const bool in_a = 64 * wvu + NT * k < 16 * (D / PE);
      const bool kact = KFULL || 64 * wvu + NT * k < KPIECES;
      st.k[k] = load_kv16<false>(kact ? (in_a ? ka : kb) : none, (r & 15) * ROW + 16 * pc);
    }
    const __amdgpu_buffer_rsrc_t va = tile_rsrc(vc + oa, la && vstage ? 16 * ROW : 0);
    const __amdgpu_buffer_rsrc_t vb = tile_rsrc(vc + ob, lb && vstage ? 16 * ROW : 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      st.v[e] = load_kv4<false>(va, (4 * gg + e) * ROW + 4 * dp);
      st.v[4 + e] = load_kv4<false>(vb, (4 * gg + e) * ROW + 4 * dp);
    }
  };
  // Step at chunk cA into LDS buffer buf.  Prefill: V rows past the context (the tail of
  // its last block: any bytes, NaN included) are staged as zeros, so that their zero
  // weights cannot turn into NaN; K rows there only meet masked scores.
  auto stage = [&](int buf, int cA, const Stage& st) {
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int q = tid + NT * k, r = q / (D / PE), pc = q % (D / PE);
      if (!KFULL && 64 * wvu + NT * k >= KPIECES) continue;  // wave-uniform
      if constexpr (EB == 2) {
        *(uint4*)&lds_k[buf][r * KROW + 8 * pc] = st.k[k];
      } else {  // 16 codes -> 16 elements: two 16-byte writes
        const uint2 x0 = O_::from_fp8(st.k[k].x), x1 = O_::from_fp8(st.k[k].y);
        const uint2 x2 = O_::from_fp8(st.k[k].z), x3 = O_::from_fp8(st.k[k].w);
        *(uint4*)&lds_k[buf][r * KROW + 16 * pc] = make_uint4(x0.x, x0.y, x1.x, x1.y);
        *(uint4*)&lds_k[buf][r * KROW + 16 * pc + 8] = make_uint4(x2.x, x2.y, x3.x, x3.y);
      }
    }
    if (vstage) {
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = st.v[e];
      if (PREFILL && 16 * (cA + 2) > ctx) {  // the step that holds the context's end
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (16 * (cA + e / 4) + 4 * gg + (e & 3) >= ctx) w[e] = 0u;
      }
      // x[e]: two 16-bit dims of token e per word; dim 2j of the pair j: the low halves of
      // the 8 tokens' words, dim 2j+1: the high halves
      auto put_pair = [&](const uint32_t (&x)[8], int dim) {
        const uint4 lo = make_uint4(__builtin_amdgcn_perm(x[1], x[0], 0x05040100u),
                                    __builtin_amdgcn_perm(x[3], x[2], 0x05040100u),
                                    __builtin_amdgcn_perm(x[5], x[4], 0x05040100u),
                                    __builtin_amdgcn_perm(x[7], x[6], 0x05040100u));
        const uint4 hi = make_uint4(__builtin_amdgcn_perm(x[1], x[0], 0x07060302u),
                                    __builtin_amdgcn_perm(x[3], x[2], 0x07060302u),
                                    __builtin_amdgcn_perm(x[5], x[4], 0x07060302u),
                                    __builtin_amdgcn_perm(x[7], x[6], 0x07060302u));
        uint16_t* base = &lds_v[buf][(gg * D + dim) * 8];
        *(uint4*)base = lo;
        *(uint4*)(base + 8) = hi;
      };
      if constexpr (EB == 2) {
        put_pair(w, 2 * dp);
      } else {  // each word holds 4 codes: dims 4dp .. 4dp+3
        uint32_t x0[8], x1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint2 c = PV_::from_fp8(w[e]);  // V in the P.V type
          x0[e] = c.x;
          x1[e] = c.y;
        }
        put_pair(x0, 4 * dp);
        put_pair(x1, 4 * dp + 2);
      }
    }
  };
  // One step from LDS buffer buf: S^T = K Q^T for chunks A and B, online softmax over
  // their 32 tokens, O += P V, for every row set of the wave.
  auto compute = [&](int buf, int cA) {
    // A = K rows: lane l reads token l%16 of a chunk, dims 32cc + 8(l/16)
    f32x4_t SA[RS], SB[RS];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) SA[rs] = SB[rs] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cc = 0; cc < NKC; ++cc) {
      const frag8 ka = __builtin_bit_cast(
          frag8, *(const uint4*)&lds_k[buf][(lane & 15) * KROW + 32 * cc + 8 * (lane >> 4)]);
      const frag8 kb = __builtin_bit_cast(
          frag8, *(const uint4*)&lds_k[buf][(16 + (lane & 15)) * KROW + 32 * cc + 8 * (lane >> 4)]);
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        SA[rs] = O_::qk(ka, qf[rs][cc], SA[rs]);
        SB[rs] = O_::qk(kb, qf[rs][cc], SB[rs]);
      }
    }
    float sv[RS][8];  // raw scores
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[rs][i] = SA[rs][i];
        sv[rs][4 + i] = SB[rs][i];
      }
    if (16 * cA + 32 > lim_lo) {  // a step reaching some row's limit: mask its tokens past it
#pragma unroll
      for (int rs = 0; rs < RS; ++rs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ta = 16 * cA + 4 * (lane >> 4) + i;
          if (ta >= lim[rs]) sv[rs][i] = kNegInf;  // causal mask / range end
          if (ta + 16 >= lim[rs]) sv[rs][4 + i] = kNegInf;
        }
    }
    // every row's first step holds a token it attends to (prefix: all of chunk A;
    // prefill: token 0), so m is finite from the first step on (a later step masked for
    // the whole row gives bm = -inf, which moves nothing)
    float bm[RS];
    bool move[RS], any = false;
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      const float* v = sv[rs];
      float x = pf_max(pf_max(pf_max(v[0], v[1]), v[2]), pf_max(pf_max(v[3], v[4]), v[5]));
      x = pf_max(pf_max(x, v[6]), v[7]);
      bm[rs] = pf_xor32_max(pf_xor16_max(x)) * c_l2;
      // Lazy rescaling: the reference max m moves only when a score exceeds it by more
      // than kRescaleSlack (and on the first step, m = -inf), so weights 2^(s - m) stay
      // <= 2^8.  (m, l, acc) stay one consistent partial -- l and acc are sums of
      // 2^(s - m) for the same m -- so the log-sum-exp algebra is unchanged; only the
      // rare rescale remains (one branch for all sets).
      move[rs] = bm[rs] > m[rs] + kRescaleSlack;
      any = any || move[rs];
    }
    if (__ballot(any) != 0) {
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        const float mn = move[rs] ? bm[rs] : m[rs];
        const float alpha = fast_exp2(m[rs] - mn);  // 0 on the first step, 1 for rows kept
        m[rs] = mn;
        if constexpr (VSUM) lrow[rs] *= alpha;  // this lane's row is row l%16
        // O rows 4(l/16) + i take the factor of row 4(l/16) + i, held by lane 4(l/16) + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * (lane >> 4) + i);
          if constexpr (!VSUM) Om[rs][i] *= ai;
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj) O[rs][jj][i] *= ai;
        }
      }
    }
    pfrag8 ahi[RS], alo[RS];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = fast_exp2(__builtin_fmaf(sv[rs][i], c_l2, -m[rs]));
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (SINGLE_P)
          hw[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p[2 * i], p[2 * i + 1]));
        else
          PV_::split2(p[2 * i], p[2 * i + 1], hw[i], lw[i]);
      }
      ahi[rs] = __builtin_bit_cast(pfrag8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      if constexpr (!SINGLE_P) alo[rs] = __builtin_bit_cast(pfrag8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      if constexpr (VSUM) {
        lrow[rs] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      } else {
        const pfrag8 ones = __builtin_bit_cast(pfrag8, make_uint4(PV_::kOne, PV_::kOne, PV_::kOne, PV_::kOne));
        Om[rs] = PV_::qk(ahi[rs], ones, Om[rs]);
        if constexpr (!SINGLE_P) Om[rs] = PV_::qk(alo[rs], ones, Om[rs]);
      }
    }
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const pfrag8 vf = __builtin_bit_cast(
          pfrag8, *(const uint4*)&lds_v[buf][((lane >> 4) * D + 16 * jj + (lane & 15)) * 8]);
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        O[rs][jj] = PV_::qk(ahi[rs], vf, O[rs][jj]);
        if constexpr (!SINGLE_P) O[rs][jj] = PV_::qk(alo[rs], vf, O[rs][jj]);
      }
    }
  };

  // Steps at chunks c0, c0 + 2, ... < c1.  Step k's loads go to ring slot k % PD, and
  // its tiles to LDS buffer k & 1.  At step ii: the loads of step ii + PD are issued into
  // the slot step ii vacated (staged one step earlier), step ii is computed from LDS
  // while they and the other steps' loads are in flight, then step ii + 1 is staged from
  // its slot.  Every step issues its loads unconditionally, padding ones through an
  // empty resource; the ring is rotated by a fully unrolled inner loop.
  constexpr int PD = kRowsDepth;
  if (c0 < c1) {
    const int n = (c1 - c0 + 1) / 2;  // steps
    Stage ring[PD];
#pragma unroll
    for (int u = 0; u < PD; ++u) issue(c0 + 2 * u, blk_pair(c0 + 2 * u), ring[u]);
    Blk next = blk_pair(c0 + 2 * PD);  // the blocks of the next step issued
    stage(0, c0, ring[0]);
    __syncthreads();
    for (int i = 0; i < n; i += PD) {
#pragma unroll
      for (int u = 0; u < PD; ++u) {
        const int ii = i + u;
        if (ii >= n) break;
        issue(c0 + 2 * (ii + PD), next, ring[u]);
        compute(ii & 1, c0 + 2 * ii);
        if (ii + 1 < n) stage((ii + 1) & 1, c0 + 2 * (ii + 1), ring[(u + 1) % PD]);
        // the next issue's blocks: scalar loads placed before the barrier, whose wait
        // for the step's LDS writes covers them too
        next = blk_pair(c0 + 2 * (ii + PD + 1));
        __syncthreads();
      }
    }
  }

  // each row's denominator: the four lane groups' shares summed (every lane of column l%16
  // then holds row l%16's), and Ol[rs][i] that of row 4(l/16) + i, the layout of O
  f32x4_t Ol[RS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    if constexpr (!VSUM) {
      Ol[rs] = Om[rs];
      continue;
    }
    float x = lrow[rs];
    auto r16 = __builtin_amdgcn_permlane16_swap(f32_bits(x), f32_bits(x), false, false);
    x = bits_f32(r16[0]) + bits_f32(r16[1]);
    auto r32 = __builtin_amdgcn_permlane32_swap(f32_bits(x), f32_bits(x), false, false);
    x = bits_f32(r32[0]) + bits_f32(r32[1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) Ol[rs][i] = __shfl(x, 4 * (lane >> 4) + i);
  }
  if constexpr (PREFILL) {
    // ---- output rows 4(l/16) + i of each set, dims 16jj + l%16: acc / l of that row,
    // rounded to the output dtype
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float li = Ol[rs][i];
        const int rr = wrow0 + 16 * rs + 4 * (lane >> 4) + i;
        if (rr >= nrows) continue;
        const float inv = li != 0.0f ? a.v_scale / li : 0.0f;  // fp8: value = code * v_scale
        const size_t o = ((size_t)(qbase + rr / G) * a.num_q_heads + g * G + rr % G) * D + (lane & 15);
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) store_out(a.out, o + 16 * jj, a.out_dtype, O[rs][jj][i] * inv);
      }
    }
  } else {
    // ---- partials: m per row (lanes 0..15: row l%16 of the set), l and acc of rows
    // 4(l/16) + i (l from the lanes of column 0), acc dims 16jj + l%16
    auto part_of = [&](int rr) {
      return a.pre_part + (((size_t)(qbase + rr / G) * a.num_q_heads + g * G + rr % G) * T + t) * STRIDE;
    };
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      if (lane < 16 && qvalid[rs]) part_of(rq[rs])[0] = m[rs];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = wrow0 + 16 * rs + 4 * (lane >> 4) + i;
        if (rr >= nrows) continue;
        float* pp = part_of(rr);
        if ((lane & 15) == 0) pp[1] = Ol[rs][i];
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) pp[4 + 16 * jj + (lane & 15)] = O[rs][jj][i];
      }
    }
  }
}

// ---- dispatch --------------------------------------------------------------------
template <bool PREFILL>
static hipError_t launch_rows(const RowsArgs& a, int64_t grid) {
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 block(64 * kRowsWaves);
#define PKV_ROWS(KV, QT)                                                                                 \
  if (a.head_dim == 128)                                                                                 \
    hipLaunchKernelGGL((rows_kernel<KV, QT, 128, PREFILL>), dim3((unsigned)grid), block, 0, a.stream, a); \
  else if (a.head_dim == 64)                                                                             \
    hipLaunchKernelGGL((rows_kernel<KV, QT, 64, PREFILL>), dim3((unsigned)grid), block, 0, a.stream, a);  \
  else                                                                                                   \
    return hipErrorInvalidValue;
  if (a.cache_dtype == kBF16 && a.q_dtype == kBF16) { PKV_ROWS(kBF16, kBF16) }
  else if (a.cache_dtype == kF16 && a.q_dtype == kF16) { PKV_ROWS(kF16, kF16) }
  else if (a.cache_dtype == kFP8 && a.q_dtype == kBF16) { PKV_ROWS(kFP8, kBF16) }
  else if (a.cache_dtype == kFP8 && a.q_dtype == kF16) { PKV_ROWS(kFP8, kF16) }
  else return hipErrorInvalidValue;
#undef PKV_ROWS
  return hipGetLastError();
}

hipError_t launch_prefix(const RowsArgs& a, int num_groups) {
  return launch_rows<false>(a, (int64_t)num_groups * a.tiles * a.splits * a.num_kv_heads);
}

hipError_t launch_prefill(const RowsArgs& a) {
  return launch_rows<true>(a, (int64_t)a.num_seqs * a.tiles * a.num_kv_heads);
}

}  // namespace pkv
