/*
 * oracle.c -- plain, slow, fp64 CPU reference for one paged decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP library and includes nothing from it.
 *
 * What it computes, each function citing the passage it follows:
 *   oracle_slot_mapping  -- logical position -> (physical block, offset) through a
 *                           per-sequence block table.
 *   oracle_kv_write      -- store each new token's K and V in its slot.
 *   oracle_decode        -- each query head's attention over its sequence's whole
 *                           cached context, read through the block table, with an
 *                           exact two-pass softmax in fp64.
 *   oracle_decode_window -- the same over a sliding window of the last tokens plus
 *                           the first (sink) tokens.
 *   oracle_prefill       -- chunked prefill: many causal query tokens per sequence
 *                           over the same paged cache.
 *   oracle_copy_blocks   -- copy-on-write copy of whole physical blocks.
 *   oracle_swap_blocks   -- blocks to / from a contiguous (host) buffer.
 *   oracle_kv_bytes      -- the pages' KV-memory closed form.
 *   codecs               -- bf16 / fp16 / OCP e4m3fn decoders, e4m3fn encoder.
 *
 * Readings taken where the pages leave a step open (each also listed in the
 * design notes): the context length counts the new token; query head h uses KV
 * head h / (H_q / H_kv); a negative slot means "skip"; fp8 is OCP e4m3fn with a
 * per-tensor fp32 scale, encoded as RNE of the fp32 quotient x / scale with
 * saturation to +-448 and NaN kept NaN.
 *
 * Mutations: building with -DORACLE_MUTATION=n plants one deliberate mistake
 * (see the MUT() sites).  The test suite uses these builds to show that its pins
 * catch each such mistake.  Normal builds define no mutation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTATION
#define ORACLE_MUTATION 0
#endif
#define MUT(n) (ORACLE_MUTATION == (n))

enum { O_F32 = 0, O_F16 = 1, O_BF16 = 2, O_FP8 = 3 };

static int elem_bytes(int dt) {
  switch (dt) {
    case O_F32: return 4;
    case O_F16: return 2;
    case O_BF16: return 2;
    case O_FP8: return 1;
    default: return 0;
  }
}

/* ---------------------------------------------------------------- codecs -- */

/* bf16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t h) {
  uint32_t u = MUT(8) ? ((uint32_t)h << 8) : ((uint32_t)h << 16);
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1.0 + m / 1024.0, e - 15);
  return sign ? -v : v;
}

/* OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 fraction bits; no infinities;
 * S.1111.111 is NaN; the largest finite magnitude is 1.75 * 2^8 = 448. */
double oracle_fp8_to_f64(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 15;
  int m = c & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

/* fp32 value -> e4m3fn code, round to nearest (ties to even), saturating. */
uint8_t oracle_f32_to_fp8(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return sign | 0x7F;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E; /* satfinite, infinities included */
  /* Spacing of the e4m3 grid around a: 2^-9 below the smallest normal 2^-6,
   * else 2^(floor(log2 a) - 3).  Dividing by the spacing is exact in fp64, so
   * rint (ties to even under the default rounding mode) rounds on the grid. */
  double quantum;
  if (a < ldexp(1.0, -6)) {
    quantum = ldexp(1.0, -9);
  } else {
    int e2;
    frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
    quantum = ldexp(1.0, (e2 - 1) - 3);
  }
  double r = MUT(7) ? trunc(a / quantum) * quantum : rint(a / quantum) * quantum;
  if (r > 448.0) r = 448.0;
  /* Encode the rounded magnitude. */
  uint8_t code;
  if (r < ldexp(1.0, -6)) {
    code = (uint8_t)(r / ldexp(1.0, -9)); /* subnormal; 0..7 */
  } else {
    int e2;
    double f = frexp(r, &e2);                 /* r = f * 2^e2 */
    int e = e2 - 1;                           /* r = (2f) * 2^e, 2f in [1, 2) */
    int m = (int)((2.0 * f - 1.0) * 8.0);     /* exact: r lies on the grid */
    code = (uint8_t)(((e + 7) << 3) | m);
  }
  return sign | code;
}

static double load_f64(const void* base, int64_t idx, int dt) {
  switch (dt) {
    case O_F32: return (double)((const float*)base)[idx];
    case O_F16: return oracle_f16_to_f64(((const uint16_t*)base)[idx]);
    case O_BF16: return oracle_bf16_to_f64(((const uint16_t*)base)[idx]);
    case O_FP8: return oracle_fp8_to_f64(((const uint8_t*)base)[idx]);
    default: return NAN;
  }
}

/* Source element as an fp32 value (sources are f32, f16 or bf16; each converts
 * exactly to fp32). */
static float load_f32(const void* base, int64_t idx, int dt) {
  return (float)load_f64(base, idx, dt);
}

/* ------------------------------------------------------ memory closed form -- */

/* KV bytes for T cached tokens: T * L * 2 * H_KV * d_h * b
 * ("Capitulo 2 -- KV cache, jerarquia de memoria...", section "Una formula util
 * para estimar memoria", the M_KV(T) equation). */
int64_t oracle_kv_bytes(int64_t T, int64_t L, int64_t H_kv, int64_t d_h, int64_t b) {
  return T * L * 2 * H_kv * d_h * b;
}

/* ------------------------------------------------------ slot resolution a0 -- */

/* Physical slot of (sequence, logical position): the block table entry at
 * position / B, offset position % B ("Optimizacion de Inferencia LLM", section
 * "PagedAttention: Conceptos de SO...", BlockTable.get_physical_block; "PagedAttention
 * por dentro", section "La tabla de paginas (block table)", token 200 -> entry 12).
 * slot = physical_block * B + offset.  A negative position gives slot -1. */
int oracle_slot_mapping(const int32_t* seq_ids, const int32_t* positions, int64_t num_tokens,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        int32_t block_size, int64_t* slot_mapping) {
  if (block_size <= 0) return -3;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t pos = positions[t];
    if (pos < 0) { slot_mapping[t] = -1; continue; }
    int64_t logical_block = MUT(3) ? pos % block_size : pos / block_size;
    int64_t offset = MUT(3) ? pos / block_size : pos % block_size;
    if (logical_block >= max_blocks_per_seq) return -5;
    int64_t physical = block_tables[(int64_t)seq_ids[t] * max_blocks_per_seq + logical_block];
    slot_mapping[t] = physical * block_size + offset;
  }
  return 0;
}

/* ------------------------------------------------------------- KV write a1 -- */

/* Store token t's K and V (each [H_kv][d_h]) at cache[slot / B][h][slot % B][:]
 * ("PagedAttention por dentro", section "La tabla de paginas (block table)": the
 * new token goes to the free slot of the last block, or the first slot of a newly
 * appended block).  Cache layout [num_blocks][H_kv][B][d_h].  Same dtype: bit copy.
 * fp8 cache: RNE-satfinite e4m3fn of fl32(fl32(x) / scale).  Other bytes unchanged.
 */
int oracle_kv_write(const int64_t* slot_mapping, int64_t num_tokens, const void* k,
                    const void* v, int src_dtype, void* k_cache, void* v_cache,
                    int64_t num_blocks, int32_t block_size, int32_t H_kv, int32_t d_h,
                    int cache_dtype, float k_scale, float v_scale) {
  int sb = elem_bytes(src_dtype), cb = elem_bytes(cache_dtype);
  if (!sb || !cb || src_dtype == O_FP8) return -2;
  if (cache_dtype != O_FP8 && cache_dtype != src_dtype) return -2;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t blk = slot / block_size, off = slot % block_size;
    if (blk >= num_blocks) return -5;
    for (int32_t h = 0; h < H_kv; ++h) {
      int64_t src = ((int64_t)t * H_kv + h) * d_h;
      int64_t dst = ((blk * H_kv + h) * block_size + off) * d_h;
      if (cache_dtype == O_FP8) {
        for (int32_t d = 0; d < d_h; ++d) {
          float kq = load_f32(k, src + d, src_dtype) / k_scale;
          float vq = load_f32(v, src + d, src_dtype) / v_scale;
          ((uint8_t*)k_cache)[dst + d] = oracle_f32_to_fp8(kq);
          ((uint8_t*)v_cache)[dst + d] = oracle_f32_to_fp8(MUT(5) ? kq : vq);
        }
      } else {
        memcpy((char*)k_cache + dst * cb, (const char*)k + src * sb, (size_t)d_h * cb);
        memcpy((char*)v_cache + dst * cb, (const char*)(MUT(5) ? k : v) + src * sb,
               (size_t)d_h * cb);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------ block copies, swap -- */

/* Copy-on-write: for each pair i, the whole physical block src[i] (every KV head, K
 * and V) is copied to block dst[i], so that the sequence about to write into a shared
 * block gets a private copy first ("PagedAttention por dentro...", section
 * "Copy-on-write para sampling paralelo": only the last affected block is copied when
 * a branch diverges; "La despensa por casilleros", section "Prefix caching...": the
 * block manager copies the block for that branch and only then writes).  A pair with
 * a negative ID is skipped.  All sources are read before any destination is written.
 * block_bytes = H_kv * B * d_h * element bytes.
 */
int oracle_copy_blocks(const int32_t* src, const int32_t* dst, int64_t num_pairs, void* k_cache,
                       void* v_cache, int64_t num_blocks, int64_t block_bytes) {
  if (num_pairs <= 0) return 0;
  char* tmp = (char*)malloc((size_t)(2 * num_pairs * block_bytes));
  if (!tmp) return -7;
  for (int64_t i = 0; i < num_pairs; ++i) {
    if (src[i] < 0 || dst[i] < 0) continue;
    if (src[i] >= num_blocks || dst[i] >= num_blocks) { free(tmp); return -5; }
    memcpy(tmp + (2 * i) * block_bytes, (char*)k_cache + src[i] * block_bytes, (size_t)block_bytes);
    memcpy(tmp + (2 * i + 1) * block_bytes, (char*)(MUT(11) ? k_cache : v_cache) + src[i] * block_bytes,
           (size_t)block_bytes);
  }
  for (int64_t i = 0; i < num_pairs; ++i) {
    if (src[i] < 0 || dst[i] < 0) continue;
    memcpy((char*)k_cache + dst[i] * block_bytes, tmp + (2 * i) * block_bytes, (size_t)block_bytes);
    memcpy((char*)v_cache + dst[i] * block_bytes, tmp + (2 * i + 1) * block_bytes, (size_t)block_bytes);
  }
  free(tmp);
  return 0;
}

/* Swap out: block ids[i] of each cache goes to row i of a contiguous buffer
 * ([num][block_bytes] for K, the same for V); swap in: row i comes back into block
 * ids[i] ("PagedAttention por dentro...", section "Estrategia 2: swap": the evicted
 * session's blocks move to CPU RAM and come back to VRAM when it is resumed).  A
 * negative ID skips its row.  direction 0 = out (cache -> buffer), 1 = in.
 */
int oracle_swap_blocks(const int32_t* ids, int64_t num, void* k_cache, void* v_cache,
                       void* k_buf, void* v_buf, int64_t num_blocks, int64_t block_bytes, int direction) {
  for (int64_t i = 0; i < num; ++i) {
    if (ids[i] < 0) continue;
    if (ids[i] >= num_blocks) return -5;
    char* kc = (char*)k_cache + ids[i] * block_bytes;
    char* vc = (char*)v_cache + ids[i] * block_bytes;
    char* kb = (char*)k_buf + i * block_bytes;
    char* vb = (char*)v_buf + i * block_bytes;
    if (direction == 0) {
      memcpy(kb, kc, (size_t)block_bytes);
      memcpy(vb, vc, (size_t)block_bytes);
    } else {
      memcpy(kc, kb, (size_t)block_bytes);
      memcpy(vc, vb, (size_t)block_bytes);
    }
  }
  return 0;
}

/* ---------------------------------------------------------- attention a2-a7 -- */

/* Decode attention for the listed (sequence, query head) pairs:
 *   out[s][h][:] = softmax_t(scale * q[s][h] . K_t) @ V_t,  t in A(s),
 * where K_t, V_t are KV head g = h / G of token t, read at physical block
 * block_tables[s][t / B], offset t % B, and dequantised (fp8: code * scale).
 * ("Capitulo 2", section "Que guarda realmente el KV cache": Attn(q_t, [K_{1:t-1},
 * k_t], [V_{1:t-1}, v_t]) -- the new token attends to itself; "Optimizacion de
 * Inferencia LLM", section "El Cuello de Botella...": softmax(q @ k.T / sqrt(d_head))
 * @ v over positions :T+1; "La despensa por casilleros", section "El mecanismo":
 * the kernel walks the physical blocks in logical order; "KV cache: la memoria de
 * trabajo", section "Trucos para que el cuaderno sea mas fino": query heads in
 * groups of G share one K/V head.)
 *
 * A(s), the attended tokens of a context of n = ctx[s] tokens:
 *   window == 0: every token, 0 .. n-1;
 *   window >  0: the last `window` tokens, n - window .. n-1 ("PagedAttention por
 *                dentro...", section "Sliding window attention": such models attend
 *                only to the last K tokens), together with the first `sinks` tokens,
 *                0 .. sinks-1 (same page, section "StreamingLLM...: los attention
 *                sinks": keep the first 4 tokens plus a window of the last K).
 * Tokens outside A(s) are never read, nor are their block-table entries.
 * The softmax is the exact two-pass form over A(s): m = max z, w = exp(z - m),
 * out = sum w V / sum w, all fp64.  ctx = 0 gives zeros.  pairs == NULL means every
 * (s, h) in order; out is [num_pairs][d_h] fp64.  bytes_read (optional) accumulates
 * the K/V bytes this call decoded.  num_threads <= 0 lets OpenMP choose.
 */
int oracle_decode_window(const void* q, int q_dtype, int32_t num_seqs, int32_t num_q_heads,
                         const void* k_cache, const void* v_cache, int cache_dtype, float k_scale,
                         float v_scale, int64_t num_blocks, int32_t block_size, int32_t H_kv,
                         int32_t d_h, const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t window, int32_t sinks, float scale,
                         const int32_t* pairs, int64_t num_pairs, double* out, int64_t* bytes_read,
                         int num_threads) {
  if (H_kv <= 0 || num_q_heads % H_kv) return -4;
  if (!elem_bytes(q_dtype) || !elem_bytes(cache_dtype)) return -2;
  if (window < 0 || sinks < 0) return -3;
  const int32_t G = num_q_heads / H_kv;
  const int cb = elem_bytes(cache_dtype);
  if (!pairs) num_pairs = (int64_t)num_seqs * num_q_heads;
  int status = 0;
  int64_t total_bytes = 0;
#ifdef _OPENMP
  if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads) reduction(+ : total_bytes)
#endif
  for (int64_t i = 0; i < num_pairs; ++i) {
    int32_t s = pairs ? pairs[2 * i] : (int32_t)(i / num_q_heads);
    int32_t h = pairs ? pairs[2 * i + 1] : (int32_t)(i % num_q_heads);
    double* o = out + i * d_h;
    int32_t g = MUT(1) ? h % H_kv : h / G;
    int32_t n = context_lens[s] - (MUT(6) ? 1 : 0);
    for (int32_t d = 0; d < d_h; ++d) o[d] = 0.0;
    if (n <= 0) continue;
    /* the attended tokens, in logical order */
    int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    double* z = (double*)malloc(sizeof(double) * (size_t)n);
    if (!tok || !z) { free(tok); free(z); status = -7; continue; }
    int32_t na = 0;
    for (int32_t t = 0; t < n; ++t) {
      int in_window = MUT(9) ? t > n - window : t >= n - window;
      int is_sink = MUT(10) ? 0 : t < sinks;
      if (window == 0 || in_window || is_sink) tok[na++] = t;
    }
    double qd_scale = MUT(4) ? 1.0 : (double)scale;
    double kscale = cache_dtype == O_FP8 ? (double)k_scale : 1.0;
    double vscale = cache_dtype == O_FP8 ? (double)v_scale : 1.0;
    const int64_t q_base = ((int64_t)s * num_q_heads + h) * d_h;
    for (int32_t j = 0; j < na; ++j) {
      int32_t t = tok[j];
      int64_t phys = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
      int64_t row = ((phys * H_kv + g) * block_size + t % block_size) * d_h;
      double acc = 0.0;
      for (int32_t d = 0; d < d_h; ++d)
        acc += load_f64(q, q_base + d, q_dtype) *
               (load_f64(MUT(2) ? v_cache : k_cache, row + d, cache_dtype) * kscale);
      z[j] = qd_scale * acc;
      total_bytes += 2 * (int64_t)d_h * cb;
    }
    double m = z[0];
    for (int32_t j = 1; j < na; ++j)
      if (z[j] > m) m = z[j];
    double wsum = 0.0;
    for (int32_t j = 0; j < na; ++j) {
      z[j] = exp(z[j] - m);
      wsum += z[j];
    }
    for (int32_t j = 0; j < na; ++j) {
      int32_t t = tok[j];
      int64_t phys = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
      int64_t row = ((phys * H_kv + g) * block_size + t % block_size) * d_h;
      for (int32_t d = 0; d < d_h; ++d)
        o[d] += z[j] * (load_f64(v_cache, row + d, cache_dtype) * vscale);
    }
    for (int32_t d = 0; d < d_h; ++d) o[d] /= wsum;
    free(tok);
    free(z);
  }
  (void)num_blocks;
  if (bytes_read) *bytes_read += total_bytes;
  return status;
}

/* Chunked prefill over the paged cache: sequence s brings n_s = cu_q[s+1] - cu_q[s]
 * query tokens, rows cu_q[s] .. cu_q[s+1]-1 of q / out ([rows][H_q][d_h]); they are the
 * last n_s tokens of its context (their K/V already written), so query i sits at
 * position p = ctx[s] - n_s + i and attends, causally, to tokens 0 .. p of the paged
 * cache:
 *   out[row][h][:] = softmax_{t <= p}(scale * q[row][h] . K_t) @ V_t
 * ("PagedAttention por dentro...", section "Chunked prefill integrado con paged KV": the
 * prompt is cut into chunks that run in the same step as decodes, over the same paged
 * KV cache; "Componentes Internos de Servicio de vLLM", section "Chunked prefill
 * protege la cola del TTFT": fixed-size chunks, 512 tokens by default).  A decode is
 * the one-token chunk.  Exact two-pass softmax in fp64, as oracle_decode.
 */
int oracle_prefill(const void* q, int q_dtype, int32_t num_seqs, int32_t num_q_heads,
                   const int32_t* cu_q, const void* k_cache, const void* v_cache, int cache_dtype,
                   float k_scale, float v_scale, int32_t block_size, int32_t H_kv, int32_t d_h,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* context_lens, float scale, double* out, int num_threads) {
  if (H_kv <= 0 || num_q_heads % H_kv) return -4;
  if (!elem_bytes(q_dtype) || !elem_bytes(cache_dtype)) return -2;
  const int32_t G = num_q_heads / H_kv;
  const int64_t rows = cu_q[num_seqs];
  int status = 0;
  double kscale = cache_dtype == O_FP8 ? (double)k_scale : 1.0;
  double vscale = cache_dtype == O_FP8 ? (double)v_scale : 1.0;
#ifdef _OPENMP
  if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
#endif
  for (int64_t r = 0; r < rows * num_q_heads; ++r) {
    const int64_t row = r / num_q_heads;
    const int32_t h = (int32_t)(r % num_q_heads);
    int32_t s = 0;
    while (cu_q[s + 1] <= row) ++s;
    const int32_t n = cu_q[s + 1] - cu_q[s];
    const int32_t i = (int32_t)(row - cu_q[s]);
    const int32_t pos = context_lens[s] - n + i;
    const int32_t g = h / G;
    double* o = out + r * d_h;
    for (int32_t d = 0; d < d_h; ++d) o[d] = 0.0;
    const int32_t na = MUT(12) ? pos : pos + 1; /* tokens 0 .. pos */
    if (na <= 0) continue;
    double* z = (double*)malloc(sizeof(double) * (size_t)na);
    if (!z) { status = -7; continue; }
    const int64_t q_base = r * d_h;
    for (int32_t t = 0; t < na; ++t) {
      int64_t phys = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
      int64_t krow = ((phys * H_kv + g) * block_size + t % block_size) * d_h;
      double acc = 0.0;
      for (int32_t d = 0; d < d_h; ++d)
        acc += load_f64(q, q_base + d, q_dtype) * (load_f64(k_cache, krow + d, cache_dtype) * kscale);
      z[t] = (double)scale * acc;
    }
    double m = z[0];
    for (int32_t t = 1; t < na; ++t)
      if (z[t] > m) m = z[t];
    double wsum = 0.0;
    for (int32_t t = 0; t < na; ++t) {
      z[t] = exp(z[t] - m);
      wsum += z[t];
    }
    for (int32_t t = 0; t < na; ++t) {
      int64_t phys = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
      int64_t vrow = ((phys * H_kv + g) * block_size + t % block_size) * d_h;
      for (int32_t d = 0; d < d_h; ++d) o[d] += z[t] * (load_f64(v_cache, vrow + d, cache_dtype) * vscale);
    }
    for (int32_t d = 0; d < d_h; ++d) o[d] /= wsum;
    free(z);
  }
  return status;
}

/* The whole context (no window): the plain decode step. */
int oracle_decode(const void* q, int q_dtype, int32_t num_seqs, int32_t num_q_heads,
                  const void* k_cache, const void* v_cache, int cache_dtype, float k_scale,
                  float v_scale, int64_t num_blocks, int32_t block_size, int32_t H_kv,
                  int32_t d_h, const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, float scale, const int32_t* pairs,
                  int64_t num_pairs, double* out, int64_t* bytes_read, int num_threads) {
  return oracle_decode_window(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache_dtype,
                              k_scale, v_scale, num_blocks, block_size, H_kv, d_h, block_tables,
                              max_blocks_per_seq, context_lens, 0, 0, scale, pairs, num_pairs, out,
                              bytes_read, num_threads);
}

int oracle_mutation(void) { return ORACLE_MUTATION; }
