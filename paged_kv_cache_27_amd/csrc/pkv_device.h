// Device-side helpers for the gfx950 paged KV kernels: element types, conversions,
// 16-lane DPP reductions and MFMA wrappers.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum Dt : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

template <int DT> struct DtInfo;
template <> struct DtInfo<kF32> { static constexpr int bytes = 4; };
template <> struct DtInfo<kF16> { static constexpr int bytes = 2; };
template <> struct DtInfo<kBF16> { static constexpr int bytes = 2; };
template <> struct DtInfo<kFP8> { static constexpr int bytes = 1; };

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8_t __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x2_t __attribute__((__vector_size__(2 * sizeof(float))));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef _Float16 f16x2_t __attribute__((__vector_size__(2 * sizeof(_Float16))));

static constexpr float kNegInf = -__builtin_huge_valf();
static constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// ---- scalar conversions to fp32 (exact) ----------------------------------------
__device__ __forceinline__ float bf16lo_f32(uint32_t w) { return bits_f32(w << 16); }
__device__ __forceinline__ float bf16hi_f32(uint32_t w) { return bits_f32(w & 0xffff0000u); }
__device__ __forceinline__ float f16lo_f32(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi_f32(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// 8 consecutive stored elements -> 8 floats.  `p` points at 8 * bytes of data that
// the caller has already loaded into registers (as 32-bit words).
template <int DT> struct Unpack8;
template <> struct Unpack8<kF32> {
  static constexpr int words = 8;
  __device__ __forceinline__ static void run(const uint32_t* w, float* o) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = bits_f32(w[i]);
  }
};
template <> struct Unpack8<kBF16> {
  static constexpr int words = 4;
  __device__ __forceinline__ static void run(const uint32_t* w, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = bf16lo_f32(w[i]);
      o[2 * i + 1] = bf16hi_f32(w[i]);
    }
  }
};
template <> struct Unpack8<kF16> {
  static constexpr int words = 4;
  __device__ __forceinline__ static void run(const uint32_t* w, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = f16lo_f32(w[i]);
      o[2 * i + 1] = f16hi_f32(w[i]);
    }
  }
};
template <> struct Unpack8<kFP8> {
  static constexpr int words = 2;
  // gfx950 converts OCP e4m3fn pairs in hardware; the scale operand is 1.0 (the
  // per-tensor scale is folded into the softmax scale / final normalisation).
  __device__ __forceinline__ static void run(const uint32_t* w, float* o) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w[i], 1.0f, false);
      f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w[i], 1.0f, true);
      o[4 * i + 0] = a[0];
      o[4 * i + 1] = a[1];
      o[4 * i + 2] = b[0];
      o[4 * i + 3] = b[1];
    }
  }
};

// ---- fp32 -> stored formats -----------------------------------------------------
// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32 rounds to nearest even
}

// out[idx] = x rounded to nearest-even in the output dtype (f32 / bf16 / f16).
__device__ __forceinline__ void store_out(void* out, size_t idx, int out_dtype, float x) {
  if (out_dtype == kF32)
    ((float*)out)[idx] = x;
  else if (out_dtype == kBF16)
    ((uint16_t*)out)[idx] = f32_to_bf16_rne(x);
  else
    ((uint16_t*)out)[idx] = f32_to_f16_rne(x);
}

// fp32 -> OCP e4m3fn, round to nearest even, saturating to +-448 (infinities
// included), NaN -> NaN.  Pure integer arithmetic on the fp32 bit pattern.
__device__ __forceinline__ uint32_t f32_to_e4m3_satfinite(float y) {
  const uint32_t u = f32_bits(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;   // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |y| >= 448 (and inf) -> 448
  if (a < 0x3c800000u) {                      // |y| < 2^-6: subnormal grid m * 2^-9
    // |y| * 512 is exact; rintf rounds half to even.  Result 0..8 (8 = 2^-6, the
    // first normal code, which the encoding reaches contiguously).
    const uint32_t m = (uint32_t)__builtin_rintf(bits_f32(a) * 512.0f);
    return sign | m;
  }
  // Normal range: keep 8 exponent + 3 fraction bits, round the 20 dropped bits to
  // nearest even (a carry moves into the exponent), then rebias 127 -> 7.
  const uint32_t kept = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  return sign | (kept - (120u << 3));
}

// ---- 16-lane (one DPP row) all-reductions ---------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return bits_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f32_bits(x), CTRL, 0xf, 0xf, true));
}
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror: after the
// four steps every lane of a 16-lane row holds the row's result.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- K/V loads -------------------------------------------------------------------
// K/V tiles are read through buffer resources that cover exactly one 16-token chunk:
// a resource of size 0 turns every load through it into zeros without a memory
// access, which the decode pipeline uses for the padding steps past a range's end.
// NT selects the nontemporal (streaming) cache policy.  A decode reads each cached
// K/V byte once unless blocks are shared between sequences; for once-read data the
// streaming policy measured ~5 % more read bandwidth on the decode's tile pattern on
// gfx950, while for shared blocks it evicts lines other readers are about to reuse.
constexpr int kRsrcWord3 = 0x00020000;  // raw untyped 32-bit buffer access on gfx9
constexpr int kAuxNT = 2;               // buffer-load cache policy bit: nontemporal
constexpr int kAuxDevice = 16;          // buffer-access cache policy bit: device scope (sc1)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// base and bytes must be the same in every lane of the wave.  They are moved to scalar
// registers explicitly: a resource the compiler cannot prove uniform is wrapped, per
// load, in a loop over the distinct values of the lanes, which also defeats its
// vector-memory wait counting across a pipelined loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  const uint64_t v = (uint64_t)(uintptr_t)base;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)u, (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}
template <bool NT>
__device__ __forceinline__ uint4 load_kv16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4_t x = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? kAuxNT : 0));
  return make_uint4(x.x, x.y, x.z, x.w);
}
template <bool NT>
__device__ __forceinline__ uint2 load_kv8(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x2_t x = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, NT ? kAuxNT : 0));
  return make_uint2(x.x, x.y);
}
template <bool NT>
__device__ __forceinline__ uint32_t load_kv4(__amdgpu_buffer_rsrc_t r, int off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, NT ? kAuxNT : 0);
}

}  // namespace pkv
