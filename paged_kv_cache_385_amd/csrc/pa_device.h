// Device-side building blocks shared by the library's kernels (gfx950):
// vector types, the 16-bit element traits with their matrix-core products, and
// the 16-byte tile loads through bounded buffer resources.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/pa.h"

namespace pa_dev {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = PA_BLOCK_SIZE;                       // tokens per block

// ---- element traits --------------------------------------------------------------
struct F16 {
  using T = _Float16;
  static constexpr uint16_t kNaN = 0x7E00;
  // E4M3 codes in bytes 0, 1 (hi = false) or 2, 3 (hi = true) of w, as two float16
  // (every E4M3 value is exact in float16)
  __device__ static uint32_t from_fp8_lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  }
  __device__ static uint32_t from_fp8_hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  }
  __device__ static f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static f32x4 mfma_pv(u16x4 a, u16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static uint16_t from_float(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  __device__ static float to_float(uint16_t x) {
    return static_cast<float>(__builtin_bit_cast(_Float16, x));
  }
  // two values rounded to nearest even, a in the low half: one operand word
  __device__ static uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
  }
  static constexpr uint32_t kOne2 = 0x3C003C00u;     // two 1.0
};

struct BF16 {
  using T = __bf16;
  static constexpr uint16_t kNaN = 0x7FC0;
  // E4M3 codes in bytes 0, 1 / 2, 3 of w, as two bfloat16 (exact)
  __device__ static uint32_t from_fp8_lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  }
  __device__ static uint32_t from_fp8_hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  }
  __device__ static f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static f32x4 mfma_pv(u16x4 a, u16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
  __device__ static uint16_t from_float(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
  __device__ static float to_float(uint16_t x) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(x) << 16);
  }
  __device__ static uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  }
  static constexpr uint32_t kOne2 = 0x3F803F80u;
};

// Eight E4M3 codes (two words, in memory order) as eight 16-bit elements: one
// matrix-core operand, in the element order the 16-bit pools use.
template <class E>
__device__ __forceinline__ u32x4 widen_fp8(uint32_t a, uint32_t b) {
  return u32x4{E::from_fp8_lo(a), E::from_fp8_hi(a), E::from_fp8_lo(b), E::from_fp8_hi(b)};
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// A buffer resource for `bytes` bytes at p (raw buffer, no swizzle; word 3 is
// the gfx9 default format).  Loads past `bytes` return zeros without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* p, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
// 16 bytes of a K/V tile.  Tiles are read once per launch unless blocks are
// shared: the streaming form sets the non-temporal bit, which keeps them from
// displacing reusable lines and reads HBM markedly faster on gfx950.
template <bool kStream>
__device__ __forceinline__ u32x4 load_tile(__amdgpu_buffer_rsrc_t r, int32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kStream ? 2 : 0));
}
__device__ __forceinline__ void store16(uint16_t* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over lanes l, l ^ 16, l ^ 32, l ^ 48 -- the four lanes that hold one
// column of a 16x16 matrix-core tile -- with gfx950's lane swaps, which stay in
// the vector ALU.  v_permlane16_swap_b32 a, b exchanges the odd 16-lane rows of a
// with the even rows of b; v_permlane32_swap_b32 a, b the upper half of a with
// the lower half of b.  Applied to two copies of x, each leaves x and its partner
// (x[l ^ 16], resp. x[l ^ 32]) in the pair, in every lane.  Written as inline
// assembly with both registers as outputs, since the builtins' second result is
// not kept apart from the first by the compiler; the s_nop gives the wait states
// the compiler itself puts before these instructions.
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float col_max4(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  a = b = __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
  swap32(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
// max of three floats as one v_max3_f32, without the canonicalising moves the
// compiler puts before fmaxf on values it cannot prove canonical (matrix-core
// results).  A NaN operand yields the larger of the others (IEEE mode).
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// col_max4 with the same raw maxima
__device__ __forceinline__ float col_max4_raw(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  const float m = max3_raw(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b),
                           __builtin_bit_cast(float, b));
  a = b = __builtin_bit_cast(uint32_t, m);
  swap32(a, b);
  return max3_raw(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float col_sum4(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  a = b = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
  swap32(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// ---- 8-bit floating point (OCP E4M3) cache codes -----------------------------------
// Code of x / scale: the division in float32, round to nearest even, saturated at
// +-448 (the hardware conversion turns larger magnitudes into NaN, so they are
// clamped first), NaN as 0x7F.
__device__ __forceinline__ uint32_t fp8_code(float x, float scale) {
  const float y = x / scale;
  if (y != y) return 0x7Fu;
  const float c = fminf(fmaxf(y, -448.f), 448.f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false)) & 0xFFu;
}

}  // namespace pa_dev
