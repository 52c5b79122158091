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

constexpr int kBlock = PA_BLOCK_SIZE;                       // tokens per block

// ---- element traits --------------------------------------------------------------
struct F16 {
  using T = _Float16;
  static constexpr uint16_t kNaN = 0x7E00;
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
};

struct BF16 {
  using T = __bf16;
  static constexpr uint16_t kNaN = 0x7FC0;
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
};

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// A buffer resource for `bytes` bytes at p (raw buffer, no swizzle; word 3 is
// the gfx9 default format).  Loads past `bytes` return zeros without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* p, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, bytes, 0x00020000);
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

}  // namespace pa_dev
