// Internal device helpers of the kvq library (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kPageTokens = 64;
constexpr int kWave = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Bytes of the code section / whole block of one (page, KV head).
__host__ __device__ constexpr int code_bytes(int bits) { return kPageTokens * kHeadDim * bits / 8; }
__host__ __device__ constexpr int block_bytes(int bits) { return code_bytes(bits) + 4 * kPageTokens; }

// fp32 <-> fp16 bit patterns.  The conversion rounds to nearest even (the default
// rounding mode of the shader); fp16 subnormals are kept.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Element loads of the three input types as fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float get(const float* p, int i) { return p[i]; }
};
template <> struct Elem<__bf16> {
  static __device__ __forceinline__ float get(const __bf16* p, int i) { return (float)p[i]; }
};
template <> struct Elem<_Float16> {
  static __device__ __forceinline__ float get(const _Float16* p, int i) { return (float)p[i]; }
};

}  // namespace kvq
