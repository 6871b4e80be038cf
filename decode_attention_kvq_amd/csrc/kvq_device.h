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

// 3-bit codes are two bit planes.  The low plane (bits 0-1 of every code) is laid out as a
// 2-bit code section; the high plane (bit 2) follows it, at byte kLowPlaneBytes:
//   keys    token o's 128 bits are the words o*4 + c/32, channel offset u = c % 32 at bit
//           key_hi_bit(u) (so that shifts and one AND put 8 of them at bit 2 of fp4 nibbles
//           in the order the 2-bit plane gives its codes)
//   values  word (o/32)*128 + c holds tokens 32*(o/32) .. +31 of channel c, token offset
//           t = o % 32 at bit value_hi_bit(t) (a 16-token run of one lane group sits in one
//           byte of each 16-bit half)
constexpr int kLowPlaneBytes = code_bytes(2);
__host__ __device__ constexpr int key_hi_bit(int u) { return 4 * ((u % 16) / 2) + 2 * (u / 16) + u % 2; }
__host__ __device__ constexpr int value_hi_bit(int t) { return t % 8 + 16 * ((t / 8) % 2) + 8 * (t / 16); }

// fp32 -> fp16 bits with the hardware conversion (operands of matrix-core products,
// where the last rounding bit does not matter).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

// fp32 -> fp16 bits, round to nearest with ties to even, in integer arithmetic from the
// binary16 definition (1 sign, 5 exponent bits with bias 15, 10 fraction bits).  Used for
// stored scales and zeros, which must round ties to even.  |x| >= 65520 gives infinity.
__device__ __forceinline__ uint16_t f32_to_f16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x7F800000u) return (uint16_t)(sign | (a > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);
  if (a < 0x38800000u) {
    // below 2^-14 the fp16 spacing is 2^-24: scale exactly, round to an integer (RNE)
    const float m = rintf(__uint_as_float(a) * 16777216.0f);
    return (uint16_t)(sign | (uint32_t)m);
  }
  uint32_t h = (((a >> 23) - 112u) << 10) | ((a >> 13) & 0x3FFu);
  const uint32_t rem = a & 0x1FFFu;
  h += (rem > 0x1000u) || (rem == 0x1000u && (h & 1u));
  return (uint16_t)(sign | h);
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
