// Dequantize cached tokens to fp32: x^ = fma(code, scale, zero) with the stored fp16
// scale and zero of the token's group.  Same page layout as the write path ("Spend Bits
// Where Queries Look", NOVA-KV project page, "Three requirements": fixed bits per
// token).  Used for inspection and tests; the decode kernel never materialises x^.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

// One thread per (token, head, 4 channels).  3-bit codes are read from their two planes.
__global__ __launch_bounds__(256) void dequant_kernel(DequantParams p) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = p.n * p.heads * (kHeadDim / 4);
  if (gid >= total) return;
  const int c4 = (int)(gid % (kHeadDim / 4));
  const int h = (int)((gid / (kHeadDim / 4)) % p.heads);
  const int64_t i = gid / ((int64_t)(kHeadDim / 4) * p.heads);
  const int64_t slot = p.slots[i];
  if (slot < 0 || slot >= p.num_pages * kPageTokens) return;
  const int64_t page = slot / kPageTokens;
  const int o = (int)(slot % kPageTokens);
  const int bits = p.bits;
  const uint8_t* blk = p.pool + (page * p.heads + h) * (int64_t)block_bytes(bits);
  const uint16_t* meta = reinterpret_cast<const uint16_t*>(blk + code_bytes(bits));
  const float sf = f16_bits_to_f32(meta[o]), zf = f16_bits_to_f32(meta[kPageTokens + o]);
  const uint32_t* words = reinterpret_cast<const uint32_t*>(blk);
  const int per_word = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 4 * c4 + e;
    uint32_t code;
    if (bits == 3) {
      const uint32_t* hi = words + kLowPlaneBytes / 4;
      if (p.which == 0) {
        code = ((words[o * 8 + c / 16] >> (2 * (c % 16))) & 3u) |
               (((hi[o * 4 + c / 32] >> key_hi_bit(c % 32)) & 1u) << 2);
      } else {
        code = ((words[(o / 16) * kHeadDim + c] >> (2 * (o % 16))) & 3u) |
               (((hi[(o / 32) * kHeadDim + c] >> value_hi_bit(o % 32)) & 1u) << 2);
      }
    } else if (p.which == 0) {
      code = (words[o * (kHeadDim / per_word) + c / per_word] >> ((c % per_word) * bits)) & mask;
    } else {
      code = (words[(o / per_word) * kHeadDim + c] >> ((o % per_word) * bits)) & mask;
    }
    r[e] = __builtin_fmaf((float)code, sf, zf);
  }
  *reinterpret_cast<f32x4*>(p.out + (i * p.heads + h) * kHeadDim + 4 * c4) = r;
}

}  // namespace

hipError_t launch_dequant(const DequantParams& p, hipStream_t stream) {
  const int64_t total = p.n * p.heads * (kHeadDim / 4);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvq
