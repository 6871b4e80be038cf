// Write path: key transform after RoPE, per-token group clip, fp16 scale/zero,
// codes, and packing into the fixed-width paged cache.
//
// Method: "WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms" §4.2 (dense
// per-KV-head key transform applied online after RoPE; values arrive already in the
// folded basis), §4.3 (QuEST: the group is one token's 128 channels, RMS-based clip),
// §5.3 (OSCAR-style percentile-clipped affine codes).  Layout: "Spend Bits Where
// Queries Look" (NOVA-KV project page), "Three requirements": every token takes the
// same number of bits in a paged cache.
//
// Work decomposition (gfx950, wave64).  Grid (token blocks, KV heads, 2): the third index
// selects keys or values, so the two halves run in separate workgroups.  A workgroup of 4
// waves handles 128 consecutive tokens of one KV head; each wave handles 32 tokens.  Lane
// l owns token l%32 and the channel half hh = l/32 (channels 64*hh .. 64*hh+63), so a
// token's group lives in two lanes and everything except one cross-lane exchange per
// group stays in-lane:
//   * transform (keys): D[out-channel][token] = T^T[out][in] . K^T[in][token] on the
//     matrix cores (32x32x16, bf16 or f16, fp32 accumulate); the rows of T^T are permuted
//     so that accumulator register r of M-tile mt on lane half hh is channel
//     64*hh + 16*mt + r.  T^T is staged once per workgroup in LDS from whole cache lines
//     of T (lane pairs swap halves to form T^T dwords; 16-byte groups XOR-swizzled).
//   * percentile clip: bottom-K / top-K insertion networks (v_med3) over the lane's
//     64 values (for K = 3 over sorted triples' candidates), one exchange with the
//     partner lane, then the order statistics; order statistics do not depend on how
//     they are found.  Positions outside the K smallest/largest use a 128-element
//     bitonic sort across the wavefront.
//   * rms clip: the 128-channel pairwise tree whose first level (stride 64) pairs the two
//     lanes of a token (one half-swap per two squares), the rest in-lane, then one
//     exchange and a correctly rounded sqrt.
//   * codes: rounded and packed a byte at a time by v_cvt_pk_u8_f32, bytes merged by shifts.
//   * keys: each lane writes its half of the token's row (16 or 32 bytes).
//   * values: when the wave's 32 tokens fill an aligned run of one page, the packed codes
//     are transposed across lanes in registers and whole words are stored; otherwise the
//     codes go through LDS as bytes and the wave merges one token at a time into its words
//     with atomic AND/OR (contiguous words per instruction), so other tokens' bits survive.
#include "kvq_device.h"
#include "kvq_encode.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kTileTokens = 32;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockTokens = kTileTokens * kWavesPerBlock;
constexpr int kTtStride = 136;   // padded LDS row of T^T (elements): spreads banks
// T^T row j keeps its 16-byte group g at group g ^ tt_swizzle(j): with the padding, the
// matrix-core operand reads stay at two lanes per bank and the staging writes (16 rows 4
// apart per instruction) drop from eight to two.
__device__ __forceinline__ int tt_swizzle(int j) { return (j >> 3) & 7; }

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<_Float16> {
  typedef half8 vec;
  static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// 64 consecutive elements (the lane's half of a token's row) as fp32.
template <typename TIn>
__device__ __forceinline__ void load_half_row(const TIn* src, float (&x)[64]) {
  if constexpr (sizeof(TIn) == 4) {
    const f32x4* p = reinterpret_cast<const f32x4*>(src);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      f32x4 w = p[q];
      x[4 * q] = w[0]; x[4 * q + 1] = w[1]; x[4 * q + 2] = w[2]; x[4 * q + 3] = w[3];
    }
  } else {
    constexpr bool bf = __is_same(TIn, __bf16);
    const u32x4* p = reinterpret_cast<const u32x4*>(src);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      u32x4 w = p[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * q + 2 * e] = half_lo_to_f32(w[e], bf);
        x[8 * q + 2 * e + 1] = half_hi_to_f32(w[e], bf);
      }
    }
  }
}

// 64 16-bit elements held as 8 x 16 B (already loaded) as fp32.
template <typename TIn>
__device__ __forceinline__ void unpack_half_row(const u32x4 (&raw)[8], float (&x)[64]) {
  constexpr bool bf = __is_same(TIn, __bf16);
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * q + 2 * e] = half_lo_to_f32(raw[q][e], bf);
      x[8 * q + 2 * e + 1] = half_hi_to_f32(raw[q][e], bf);
    }
}

// k' = k . T on the matrix cores for the wave's 32 tokens.  kop[ks]: this lane's operand
// chunk of K-step ks (elements 16*ks + 8*(lane/32) .. +7 of its token's row, loaded
// up front).  tt: T^T of the head in LDS.
template <typename TIn>
__device__ __forceinline__ void transform_mfma(const u32x4 (&kop)[8], const uint16_t* tt, int lane,
                                               float (&x)[64]) {
  typedef typename Mfma<TIn>::vec vec;
  const int rho = lane & 31, kk = lane >> 5;
  f32x16 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    vec b = __builtin_bit_cast(vec, kop[ks]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int ch = 64 * ((rho >> 2) & 1) + 16 * mt + 4 * (rho >> 3) + (rho & 3);
      const int grp = (2 * ks + kk) ^ tt_swizzle(ch);
      u32x4 araw = *reinterpret_cast<const u32x4*>(tt + ch * kTtStride + 8 * grp);
      acc[mt] = Mfma<TIn>::mma(__builtin_bit_cast(vec, araw), b, acc[mt]);
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) x[16 * mt + r] = acc[mt][r];
}

// fp32 inputs: k' = k . T with fp32 fused multiply-adds (c ascending).
__device__ __forceinline__ void transform_f32(const float* tok_row, const float* t_head, int hh,
                                              float (&x)[64]) {
#pragma unroll
  for (int m = 0; m < 64; ++m) x[m] = 0.0f;
  for (int c = 0; c < kHeadDim; ++c) {
    const float kc = tok_row[c];
    const f32x4* tr = reinterpret_cast<const f32x4*>(t_head + c * kHeadDim + 64 * hh);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      f32x4 w = tr[q];
      x[4 * q] = __builtin_fmaf(kc, w[0], x[4 * q]);
      x[4 * q + 1] = __builtin_fmaf(kc, w[1], x[4 * q + 1]);
      x[4 * q + 2] = __builtin_fmaf(kc, w[2], x[4 * q + 2]);
      x[4 * q + 3] = __builtin_fmaf(kc, w[3], x[4 * q + 3]);
    }
  }
}

// Inserts v into the sorted K smallest (lo) and K largest (hi) values seen so far.
template <int K>
__device__ __forceinline__ void insert_extreme(float v, float w, float (&lo)[K], float (&hi)[K]) {
#pragma unroll
  for (int k = K - 1; k >= 1; --k) {
    lo[k] = __builtin_amdgcn_fmed3f(lo[k - 1], lo[k], v);
    hi[k] = __builtin_amdgcn_fmed3f(hi[k - 1], hi[k], w);
  }
  lo[0] = fminf(lo[0], v);
  hi[0] = fmaxf(hi[0], w);
}

// Smallest / largest K values of the token's 128 (lane + partner lane), sorted:
// lo[k] = s[k], hi[k] = s[127-k].
template <int K>
__device__ __forceinline__ void select_extremes(const float (&x)[64], float (&lo)[K], float (&hi)[K]) {
#pragma unroll
  for (int k = 0; k < K; ++k) { lo[k] = __builtin_inff(); hi[k] = -__builtin_inff(); }
  if constexpr (K == 3) {
    // The lane's values in triples, each sorted by one min3, med3 and max3.  A value among
    // the 3 smallest is either the minimum of its triple and among the 3 smallest triple
    // minima, or the smallest triple median (a smaller median would bring its own minimum:
    // 3 smaller values), or the smallest triple maximum (its two triple-mates are smaller,
    // so nothing else is).  Mirrored for the 3 largest.  13 operations per triple instead
    // of 18 for inserting each value.
    float lmed = __builtin_inff(), lmax = __builtin_inff(), hmed = -__builtin_inff(), hmin = -__builtin_inff();
#pragma unroll
    for (int m = 0; m + 3 <= 64; m += 3) {
      const float a = x[m], b = x[m + 1], c = x[m + 2];
      const float mn = fminf(fminf(a, b), c), md = __builtin_amdgcn_fmed3f(a, b, c);
      const float mx = fmaxf(fmaxf(a, b), c);
      insert_extreme<K>(mn, mx, lo, hi);
      lmed = fminf(lmed, md);
      lmax = fminf(lmax, mx);
      hmed = fmaxf(hmed, md);
      hmin = fmaxf(hmin, mn);
    }
    insert_extreme<K>(x[63], x[63], lo, hi);
    insert_extreme<K>(lmed, hmed, lo, hi);
    insert_extreme<K>(lmax, hmin, lo, hi);
  } else {
#pragma unroll
    for (int m = 0; m < 64; ++m) insert_extreme<K>(x[m], x[m], lo, hi);
  }
  float plo[K], phi[K];
#pragma unroll
  for (int k = 0; k < K; ++k) { plo[k] = __shfl_xor(lo[k], 32); phi[k] = __shfl_xor(hi[k], 32); }
#pragma unroll
  for (int j = 0; j < K; ++j) {
#pragma unroll
    for (int k = K - 1; k >= 1; --k) {
      lo[k] = __builtin_amdgcn_fmed3f(lo[k - 1], lo[k], plo[j]);
      hi[k] = __builtin_amdgcn_fmed3f(hi[k - 1], hi[k], phi[j]);
    }
    lo[0] = fminf(lo[0], plo[j]);
    hi[0] = fmaxf(hi[0], phi[j]);
  }
}

// Clip bounds of the lane's token (both lanes of the token get the same values).
// The bitonic path sorts each token of the wave in turn through a 128-float LDS buffer.
template <int KSEL>
__device__ __forceinline__ void clip_bounds(const float (&x)[64], int quant, float alpha, int ilo,
                                            int ihi, float flo, float fhi, int lane, float* sortbuf,
                                            float& lo, float& hi) {
  if (quant == 1) {
    const float cl = rms_bound(x, alpha);
    lo = -cl;
    hi = cl;
    return;
  }
  const int ilo1 = ilo + 1 < kHeadDim ? ilo + 1 : kHeadDim - 1;
  const int ihi1 = ihi + 1 < kHeadDim ? ihi + 1 : kHeadDim - 1;
  if constexpr (KSEL > 0) {
    float bl[KSEL], bh[KSEL];
    select_extremes<KSEL>(x, bl, bh);
    lo = interpolate(order_stat<KSEL>(bl, bh, ilo), order_stat<KSEL>(bl, bh, ilo1), flo);
    hi = interpolate(order_stat<KSEL>(bl, bh, ihi), order_stat<KSEL>(bl, bh, ihi1), fhi);
  } else {
    const int hh = lane >> 5;
    lo = 0.0f;
    hi = 0.0f;
    for (int tok = 0; tok < kTileTokens; ++tok) {
      if ((lane & 31) == tok) {
#pragma unroll
        for (int m = 0; m < 64; ++m) sortbuf[64 * hh + m] = x[m];
      }
      wave_sync();
      float a = sortbuf[lane], b = sortbuf[lane + 64];
      // bitonic network over element indices i = lane (a) and i = lane + 64 (b)
      for (int k = 2; k <= kHeadDim; k <<= 1) {
        for (int j = k >> 1; j >= 1; j >>= 1) {
          if (j == 64) {
            const float mn = fminf(a, b), mx = fmaxf(a, b);
            a = mn;
            b = mx;
          } else {
            const float pa = __shfl_xor(a, j), pb = __shfl_xor(b, j);
            const bool up_a = (lane & k) == 0, up_b = ((lane + 64) & k) == 0;
            const bool low = (lane & j) == 0;
            a = (low == up_a) ? fminf(a, pa) : fmaxf(a, pa);
            b = (low == up_b) ? fminf(b, pb) : fmaxf(b, pb);
          }
        }
      }
      wave_sync();
      sortbuf[lane] = a;
      sortbuf[lane + 64] = b;
      wave_sync();
      if ((lane & 31) == tok) {
        lo = interpolate(sortbuf[ilo], sortbuf[ilo1], flo);
        hi = interpolate(sortbuf[ihi], sortbuf[ihi1], fhi);
      }
      wave_sync();
    }
  }
}

// Codes of a lane's values, packed R = 32/bits to a word (value m at bits bits*(m % R) of
// word m / R).  The clamped t in [0, L] goes through v_cvt_pk_u8_f32, which rounds to the
// nearest integer with ties to even (checked for every fp32 value in [0, 256)) and writes
// one byte of a word: byte-word s gets the codes of values i * R/4 + s (i = 0..3) in its
// bytes, and shifting it by bits * s before merging puts value e at bits bits * e.
template <int NW, int BITS>
__device__ __forceinline__ void pack_codes(const float* x, const GroupQuant& g, uint32_t (&w)[NW]) {
  constexpr int R = 32 / BITS, S = R / 4;
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    uint32_t acc = 0u;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      uint32_t b = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = __builtin_amdgcn_fmed3f(code_arg(x[R * q + i * S + s], g), 0.0f, g.lmax);
        b = __builtin_amdgcn_cvt_pk_u8_f32(c, (unsigned)i, b);
      }
      acc = s == 0 ? b : (acc | (b << (BITS * s)));
    }
    w[q] = acc;
  }
}

// 3-bit codes of the lane's 64 channels (channel 64*hh + j in x[j]) split into the two
// planes: lo[q] holds (code & 3) of channels 16q .. 16q+15 at bits 2*(j % 16) (a 2-bit
// word), hb[j / 32] bit j % 32 is bit 2 of channel j's code.
__device__ __forceinline__ void split_codes3(const float* x, const GroupQuant& g, uint32_t (&lo)[4],
                                             uint32_t (&hb)[2]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) lo[q] = 0u;
  hb[0] = hb[1] = 0u;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const float t = __builtin_amdgcn_fmed3f(code_arg(x[j], g), 0.0f, g.lmax) + 8388608.0f;
    const uint32_t code = __float_as_uint(t) & 7u;          // 0x4B000000 + code, code <= 7
    lo[j / 16] |= (code & 3u) << (2 * (j % 16));
    hb[j / 32] |= (code >> 2) << (j % 32);
  }
}

// The same for a key half row, with the high-plane words of the row built directly:
// bit 2 of channel offset u = j % 32 at key_hi_bit(u) of wh[j / 32].
__device__ __forceinline__ void split_codes3_key(const float* x, const GroupQuant& g, uint32_t (&lo)[4],
                                                 uint32_t (&wh)[2]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) lo[q] = 0u;
  wh[0] = wh[1] = 0u;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const float t = __builtin_amdgcn_fmed3f(code_arg(x[j], g), 0.0f, g.lmax) + 8388608.0f;
    const uint32_t code = __float_as_uint(t) & 7u;
    lo[j / 16] |= (code & 3u) << (2 * (j % 16));
    const int hbit = key_hi_bit(j % 32);
    wh[j / 32] |= hbit >= 2 ? (code & 4u) << (hbit - 2) : (code & 4u) >> (2 - hbit);
  }
}

// Value of lane (lane ^ d) for d = 1, 2, 4, 8 (d < 16: within a row of 16 lanes).
template <int D> __device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (D == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad [1,0,3,2]
  if constexpr (D == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad [2,3,0,1]
  if constexpr (D == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (4 << 10) | 0x1F);    // xor 4
  if constexpr (D == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false); // row rotate 8
  if constexpr (D == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (16 << 10) | 0x1F);  // xor 16
  return v;
}

// Transpose of packed codes across the G = 32/BITS lanes of a group (lanes with equal
// lane / G): before, lane r's word k holds the codes of its token for G channels (channel
// j at bits BITS*j); after, lane r's word k holds channel r of those G channels for the G
// tokens of the group (token t at bits BITS*t).  Butterfly over the lane bits: at step s the
// lanes r and r ^ 2^s swap the codes whose position differs from their own in bit s, by a
// rotate and a bit-field merge.
template <int BITS, int NW>
__device__ __forceinline__ void transpose_codes(uint32_t (&w)[NW], int lane) {
  constexpr int LOG_BITS = BITS == 1 ? 0 : (BITS == 2 ? 1 : 2);
  constexpr int STEPS = 5 - LOG_BITS;
  // step st swaps blocks of BITS * 2^st bits
  constexpr uint32_t kKeep[5] = {0x55555555u, 0x33333333u, 0x0F0F0F0Fu, 0x00FF00FFu, 0x0000FFFFu};
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int d = 1 << st;
    const bool upper = (lane >> st) & 1;
    const uint32_t keep = upper ? ~kKeep[st + LOG_BITS] : kKeep[st + LOG_BITS];
    const uint32_t amt = upper ? (uint32_t)(BITS * d) : (uint32_t)(32 - BITS * d);
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      uint32_t pv;
      switch (st) {
        case 0: pv = xor_lane<1>(w[k]); break;
        case 1: pv = xor_lane<2>(w[k]); break;
        case 2: pv = xor_lane<4>(w[k]); break;
        case 3: pv = xor_lane<8>(w[k]); break;
        default: pv = xor_lane<16>(w[k]); break;
      }
      const uint32_t rot = __builtin_amdgcn_alignbit(pv, pv, amt);
      w[k] = (w[k] & keep) | (rot & ~keep);
    }
  }
}

// Grid (token blocks, KV heads, 2): blockIdx.z = 0 writes keys, 1 writes values.  A
// workgroup of 4 waves covers 128 consecutive tokens of one head; lane l of a wave owns
// token l % 32 and the channel half l / 32.
// Four resident waves per SIMD (128 VGPRs): measured faster than three despite a few
// spilled registers, since the waves' loads then overlap other waves' arithmetic.
// THREE: the kernel also handles 3-bit codes (compiled separately, so that the 2- and
// 4-bit kernels keep their register allocation).
template <typename TIn, int KSEL, bool THREE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void append_kernel(AppendParams p) {
  // keys: T^T of the head (transform); values: codes as bytes [token][channel] per wave
  constexpr int kTtBytes = kHeadDim * kTtStride * 2;
  constexpr int kVbufBytes = kWavesPerBlock * kTileTokens * 32 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kTtBytes > kVbufBytes ? kTtBytes : kVbufBytes];
  __shared__ float sortbuf[kWavesPerBlock][kHeadDim];

  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tl = lane & 31, hh = lane >> 5;
  const int64_t tile0 = (int64_t)blockIdx.x * kBlockTokens + wave * kTileTokens;
  const int64_t i = tile0 + tl;
  const bool in_range = i < p.n;
  const TokenRef ref = in_range ? token_ref(p, i) : TokenRef{-1, 0};   // (row 0 exists)
  const int64_t slot = ref.slot;
  const bool valid = slot >= 0 && slot < p.num_pages * kPageTokens;   // others are skipped
  // a window flush's workgroup without a token to write (most of them) ends here; other
  // batches skip the vote, whose barrier would hold the row loads behind the slot loads
  if (p.slot_mode == kSlotsFlush && !__syncthreads_or(valid)) return;
  const int64_t page = valid ? slot / kPageTokens : 0;
  const int o = valid ? (int)(slot % kPageTokens) : 0;
  const TIn* row = reinterpret_cast<const TIn*>(is_v ? p.v : p.k) + (ref.src * p.heads + h) * kHeadDim;
  constexpr bool kMfmaType = sizeof(TIn) == 2;

  float x[64];
  float lo, hi;
  if (!is_v) {
    // ---------------- keys ----------------
    uint16_t* tt = reinterpret_cast<uint16_t*>(lds);
    if constexpr (kMfmaType) {
      // This thread's share of T goes out first, then the row loads: loads complete in
      // order, so T^T is staged (and the barrier passed) while the rows are still in flight.
      // Wave w reads rows 32w .. 32w + 31 of T, 8 half rows (1 KB, whole cache lines) per
      // load: load i gives lane l the 8 elements from column 64 (i % 2) + 8 (l % 8) of row
      // 32w + 8 (i / 2) + l / 8.
      const TIn* th = reinterpret_cast<const TIn*>(p.t) + (int64_t)h * kHeadDim * kHeadDim;
      u32x4 tl[8];
      if (p.t != nullptr) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          tl[i] = *reinterpret_cast<const u32x4*>(th + (32 * wave + 8 * (i >> 1) + (lane >> 3)) * kHeadDim +
                                                  64 * (i & 1) + 8 * (lane & 7));
      }
      u32x4 kraw[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        // with a transform: the matrix-core operand of K-step q; without: the half-row
        const int koff = p.t != nullptr ? 16 * q + 8 * hh : 64 * hh + 8 * q;
        kraw[q] = *reinterpret_cast<const u32x4*>(row + koff);
      }
      if (p.t != nullptr) {
        // Lanes l and l ^ 8 hold rows r and r + 1 (r even) at the same 8 columns; they swap
        // halves so that the even lane has both rows at the first 4 columns and the odd lane
        // at the last 4.  Each lane then writes, for 4 columns j, the dword (T[r][j],
        // T[r+1][j]) of T^T row j.
        // The rows j = 64 (i % 2) + 8 m + 4 odd + e (m = l % 8) all have tt_swizzle(j) = m.
        const bool odd = (lane >> 3) & 1;
        const int m = lane & 7;
        const uint32_t keep = odd ? ~0u : 0u;
        // byte selectors: the low half from row r, the high half from row r + 1, whichever
        // operand holds them (own dword for row r on even lanes, for row r + 1 on odd ones)
        const uint32_t sel_lo = odd ? 0x01000504u : 0x05040100u;
        const uint32_t sel_hi = odd ? 0x03020706u : 0x07060302u;
        uint32_t* tt32 = reinterpret_cast<uint32_t*>(tt) + (8 * m + 4 * (int)odd) * (kTtStride / 2) + (lane >> 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // own dwords for the lane's 4 columns; the partner gets the other two
          const uint32_t own0 = (keep & tl[i][2]) | (~keep & tl[i][0]);
          const uint32_t own1 = (keep & tl[i][3]) | (~keep & tl[i][1]);
          const uint32_t snd0 = (keep & tl[i][0]) | (~keep & tl[i][2]);
          const uint32_t snd1 = (keep & tl[i][1]) | (~keep & tl[i][3]);
          const uint32_t got0 = xor_lane<8>(snd0), got1 = xor_lane<8>(snd1);
          const int grp = (4 * wave + (i >> 1)) ^ m;                // swizzled 16-byte group
          uint32_t* dst = tt32 + 64 * (i & 1) * (kTtStride / 2) + 4 * grp;
          dst[0 * (kTtStride / 2)] = __builtin_amdgcn_perm(got0, own0, sel_lo);
          dst[1 * (kTtStride / 2)] = __builtin_amdgcn_perm(got0, own0, sel_hi);
          dst[2 * (kTtStride / 2)] = __builtin_amdgcn_perm(got1, own1, sel_lo);
          dst[3 * (kTtStride / 2)] = __builtin_amdgcn_perm(got1, own1, sel_hi);
        }
        __syncthreads();
        transform_mfma<TIn>(kraw, tt, lane, x);
      } else {
        unpack_half_row<TIn>(kraw, x);
      }
    } else if (p.t == nullptr) {
      load_half_row<TIn>(row + 64 * hh, x);
    } else {
      transform_f32(reinterpret_cast<const float*>(row),
                    reinterpret_cast<const float*>(p.t) + (int64_t)h * kHeadDim * kHeadDim, hh, x);
    }
    clip_bounds<KSEL>(x, p.quant_k, p.alpha_k, p.ilo, p.ihi, p.flo, p.fhi, lane, sortbuf[wave], lo, hi);
    const GroupQuant g = make_quant(lo, hi, p.bits_k);
    uint8_t* blk = p.kpool + (page * p.heads + h) * (int64_t)block_bytes(p.bits_k);
    if (p.bits_k == 2) {
      uint32_t w[4];
      pack_codes<4, 2>(x, g, w);
      if (valid) *reinterpret_cast<u32x4*>(blk + o * 32 + 16 * hh) = u32x4{w[0], w[1], w[2], w[3]};
    } else if (THREE && p.bits_k == 3) {
      uint32_t w[4], wh[2];
      split_codes3_key(x, g, w, wh);
      if (valid) {
        *reinterpret_cast<u32x4*>(blk + o * 32 + 16 * hh) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x2*>(blk + kLowPlaneBytes + o * 16 + 8 * hh) = u32x2{wh[0], wh[1]};
      }
    } else {
      uint32_t w[8];
      pack_codes<8, 4>(x, g, w);
      if (valid) {
        *reinterpret_cast<u32x4*>(blk + o * 64 + 32 * hh) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(blk + o * 64 + 32 * hh + 16) = u32x4{w[4], w[5], w[6], w[7]};
      }
    }
    if (valid) {
      uint16_t* meta = reinterpret_cast<uint16_t*>(blk + code_bytes(p.bits_k));
      meta[hh * kPageTokens + o] = hh ? g.z16 : g.s16;
    }
    return;
  }

  // ---------------- values ----------------
  if constexpr (kMfmaType) {
    u32x4 vraw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) vraw[q] = *reinterpret_cast<const u32x4*>(row + 64 * hh + 8 * q);
    unpack_half_row<TIn>(vraw, x);
  } else {
    load_half_row<TIn>(row + 64 * hh, x);
  }
  clip_bounds<KSEL>(x, p.quant_v, p.alpha_v, p.ilo, p.ihi, p.flo, p.fhi, lane, sortbuf[wave], lo, hi);
  const GroupQuant g = make_quant(lo, hi, p.bits_v);
  const int bits = p.bits_v;
  const int64_t vbb = block_bytes(bits);
  uint8_t* blk = p.vpool + (page * p.heads + h) * vbb;
  if (valid) {
    uint16_t* meta = reinterpret_cast<uint16_t*>(blk + code_bytes(bits));
    meta[hh * kPageTokens + o] = hh ? g.z16 : g.s16;
  }
  const int64_t slot0 = __shfl(slot, 0);
  const bool aligned_run = __all(valid && slot == slot0 + tl) && (slot0 % kTileTokens) == 0;
  if (aligned_run) {
    // the wave's 32 tokens fill whole words: transpose the packed codes across lanes and
    // store each word once (lane r of a group of 32/bits lanes: one channel per word)
    uint32_t* words = reinterpret_cast<uint32_t*>(p.vpool + ((slot0 / kPageTokens) * p.heads + h) * vbb);
    const int o0 = (int)(slot0 % kPageTokens);
    if (bits == 2) {
      uint32_t w[4];
      pack_codes<4, 2>(x, g, w);
      transpose_codes<2, 4>(w, lane);
      const int r = lane & 15, g16 = (lane >> 4) & 1;
      uint32_t* dst = words + (o0 / 16 + g16) * kHeadDim + 64 * hh + r;
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[16 * k] = w[k];
    } else if (THREE && bits == 3) {
      uint32_t w[4], hb[2];
      split_codes3(x, g, w, hb);
      transpose_codes<2, 4>(w, lane);                       // the low plane as 2-bit codes
      const int r = lane & 15, g16 = (lane >> 4) & 1;
      uint32_t* dst = words + (o0 / 16 + g16) * kHeadDim + 64 * hh + r;
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[16 * k] = w[k];
      // high plane: one word per channel holds the wave's 32 tokens.  A 32 x 32 bit
      // transpose over the lanes of each half turns lane tl's bits of channels 64hh + 32k + j
      // into lane tl's word k = channel 64hh + 32k + tl with token t at bit t; a byte permute
      // moves token t to value_hi_bit(t)
      transpose_codes<1, 2>(hb, lane);
      uint32_t* hw = words + kLowPlaneBytes / 4 + (o0 / 32) * kHeadDim + 64 * hh + tl;
      hw[0] = __builtin_amdgcn_perm(hb[0], hb[0], 0x03010200u);
      hw[32] = __builtin_amdgcn_perm(hb[1], hb[1], 0x03010200u);
    } else {
      uint32_t w[8];
      pack_codes<8, 4>(x, g, w);
      transpose_codes<4, 8>(w, lane);
      const int r = lane & 7, g8 = (lane >> 3) & 3;
      uint32_t* dst = words + (o0 / 8 + g8) * kHeadDim + 64 * hh + r;
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[8 * k] = w[k];
    }
    return;
  }
  // codes as bytes [token][channel] in LDS for the merge below
  uint32_t* vb = reinterpret_cast<uint32_t*>(lds) + wave * kTileTokens * 32;
  {
    uint32_t w[16];
    pack_codes<16, 8>(x, g, w);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(vb + tl * 32 + 16 * hh + 4 * q) = u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
  }
  wave_sync();
  {
    // token by token, the whole wave merges one token's codes into its 128 words (lane l:
    // channels l and l + 64), so each atomic instruction covers contiguous words; the
    // AND/OR merge keeps other tokens' bits of the shared words
    const bool three = THREE && bits == 3;
    const int per_word = three ? 16 : 32 / bits;              // (3-bit: the low plane)
    const uint32_t fmask = three ? 3u : (1u << bits) - 1u;
    for (int t = 0; t < kTileTokens; ++t) {
      const int64_t st = __shfl(slot, t);
      if (st < 0 || st >= p.num_pages * kPageTokens) continue;   // same for the whole wave
      const int ot = (int)(st % kPageTokens);
      const int sh = (ot % per_word) * (three ? 2 : bits);
      uint8_t* tblk = p.vpool + ((st / kPageTokens) * p.heads + h) * vbb;
      uint32_t* words = reinterpret_cast<uint32_t*>(tblk) + (ot / per_word) * kHeadDim;
      uint32_t* hwords = reinterpret_cast<uint32_t*>(tblk + kLowPlaneBytes) + (ot / 32) * kHeadDim;
      const int hb = value_hi_bit(ot % 32);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int c = lane + 64 * half;
        const uint32_t full = vb[t * 32 + c / 4] >> (8 * (c % 4));
        const uint32_t code = full & fmask;
        atomicAnd(words + c, ~(fmask << sh));
        atomicOr(words + c, code << sh);
        if (three) {                           // bit 2 into the high plane
          atomicAnd(hwords + c, ~(1u << hb));
          atomicOr(hwords + c, ((full >> 2) & 1u) << hb);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Small batches (a decode step's new tokens): one workgroup per (token, KV head), so the
// whole step is a few hundred instructions deep.  Lane l holds channels 2l and 2l+1.
// ---------------------------------------------------------------------------------
constexpr int kSmallMaxTokens = kSmallAppendMaxTokens;

// Five waves per (token, KV head): waves 0-3 share the key transform, wave 0 then writes
// the key and wave 4 the value.
constexpr int kSmallWaves = 5;
template <typename TIn, int KSEL>
__global__ __launch_bounds__(64 * kSmallWaves) void append_small_kernel(AppendParams p) {
  __shared__ float part[4][kHeadDim];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  append_token<TIn, KSEL, 4>(p, blockIdx.x, blockIdx.y, wave, lane, part);
}

template <typename TIn>
hipError_t launch_typed(const AppendParams& p, hipStream_t stream) {
  const int ksel = select_width(p);
  if (p.n <= kSmallMaxTokens) {
    const dim3 grid((unsigned)p.n, (unsigned)p.heads), block(64 * kSmallWaves);
    if (ksel == 3) hipLaunchKernelGGL((append_small_kernel<TIn, 3>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((append_small_kernel<TIn, 0>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((p.n + kBlockTokens - 1) / kBlockTokens), (unsigned)p.heads, 2u), block(256);
  if (p.bits_k == 3 || p.bits_v == 3) {
    if (ksel == 3) hipLaunchKernelGGL((append_kernel<TIn, 3, true>), grid, block, 0, stream, p);
    else if (ksel == 8) hipLaunchKernelGGL((append_kernel<TIn, 8, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((append_kernel<TIn, 0, true>), grid, block, 0, stream, p);
  } else {
    if (ksel == 3) hipLaunchKernelGGL((append_kernel<TIn, 3, false>), grid, block, 0, stream, p);
    else if (ksel == 8) hipLaunchKernelGGL((append_kernel<TIn, 8, false>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((append_kernel<TIn, 0, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendParams& p, int in_dtype, hipStream_t stream) {
  switch (in_dtype) {
    case 0: return launch_typed<float>(p, stream);
    case 1: return launch_typed<__bf16>(p, stream);
    default: return launch_typed<_Float16>(p, stream);
  }
}

}  // namespace kvq
