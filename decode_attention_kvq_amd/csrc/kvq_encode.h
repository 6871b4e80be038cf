// Per-group encoding of the write path: clip bounds, fp16 scale and zero, codes, the
// one-token-per-workgroup append, and where a token goes (slot modes).
//
// Method: "WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms" §4.2 (key
// transform after RoPE), §4.3 (RMS clip of a token's 128-channel group), §5.3
// (percentile-clipped affine codes); "Spend Bits Where Queries Look", "Three
// requirements" (fixed bits per token in a paged cache).
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __forceinline__ float half_lo_to_f32(uint32_t w, bool bf16) {
  return bf16 ? __uint_as_float(w << 16) : f16_bits_to_f32(w & 0xFFFFu);
}
__device__ __forceinline__ float half_hi_to_f32(uint32_t w, bool bf16) {
  return bf16 ? __uint_as_float(w & 0xFFFF0000u) : f16_bits_to_f32(w >> 16);
}

template <int K>
__device__ __forceinline__ float order_stat(const float (&lo)[K], const float (&hi)[K], int r) {
  float v = lo[0];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    v = (r == k) ? lo[k] : v;
    v = (r == kHeadDim - 1 - k) ? hi[k] : v;
  }
  return v;
}

#pragma clang fp contract(off)

__device__ __forceinline__ float interpolate(float s0, float s1, float f) {
  return __builtin_fmaf(f, s1 - s0, s0) + 0.0f;
}

// Sum of squares of the token's 128 values in the encoder's order: one pairwise tree over
// the channel index c (stride 64, 32, ..., 1: element c < stride adds element c + stride).
// The lane holds channels 64*hh + m in x[m] and its partner lane (lane ^ 32) the other
// half, so stride 64 adds the two lanes' m-th squares.  One half-swap of the squares of
// m = 2j and 2j + 1 puts both partners' values of 2j in the low lanes and of 2j + 1 in the
// high lanes, so each lane adds one of the two sums: t[j] is c = 2j (low lanes) or 2j + 1
// (high lanes).  Strides 32 .. 2 then pair t[j] with t[j + 16 .. 1] in-lane, and stride 1
// adds the partners' t[0].  Additions commute, so both lanes end with the same total.
__device__ __forceinline__ float rms_bound(const float (&x)[64], float alpha) {
  float t[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float a = x[2 * j] * x[2 * j], b = x[2 * j + 1] * x[2 * j + 1];
    // lanes 32..63 of a trade places with lanes 0..31 of b
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    t[j] = __uint_as_float((uint32_t)r[0]) + __uint_as_float((uint32_t)r[1]);
  }
#pragma unroll
  for (int stride = 16; stride >= 1; stride >>= 1)
#pragma unroll
    for (int j = 0; j < stride; ++j) t[j] = t[j] + t[j + stride];
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[0]), __float_as_uint(t[0]), false, false);
  const float total = __uint_as_float((uint32_t)r[0]) + __uint_as_float((uint32_t)r[1]);
  const float rms = sqrtf(total / 128.0f);
  return alpha * rms;
}

__device__ __forceinline__ float sat_f16(float v) { return fminf(fmaxf(v, -65504.0f), 65504.0f); }

struct GroupQuant {
  float zf, r, lmax;
  uint16_t s16, z16;
};

__device__ __forceinline__ GroupQuant make_quant(float lo, float hi, int bits) {
  GroupQuant g;
  g.lmax = (float)((1 << bits) - 1);
  const float s = (hi - lo) / g.lmax;
  g.s16 = f32_to_f16_rne(sat_f16(s));
  g.z16 = f32_to_f16_rne(sat_f16(lo));
  const float sf = f16_bits_to_f32(g.s16);
  g.zf = f16_bits_to_f32(g.z16);
  g.r = (sf == 0.0f) ? 0.0f : 1.0f / sf;
  return g;
}

// (x - zero) * r with two separate roundings (the encoder's definition of the code argument)
__device__ __forceinline__ float code_arg(float x, const GroupQuant& g) { return (x - g.zf) * g.r; }

#pragma clang fp contract(on)

// ---------------------------------------------------------------------------------
// One token per workgroup: lane l of a wave holds channels 2l and 2l+1 of the token.
// ---------------------------------------------------------------------------------
template <typename TIn> __device__ __forceinline__ float2 load_pair(const TIn* row, int l) {
  if constexpr (sizeof(TIn) == 4) {
    return reinterpret_cast<const float2*>(row)[l];
  } else {
    constexpr bool bf = __is_same(TIn, __bf16);
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[l];
    return float2{half_lo_to_f32(w, bf), half_hi_to_f32(w, bf)};
  }
}

// Bitonic sort of the wave's 128 values (element i: lane i's a for i < 64, lane i-64's b),
// ascending.
__device__ __forceinline__ void wave_sort128(float& a, float& b, int lane) {
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
}
// Sorted element r (uniform r).
__device__ __forceinline__ float sorted_at(float a, float b, int r) {
  return r < 64 ? __shfl(a, r) : __shfl(b, r - 64);
}

// Cross-lane exchanges on the VALU (no LDS): the two values of a lane pair, in some
// order, for the pairings lane ^ 1, ^ 2 (quad permutes), 7 - lane within 8 (half-row
// mirror), lane ^ 8 (row rotate), lane ^ 16 and lane ^ 32 (row swaps).  Every use below is
// symmetric in the pair.
template <int LVL>
__device__ __forceinline__ void pair_of(float v, float& x0, float& x1) {
  const int u = __float_as_int(v);
  if constexpr (LVL <= 3) {
    constexpr int ctrl = LVL == 0 ? 0xB1 : LVL == 1 ? 0x4E : LVL == 2 ? 0x141 : 0x128;
    x0 = v;
    x1 = __int_as_float(__builtin_amdgcn_mov_dpp(u, ctrl, 0xF, 0xF, false));
  } else {
    auto r = LVL == 4 ? __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false)
                      : __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    x0 = __uint_as_float((uint32_t)r[0]);
    x1 = __uint_as_float((uint32_t)r[1]);
  }
}

// Bottom-3 / top-3 of the wave's 128 values (2 a lane), in every lane: each lane starts
// from its pair, then six levels merge two sorted triples (k-th smallest of two sorted
// lists: the smallest over splits of max(A[i-1], B[k-1-i])).
template <int LVL>
__device__ __forceinline__ void merge3(float (&lo)[3], float (&hi)[3]) {
  float l0[3], l1[3], h0[3], h1[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    pair_of<LVL>(lo[k], l0[k], l1[k]);
    pair_of<LVL>(hi[k], h0[k], h1[k]);
  }
  lo[0] = fminf(l0[0], l1[0]);
  lo[1] = fminf(fminf(l0[1], l1[1]), fmaxf(l0[0], l1[0]));
  lo[2] = fminf(fminf(l0[2], l1[2]), fminf(fmaxf(l0[0], l1[1]), fmaxf(l0[1], l1[0])));
  hi[0] = fmaxf(h0[0], h1[0]);
  hi[1] = fmaxf(fmaxf(h0[1], h1[1]), fminf(h0[0], h1[0]));
  hi[2] = fmaxf(fmaxf(h0[2], h1[2]), fmaxf(fminf(h0[0], h1[1]), fminf(h0[1], h1[0])));
}
__device__ __forceinline__ void wave_extremes3(float a, float b, float (&lo)[3], float (&hi)[3]) {
  lo[0] = fminf(a, b);
  lo[1] = fmaxf(a, b);
  lo[2] = __builtin_inff();
  hi[0] = lo[1];
  hi[1] = lo[0];
  hi[2] = -__builtin_inff();
  merge3<0>(lo, hi);
  merge3<1>(lo, hi);
  merge3<2>(lo, hi);
  merge3<3>(lo, hi);
  merge3<4>(lo, hi);
  merge3<5>(lo, hi);
}

#pragma clang fp contract(off)
// Sum of squares in the encoder's order: one pairwise tree over the channel index (stride
// 64, 32, ..., 1).  Channel 2l+e is (lane l, e), so channel stride 64 pairs lanes l and
// l + 32 (a half swap), strides 32 .. 2 pair lanes m and m + 16 .. m + 1 (lane ^ 16 .. ^ 1
// for the lanes m < stride whose sums the tree keeps), and stride 1 adds a lane's two
// values; additions commute, so each level adds the pair and every lane ends with the total.
__device__ __forceinline__ float wave_rms_bound(float a, float b, float alpha) {
  float sa = a * a, sb = b * b, x0, x1, y0, y1;
  pair_of<5>(sa, x0, x1); pair_of<5>(sb, y0, y1); sa = x0 + x1; sb = y0 + y1;     // 64
  pair_of<4>(sa, x0, x1); pair_of<4>(sb, y0, y1); sa = x0 + x1; sb = y0 + y1;     // 32
  pair_of<3>(sa, x0, x1); pair_of<3>(sb, y0, y1); sa = x0 + x1; sb = y0 + y1;     // 16
  x1 = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(sa), (4 << 10) | 0x1F));
  y1 = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(sb), (4 << 10) | 0x1F));
  sa = sa + x1; sb = sb + y1;                                                     // 8
  pair_of<1>(sa, x0, x1); pair_of<1>(sb, y0, y1); sa = x0 + x1; sb = y0 + y1;     // 4
  pair_of<0>(sa, x0, x1); pair_of<0>(sb, y0, y1); sa = x0 + x1; sb = y0 + y1;     // 2
  return alpha * sqrtf((sa + sb) / 128.0f);                                       // 1
}
#pragma clang fp contract(on)

// Quantizes the token's 128 values (lane l: channels 2l, 2l+1) and stores codes and
// metadata of one (token, head) in the key (is_v = false) or value block.
template <int KSEL>
__device__ __forceinline__ void small_quantize_store(float a, float b, bool is_v, int64_t page, int o, int h,
                                                     int lane, const AppendParams& p) {
  const int quant = is_v ? p.quant_v : p.quant_k;
  const int bits = is_v ? p.bits_v : p.bits_k;
  float lo, hi;
  if (quant == 1) {
    const float cl = wave_rms_bound(a, b, is_v ? p.alpha_v : p.alpha_k);
    lo = -cl;
    hi = cl;
  } else if (KSEL == 3) {
    float bl[3], bh[3];
    wave_extremes3(a, b, bl, bh);
    const int ilo1 = p.ilo + 1 < kHeadDim ? p.ilo + 1 : kHeadDim - 1;
    const int ihi1 = p.ihi + 1 < kHeadDim ? p.ihi + 1 : kHeadDim - 1;
    lo = interpolate(order_stat<3>(bl, bh, p.ilo), order_stat<3>(bl, bh, ilo1), p.flo);
    hi = interpolate(order_stat<3>(bl, bh, p.ihi), order_stat<3>(bl, bh, ihi1), p.fhi);
  } else {
    float sa = a, sb = b;
    wave_sort128(sa, sb, lane);
    const int ilo1 = p.ilo + 1 < kHeadDim ? p.ilo + 1 : kHeadDim - 1;
    const int ihi1 = p.ihi + 1 < kHeadDim ? p.ihi + 1 : kHeadDim - 1;
    lo = interpolate(sorted_at(sa, sb, p.ilo), sorted_at(sa, sb, ilo1), p.flo);
    hi = interpolate(sorted_at(sa, sb, p.ihi), sorted_at(sa, sb, ihi1), p.fhi);
  }
  const GroupQuant g = make_quant(lo, hi, bits);
  // rint by the fp32 addition of 2^23 (the sum's bit pattern is 0x4B000000 + code)
  const uint32_t code_a = __float_as_uint(__builtin_amdgcn_fmed3f(code_arg(a, g), 0.0f, g.lmax) + 8388608.0f) - 0x4B000000u;
  const uint32_t code_b = __float_as_uint(__builtin_amdgcn_fmed3f(code_arg(b, g), 0.0f, g.lmax) + 8388608.0f) - 0x4B000000u;
  uint8_t* blk = (is_v ? p.vpool : p.kpool) + (page * p.heads + h) * (int64_t)block_bytes(bits);
  if (lane < 2) {
    uint16_t* meta = reinterpret_cast<uint16_t*>(blk + code_bytes(bits));
    meta[lane * kPageTokens + o] = lane ? g.z16 : g.s16;
  }
  if (bits == 3) {
    if (!is_v) {
      // low plane: the 2-bit token row of (code & 3); high plane: bit 2 of both channels at
      // key_hi_bit of their offsets, OR-ed over the 16 lanes of a word (quads, half-row
      // mirror, row mirror)
      uint32_t wl = ((code_a & 3u) | ((code_b & 3u) << 2)) << (4 * (lane % 8));
      wl |= (uint32_t)__builtin_amdgcn_mov_dpp((int)wl, 0xB1, 0xF, 0xF, false);
      wl |= (uint32_t)__builtin_amdgcn_mov_dpp((int)wl, 0x4E, 0xF, 0xF, false);
      wl |= (uint32_t)__builtin_amdgcn_mov_dpp((int)wl, 0x141, 0xF, 0xF, false);
      uint32_t wh = ((code_a >> 2) | ((code_b >> 2) << 1)) << key_hi_bit((2 * lane) % 32);
      wh |= (uint32_t)__builtin_amdgcn_mov_dpp((int)wh, 0xB1, 0xF, 0xF, false);
      wh |= (uint32_t)__builtin_amdgcn_mov_dpp((int)wh, 0x4E, 0xF, 0xF, false);
      wh |= (uint32_t)__builtin_amdgcn_mov_dpp((int)wh, 0x141, 0xF, 0xF, false);
      wh |= (uint32_t)__builtin_amdgcn_mov_dpp((int)wh, 0x140, 0xF, 0xF, false);
      if (lane % 8 == 0) reinterpret_cast<uint32_t*>(blk + o * 32)[lane / 8] = wl;
      if (lane % 16 == 0) reinterpret_cast<uint32_t*>(blk + kLowPlaneBytes + o * 16)[lane / 16] = wh;
    } else {
      // low plane words (o/16)*128 + c at bit 2*(o%16); high plane words (o/32)*128 + c at
      // value_hi_bit(o%32); other tokens' bits are kept
      const int sh = 2 * (o % 16), hb = value_hi_bit(o % 32);
      uint32_t* wl = reinterpret_cast<uint32_t*>(blk) + (o / 16) * kHeadDim + 2 * lane;
      uint32_t* wh = reinterpret_cast<uint32_t*>(blk + kLowPlaneBytes) + (o / 32) * kHeadDim + 2 * lane;
      atomicAnd(wl, ~(3u << sh));
      atomicOr(wl, (code_a & 3u) << sh);
      atomicAnd(wl + 1, ~(3u << sh));
      atomicOr(wl + 1, (code_b & 3u) << sh);
      atomicAnd(wh, ~(1u << hb));
      atomicOr(wh, (code_a >> 2) << hb);
      atomicAnd(wh + 1, ~(1u << hb));
      atomicOr(wh + 1, (code_b >> 2) << hb);
    }
  } else if (!is_v) {
    // token row: word w of 32/bits channels; lane l's pair sits at bits 2*bits*(l % (16/bits))
    const int lpw = 16 / bits;                  // lanes per word
    uint32_t wv = (code_a | (code_b << bits)) << (2 * bits * (lane % lpw));
    // OR over the word's lanes: quad permutes, then (8 lanes) the half-row mirror
    wv |= (uint32_t)__builtin_amdgcn_mov_dpp((int)wv, 0xB1, 0xF, 0xF, false);
    wv |= (uint32_t)__builtin_amdgcn_mov_dpp((int)wv, 0x4E, 0xF, 0xF, false);
    if (lpw == 8) wv |= (uint32_t)__builtin_amdgcn_mov_dpp((int)wv, 0x141, 0xF, 0xF, false);
    if (lane % lpw == 0) reinterpret_cast<uint32_t*>(blk + o * (kHeadDim * bits / 8))[lane / lpw] = wv;
  } else {
    // channel-major words: channel c's word (o / R) at bits bits * (o % R); other tokens'
    // bits of the words are kept
    const int R = 32 / bits;
    const uint32_t fmask = (1u << bits) - 1u;
    const int sh = (o % R) * bits;
    uint32_t* words = reinterpret_cast<uint32_t*>(blk) + (o / R) * kHeadDim + 2 * lane;
    atomicAnd(words, ~(fmask << sh));
    atomicOr(words, code_a << sh);
    atomicAnd(words + 1, ~(fmask << sh));
    atomicOr(words + 1, code_b << sh);
  }
}

// Cache slot (negative: skip the token) and source row (of p.k / p.v) of token i.
struct TokenRef {
  int64_t slot, src;
};
__device__ __forceinline__ int64_t window_cache_slot(const AppendParams& p, int64_t b, int64_t j) {
  if (j < 0 || j / kPageTokens >= p.max_pages) return -1;
  const int32_t pid = p.block_table[b * p.max_pages + j / kPageTokens];
  return pid < 0 ? -1 : (int64_t)pid * kPageTokens + j % kPageTokens;
}
__device__ __forceinline__ TokenRef token_ref(const AppendParams& p, int64_t i) {
  if (p.slot_mode == kSlotsGiven) return {p.slots[i], i};
  if (p.slot_mode == kSlotsPrefill) {
    // sequence b with cu_seqlens[b] <= i < cu_seqlens[b + 1]; the middle positions
    // [sink, sink + quantized) of a fresh prompt go to cache index position - sink
    int lo = 0, hi = p.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.cu_seqlens[mid] <= i) lo = mid;
      else hi = mid;
    }
    const int64_t pos = i - p.cu_seqlens[lo];
    const int nq = window_quantized(p.cu_seqlens[lo + 1] - p.cu_seqlens[lo], p.win);
    if (pos < p.win.sink || pos >= p.win.sink + nq) return {-1, i};
    return {window_cache_slot(p, lo, pos - p.win.sink), i};
  }
  // flush after a decode step: sequence b quantizes the batch that its new position made
  // eligible (if any), reading the window row's ring slots
  const int64_t b = i / p.win.flush;
  const int f = (int)(i % p.win.flush);
  const int len = max(p.seq_lens[b], 0);
  const int q0 = window_quantized(max(len - 1, 0), p.win), q1 = window_quantized(len, p.win);
  const int row = p.win_rows ? p.win_rows[b] : (int)b;
  if (f >= q1 - q0 || row < 0 || row >= p.num_rows) return {-1, 0};
  const int j = q0 + f;
  return {window_cache_slot(p, b, j), (int64_t)row * window_width(p.win) + window_slot(p.win.sink + j, p.win)};
}

// The append of token i (its row of p.k / p.v from token_ref) for KV head h by one workgroup: waves 0-3 each
// multiply a quarter of the rows of T (all their loads in flight at once), wave 0 adds the
// four partial products in order and writes the key, wave VW writes the value (before the
// workgroup barrier when VW >= 4, after it otherwise).  Every wave of the workgroup must
// call it (it holds one barrier); part: LDS scratch [4][128].
template <typename TIn, int KSEL, int VW>
__device__ __forceinline__ void append_token(const AppendParams& p, int64_t i, int h, int wave, int lane,
                                             float (*part)[kHeadDim]) {
  const TokenRef ref = token_ref(p, i);
  const int64_t slot = ref.slot;
  if (slot < 0 || slot >= p.num_pages * kPageTokens) return;   // skipped (whole workgroup)
  const int64_t page = slot / kPageTokens;
  const int o = (int)(slot % kPageTokens);
  const TIn* krow = reinterpret_cast<const TIn*>(p.k) + (ref.src * p.heads + h) * kHeadDim;
  const TIn* vrow = reinterpret_cast<const TIn*>(p.v) + (ref.src * p.heads + h) * kHeadDim;
  if (VW >= 4 && wave == VW) {
    const float2 v = load_pair<TIn>(vrow, lane);
    small_quantize_store<KSEL>(v.x, v.y, true, page, o, h, lane, p);
  } else if (wave < 4 && p.t != nullptr) {
    // rows c = 32 wave .. 32 wave + 31: k'[2l..2l+1] partial = sum_c k[c] T[c][2l..2l+1]
    const TIn* th = reinterpret_cast<const TIn*>(p.t) + (int64_t)h * kHeadDim * kHeadDim;
    float2 tv[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) tv[c] = load_pair<TIn>(th + (32 * wave + c) * kHeadDim, lane);
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const float kc = Elem<TIn>::get(krow, 32 * wave + c);
      a = __builtin_fmaf(kc, tv[c].x, a);
      b = __builtin_fmaf(kc, tv[c].y, b);
    }
    part[wave][2 * lane] = a;
    part[wave][2 * lane + 1] = b;
  }
  __syncthreads();
  if (wave == 0) {
    float a, b;
    if (p.t != nullptr) {
      a = ((part[0][2 * lane] + part[1][2 * lane]) + part[2][2 * lane]) + part[3][2 * lane];
      b = ((part[0][2 * lane + 1] + part[1][2 * lane + 1]) + part[2][2 * lane + 1]) + part[3][2 * lane + 1];
    } else {
      const float2 v = load_pair<TIn>(krow, lane);
      a = v.x;
      b = v.y;
    }
    small_quantize_store<KSEL>(a, b, false, page, o, h, lane, p);
  } else if (VW < 4 && wave == VW) {
    const float2 v = load_pair<TIn>(vrow, lane);
    small_quantize_store<KSEL>(v.x, v.y, true, page, o, h, lane, p);
  }
}

}  // namespace
}  // namespace kvq
