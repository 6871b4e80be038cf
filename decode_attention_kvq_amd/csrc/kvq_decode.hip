// Read path: one decode step of grouped-query attention over the quantized paged cache.
//
// Method: "WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms" §4.1 (query
// heads of a group share one KV head), §4.2 (query-side compensation q' = q T^-T after
// RoPE; values stay in the folded basis that W_O absorbs); "Spend Bits Where Queries
// Look" (NOVA-KV project page), "Three requirements": the cache is read on every step,
// so per-element read work is paid over the whole cache.
//
// One kernel (plus a merge when a sequence is split across workgroups): decode_kernel,
// grid (chunk, KV head, sequence), 4 waves per workgroup, 2 resident waves per SIMD.
//  * Prologue: q' = q T^-T in fp32, scaled to log2 units, turned into the matrix-core
//    operand each lane holds.  Its loads go out before the first pages' loads so the
//    arithmetic overlaps them.
//  * Page walk: each wave walks a run of pages through a register ring: the buffer loads
//    (nontemporal) of page i + PIPE are issued when page i has been used, so PIPE pages
//    are in flight per wave.
// Contractions, fp32 accumulation:
//   scores  S[token][col] = codes_K[token][ch] . q''[ch][col]
//   output  O[ch][col]   += codes_V[ch][token] . P~[token][col]
// 2-bit keys use the scaled fp4 x fp6 16x16x128 product: a 2-bit code in the low bits of
// an fp4 nibble is the exact value code/2, so one AND yields 8 operands, and q' is carried
// as three fp6 terms with per-term E8M0 scales (about 12 significant bits, like fp16).
// 4-bit keys and the P.V product use 16x16x32 fp16 products: an AND of the packed word
// with a mask leaves, in each 16-bit half, one code at bit b*e of the mantissa of a
// subnormal fp16, i.e. the exact value code * 2^(b*e) * 2^-24 (codes in the top bits of a
// half are shifted down first); the factor 2^-(b*e) is folded into the other operand.
// Scale and zero are applied outside the products:
//   score_t = s_t * (q . code_t) + z_t * sum(q)
//   out     = (sum_t p_t s_t code_t + sum_t p_t z_t) / sum_t p_t
//
// Column packing.  The 16 columns hold GP >= G query heads repeated in 16/GP blocks;
// score tile b (16 tokens) only feeds the columns of block b % (16/GP), so one 16x16
// accumulator holds 64 tokens x 4 heads at GP = 4 and every lane's softmax work is
// useful.  A lane (column n = block * GP + head, lane group kg) holds the scores of
// tokens 16*kg + 4*b + r of its tiles b, which are exactly the tokens it must feed to
// the P.V product for column n: no data moves between lanes.  Each column keeps its
// own running max, so the only cross-lane steps per page are over the four lane groups
// of a column; columns of one head are merged once at the end.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
// Two waves per SIMD: more resident waves measured slower (the SIMD's issue is the limit,
// not latency), and two leave room for a three-page register ring.
constexpr int kWavesPerSimd = 2;
constexpr int kResidentWaves = 256 * 4 * kWavesPerSimd;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half8 as_half8(u32x4 w) { return __builtin_bit_cast(half8, w); }

// Position class e of the code pair p of a word (the fp16 mantissa bit offset is b*e).
template <int B> __host__ __device__ constexpr int pair_class(int p) {
  return B == 2 ? (p <= 4 ? p : p - 5) : (p <= 1 ? p : p - 2);
}

// Two codes (pair p of word w: positions p and p + 16/b of the word) as two subnormal fp16.
template <int B>
__device__ __forceinline__ uint32_t code_pair(uint32_t w, uint32_t w_shifted, int p) {
  if constexpr (B == 2) {
    return p <= 4 ? (w & (0x00030003u << (2 * p))) : (w_shifted & (0x00030003u << (2 * (p - 5))));
  } else {
    return p <= 1 ? (w & (0x000F000Fu << (4 * p))) : (w_shifted & (0x000F000Fu << (4 * (p - 2))));
  }
}
template <int B> __device__ __forceinline__ uint32_t shifted(uint32_t w) { return B == 2 ? (w >> 10) : (w >> 8); }


__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  half2_t h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Reductions over the four lane groups of a column (lanes l, l^16, l^32, l^48) with the
// gfx950 row/half swaps: after a swap of a value with itself, the pair (dst, src) holds
// the value of the lane and of its partner in some order, so max/sum of the pair is the
// reduction over the partners.
__device__ __forceinline__ float col_max(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
  const uint32_t w = __builtin_bit_cast(uint32_t, v);
  auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)c[0]), __builtin_bit_cast(float, (uint32_t)c[1]));
}
__device__ __forceinline__ int col_max_i(int v) {
  auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = max((int)a[0], (int)a[1]);
  auto c = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return max((int)c[0], (int)c[1]);
}
__device__ __forceinline__ float col_sum(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
  const uint32_t w = __builtin_bit_cast(uint32_t, v);
  auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __builtin_bit_cast(float, (uint32_t)c[0]) + __builtin_bit_cast(float, (uint32_t)c[1]);
}

// Channel of the K-code operand element j at K-step s for lane group kg.
template <int BK> __host__ __device__ constexpr int k_channel(int s, int kg, int j) {
  if constexpr (BK == 2) {
    return 16 * (2 * kg + s / 2) + (4 * (s % 2) + j / 2) + 8 * (j % 2);
  } else {
    return 8 * (4 * kg + s) + j / 2 + 4 * (j % 2);
  }
}
// Position class of channel c in a K row word.
template <int BK> __host__ __device__ constexpr int k_channel_class(int c) {
  return BK == 2 ? pair_class<2>((c % 16) % 8) : pair_class<4>((c % 8) % 4);
}
// Token (0..15 within the lane group) of V operand element j at step s, and its class.
template <int BV> __host__ __device__ constexpr int v_token(int s, int j) {
  return BV == 2 ? (4 * s + j / 2) + 8 * (j % 2) : 8 * s + j / 2 + 4 * (j % 2);
}
template <int BV> __host__ __device__ constexpr int v_token_class(int u) {
  return BV == 2 ? pair_class<2>(u % 8) : pair_class<4>((u % 8) % 4);
}

// ---- 2-bit keys on the scaled fp4 x fp6 matrix-core product (16x16x128) ----
// A 2-bit code c in the low two bits of an fp4 (e2m1) nibble is the exact value c/2, so an
// AND with 0x33333333 turns a packed word into 8 fp4 operands (its even codes) and a shift
// plus AND gives the odd ones.  Lane group kg reads words 2kg, 2kg+1 of the token's row
// (channels 32kg .. 32kg+31); operand element j of the lane is channel k2_channel(kg, j).
// fp4 and fp6 operands of this product share one layout (lane group g, element j is
// contraction index 32g + j), and each lane's 32 elements carry their own E8M0 scale.
__host__ __device__ constexpr int k2_channel(int kg, int j) {
  return 32 * kg + 16 * (j / 16) + 2 * (j % 8) + (j / 8) % 2;
}
constexpr uint32_t kFp4CodeMask = 0x33333333u;
constexpr uint32_t kFp4HighMask = 0x44444444u;   // bit 2 of every nibble: the fp4 value 2
constexpr int kQTerms = 3;          // fp6 terms of q'': about 12 significant bits together

typedef int v8i __attribute__((ext_vector_type(8)));
// D = A(fp4, unit scales) . B(fp6 e2m3, scale byte `opsel` of sb) + C; opsel is a constant
// after unrolling.
__device__ __forceinline__ f32x4 mma_fp4_fp6(int opsel, const v8i& a, const v8i& b, f32x4 c, int sb) {
  switch (opsel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 2, 0, 0x7F7F7F7F, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 2, 0, 0x7F7F7F7F, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 2, 0, 0x7F7F7F7F, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 2, 0, 0x7F7F7F7F, 3, sb);
  }
}

// fp6 e2m3 (1 sign, 2 exponent bits with bias 1, 3 fraction bits; largest 7.5), round to
// nearest even, for |v| <= 7.5.
__device__ __forceinline__ uint32_t e2m3_encode(float v) {
  const float a = fabsf(v);
  uint32_t mag;
  if (a < 1.0f) {
    mag = (uint32_t)rintf(a * 8.0f);                       // 8 encodes 1.0 (exponent 1)
  } else {
    const int e = ilogbf(a);                               // 0, 1 or 2
    mag = (uint32_t)((e + 1) * 8) + (uint32_t)rintf((ldexpf(a, -e) - 1.0f) * 8.0f);
  }
  mag = mag > 31u ? 31u : mag;
  return (v < 0.0f ? 32u : 0u) | mag;
}
__device__ __forceinline__ float e2m3_decode(uint32_t c) {
  const uint32_t mag = c & 31u, e = mag >> 3, m = mag & 7u;
  const float a = e == 0 ? (float)m * 0.125f : ldexpf(1.0f + (float)m * 0.125f, (int)e - 1);
  return (c & 32u) ? -a : a;
}

// ---------------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------------
// Cache policy of the page loads: nontemporal.  Each cache byte is read once per step, so
// keeping it in the caches only costs; streaming with this hint measured ~15% more
// bandwidth than the default policy on the same access pattern.
constexpr int kStreamPolicy = 2;   // gfx950 CPol NT bit

// Pages in flight per wave: a register ring of PIPE pages.
template <int BK, int BV> constexpr int pipe_depth() { return BK + BV <= 4 ? 3 : 2; }

// 3-bit codes are a 2-bit low plane plus a 1-bit high plane: everything the low plane
// needs is the 2-bit machinery (plane width of the low plane).
template <int B> constexpr int low_bits() { return B == 3 ? 2 : B; }

// A page's K and V blocks as seen by one lane, loaded straight into the registers the
// matrix-core operands are built from.  A = accumulators (GP/4) of score rows per lane.
template <int BK, int BV, int A> struct PageRegs {
  typedef std::conditional_t<BK == 4, u32x4, u32x2> KRow;
  KRow k[4];                   // K codes of tile t4: 32 channels of the lane's token (low plane)
  u32x4 v[BV == 4 ? 4 : 2];    // V codes: the lane's V row(s), two 16 B halves each (low plane)
  u32x2 meta[A][4];            // fp16 (s_k, z_k, s_v, z_v) of the lane's 4 tokens per row group
  uint32_t kh[BK == 3 ? 4 : 1];   // 3-bit keys: high-plane bits of the 32 channels, per tile
  u32x4 vh[BV == 3 ? 2 : 1];      // 3-bit values: high-plane words of the lane's channels
};

// Buffer resource of one 128-channel block: loads past num_records bytes return zero and
// touch no memory, which is how a page that does not exist is "loaded".
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, 0x00020000);
}

// Per-lane byte offsets inside a block (the same for every page).
template <int BK, int BV, int A> struct LaneOffsets {
  int k, v, meta[A], kh, vh;
};

template <int BK, int BV, int A>
__device__ __forceinline__ void load_page(PageRegs<BK, BV, A>& r, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rv, const LaneOffsets<BK, BV, A>& o) {
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) {
    if constexpr (BK != 4) r.k[t4] = __builtin_amdgcn_raw_buffer_load_b64(rk, o.k + 128 * t4, 0, kStreamPolicy);
    else r.k[t4] = __builtin_amdgcn_raw_buffer_load_b128(rk, o.k + 256 * t4, 0, kStreamPolicy);
  }
  if constexpr (BK == 3) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) r.kh[t4] = __builtin_amdgcn_raw_buffer_load_b32(rk, o.kh + 64 * t4, 0, kStreamPolicy);
  }
#pragma unroll
  for (int rr = 0; rr < (BV == 4 ? 2 : 1); ++rr) {
    r.v[2 * rr] = __builtin_amdgcn_raw_buffer_load_b128(rv, o.v + 512 * rr, 0, kStreamPolicy);
    r.v[2 * rr + 1] = __builtin_amdgcn_raw_buffer_load_b128(rv, o.v + 512 * rr + 256, 0, kStreamPolicy);
  }
  if constexpr (BV == 3) {
    r.vh[0] = __builtin_amdgcn_raw_buffer_load_b128(rv, o.vh, 0, kStreamPolicy);
    r.vh[1] = __builtin_amdgcn_raw_buffer_load_b128(rv, o.vh + 256, 0, kStreamPolicy);
  }
#pragma unroll
  for (int a = 0; a < A; ++a) {
    r.meta[a][0] = __builtin_amdgcn_raw_buffer_load_b64(rk, code_bytes(BK) + o.meta[a], 0, kStreamPolicy);
    r.meta[a][1] = __builtin_amdgcn_raw_buffer_load_b64(rk, code_bytes(BK) + 128 + o.meta[a], 0, kStreamPolicy);
    r.meta[a][2] = __builtin_amdgcn_raw_buffer_load_b64(rv, code_bytes(BV) + o.meta[a], 0, kStreamPolicy);
    r.meta[a][3] = __builtin_amdgcn_raw_buffer_load_b64(rv, code_bytes(BV) + 128 + o.meta[a], 0, kStreamPolicy);
  }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its outstanding global loads (the page loads in flight stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// T^-T of a cache written without a key transform: the prologue always reads a matrix, so
// its loads need no branch.
struct IdentityMatrix {
  float v[kHeadDim * kHeadDim];
  constexpr IdentityMatrix() : v{} {
    for (int i = 0; i < kHeadDim; ++i) v[i * (kHeadDim + 1)] = 1.0f;
  }
};
__device__ constexpr IdentityMatrix kIdentity{};

template <typename TQ, int BK, int BV, int GP>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  constexpr int NB = 16 / GP;        // column blocks
  constexpr int A = GP / 4;          // score accumulators (tiles per column)
  constexpr int PIPE = pipe_depth<BK, BV>();
  constexpr int KB = block_bytes(BK), VB = block_bytes(BV);
  constexpr int BVL = low_bits<BV>();   // low-plane width of the values
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int kg = lane >> 4, n = lane & 15;
  const int beta = n / GP;           // column block of this lane
  const int G = p.group;

  // merge buffers (per wave: 16 columns x 128 channels, then 16 x (m, l))
  __shared__ __attribute__((aligned(16))) uint8_t smem[kWaves * 16 * (kHeadDim + 2) * 4];
  // prologue scratch: q, then q'; the fp16 operand; two constants per head
  __shared__ __attribute__((aligned(16))) float qs[GP * kHeadDim];
  __shared__ __attribute__((aligned(16))) uint16_t qh[GP * kHeadDim];
  __shared__ float hconst[GP * 2];

  // ---- this wave's pages ----
  // with full-precision windows the cache holds the quantized middle positions only
  const int nseq = min(p.win.flush > 0 ? window_quantized(max(p.seq_lens[b] - p.win_pending, 0), p.win)
                                       : p.seq_lens[b],
                       p.max_pages * kPageTokens);
  const int npages = (nseq + kPageTokens - 1) / kPageTokens;
  const int wv = chunk * kWaves + wave;
  const int pg0 = wv * p.pages_per_wave;
  const int np = max(0, min(pg0 + p.pages_per_wave, npages) - pg0);
  const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;

  // the wave's page ids (at most 64) sit one per lane; the walk reads them with readlane
  int my_page = -1;                        // validated after the prologue loads are out
  if (np > 0) my_page = bt[pg0 + min(lane, np - 1)];
  auto page_id = [&](int i) -> int { return __builtin_amdgcn_readlane(my_page, i); };
  // lane offsets inside a block: K tile t4 holds token 16*(n/4) + 4*t4 + n%4; the V rows
  // are the lane group's; metadata of tokens 16*kg + 4*(a*NB + beta) + 0..3
  LaneOffsets<BK, BV, A> lo;
  {
    const int tok0 = 16 * (n >> 2) + (n & 3);
    lo.k = BK != 4 ? tok0 * 32 + kg * 8 : tok0 * 64 + kg * 16;
    lo.v = (BV != 4 ? kg : 2 * kg) * kHeadDim * 4 + n * 16;
    // high planes: the token's 16-byte key row (4 bytes per lane group); the value words of
    // the lane's channels in the 32-token row that holds its lane group's 16 tokens
    lo.kh = kLowPlaneBytes + tok0 * 16 + kg * 4;
    lo.vh = kLowPlaneBytes + (kg / 2) * kHeadDim * 4 + n * 16;
#pragma unroll
    for (int a = 0; a < A; ++a) lo.meta[a] = 2 * (16 * kg + 4 * (a * NB + beta));
  }
  // loads page i of the run (a page past the run or with an invalid id loads nothing)
  auto load = [&](PageRegs<BK, BV, A>& r, int i) {
    const int pid = i < np ? page_id(i) : -1;
    const int64_t page = pid >= 0 ? pid : 0;
    const int64_t blk = page * p.heads_kv + kvh;
    load_page<BK, BV, A>(r, block_rsrc(p.kpool + blk * KB, pid >= 0 ? KB : 0),
                         block_rsrc(p.vpool + blk * VB, pid >= 0 ? VB : 0), lo);
  };

  // ---- prologue: q' = q T^-T (fp32, log2 units), then the fp16 operand ----
  // Loads of q and T^-T go out first, then the first pages' loads, so the arithmetic below
  // overlaps the page fetch.
  constexpr int QPER = (GP * kHeadDim + kThreads - 1) / kThreads;  // q elements per thread
  const TQ* qb = reinterpret_cast<const TQ*>(p.q) + ((int64_t)b * p.heads_q + (int64_t)kvh * G) * kHeadDim;
  float qreg[QPER];
#pragma unroll
  for (int k = 0; k < QPER; ++k) {   // rows past the group read row 0 and are zeroed below
    const int idx = (int)threadIdx.x + kThreads * k;
    qreg[k] = Elem<TQ>::get(qb, idx < G * kHeadDim ? idx : idx % kHeadDim);
  }
  // lane (quad, cgrp) of wave w < 4: columns j0..j0+3 (j0 = 32w + 4 quad) of rows
  // 16 cgrp..+15; the other waves take no part in the product
  const bool tw = wave < 4;
  const int quad = lane & 7, cgrp = lane >> 3;
  const int j0 = 32 * (tw ? wave : 0) + 4 * quad;
  // both candidates live in global memory; saying so keeps these global (not flat) loads,
  // whose completion the compiler counts precisely
  typedef __attribute__((address_space(1))) const f32x4 gf32x4;
  const gf32x4* tsrc = (const gf32x4*)(p.tinv ? p.tinv + (int64_t)kvh * kHeadDim * kHeadDim : kIdentity.v);
  f32x4 trow[16];
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) trow[cc] = tw ? tsrc[((16 * cgrp + cc) * kHeadDim + j0) / 4] : f32x4{};
  my_page = (lane < np && my_page >= 0 && my_page < p.num_pages) ? my_page : -1;
  PageRegs<BK, BV, A> ring[PIPE];
#pragma unroll
  for (int d = 0; d < PIPE; ++d) load(ring[d], d);
#pragma unroll
  for (int k = 0; k < QPER; ++k) {
    const int idx = (int)threadIdx.x + kThreads * k;
    if (idx < GP * kHeadDim) qs[idx] = idx < G * kHeadDim ? qreg[k] : 0.0f;
  }
  lds_barrier();
  float qacc[GP][4];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cc = 0; cc < 16; cc += 4) {
      const float4 qv = *reinterpret_cast<const float4*>(qs + g * kHeadDim + 16 * cgrp + cc);
      const float qq[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int k = 0; k < 4; ++k) a4[k] = __builtin_fmaf(qq[e], trow[cc + e][k], a4[k]);
      }
    }
    // sum over the 8 row groups (lane bits 3..5): xor 8 by a row rotation, then the swaps
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = __builtin_bit_cast(int, a4[k]);
      const float v = a4[k] + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(u, 0x128, 0xF, 0xF, false));
      qacc[g][k] = col_sum(v);
    }
  }
  lds_barrier();                           // every read of q is done: q' replaces it
  if (tw && cgrp == 0) {
#pragma unroll
    for (int g = 0; g < GP; ++g)
      if (g < G) {
        float4 o;
        o.x = qacc[g][0] * p.score_scale;
        o.y = qacc[g][1] * p.score_scale;
        o.z = qacc[g][2] * p.score_scale;
        o.w = qacc[g][3] * p.score_scale;
        *reinterpret_cast<float4*>(qs + g * kHeadDim + j0) = o;
      }
  }
  lds_barrier();
  // 2-bit keys: q' as three fp6 terms t_k with scales 2^(e1 - 4k), e1 per head so that
  // max|q'| 2^-e1 <= 7.5; each term holds the previous remainder to within a quarter of its
  // scale, so the sum of the three represents q' to about 2^-12 of its largest element.
  // The product with the fp4 codes (value c/2) gives half of q'.code: F = 2.
  v8i bq6[kQTerms];
  int sreg[kQTerms];
  u32x4 bq[BK != 4 ? 1 : NB][4];     // fp16 operands (4-bit keys)
  const int gq = n % GP;
  if constexpr (BK != 4) {
    uint8_t* qcode = smem;                                         // [term][head][channel]
    uint32_t* qpack = reinterpret_cast<uint32_t*>(smem + kQTerms * GP * kHeadDim);  // [term][kg][head][6]
    int* qexp = reinterpret_cast<int*>(qpack + kQTerms * 4 * GP * 6);
    for (int g = wave; g < GP; g += kWaves) {
      const float a0 = g < G ? qs[g * kHeadDim + lane] : 0.0f, a1 = g < G ? qs[g * kHeadDim + lane + 64] : 0.0f;
      float amax = fmaxf(fabsf(a0), fabsf(a1));
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
      int e1 = 0;
      if (amax > 0.0f) {
        const int E = ilogbf(amax);
        e1 = ldexpf(amax, 2 - E) <= 7.5f ? E - 2 : E - 1;
      }
      e1 = max(e1, -118);                  // the last term's scale stays a normal E8M0 value
      float r0 = a0, r1 = a1, qsum = 0.0f;
#pragma unroll
      for (int k = 0; k < kQTerms; ++k) {
        const int e = e1 - 4 * k;
        const uint32_t c0 = e2m3_encode(ldexpf(r0, -e)), c1 = e2m3_encode(ldexpf(r1, -e));
        const float v0 = ldexpf(e2m3_decode(c0), e), v1 = ldexpf(e2m3_decode(c1), e);
        r0 -= v0;
        r1 -= v1;
        qsum += v0 + v1;
        qcode[(k * GP + g) * kHeadDim + lane] = (uint8_t)c0;
        qcode[(k * GP + g) * kHeadDim + lane + 64] = (uint8_t)c1;
      }
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) qsum += __shfl_xor(qsum, d);
      if (lane == 0) {
        hconst[2 * g] = qsum;
        hconst[2 * g + 1] = 2.0f;
        qexp[g] = e1;
      }
    }
    lds_barrier();
    // operand words: element j of lane group kg at bits 6j .. 6j+5 of six dwords
    for (int it = threadIdx.x; it < kQTerms * 4 * GP * 6; it += kThreads) {
      const int d = it % 6, g = (it / 6) % GP, kgi = (it / (6 * GP)) % 4, k = it / (24 * GP);
      const uint8_t* src = qcode + (k * GP + g) * kHeadDim;
      uint32_t word = 0;
      const int j0 = (32 * d) / 6, j1 = min(31, (32 * d + 31) / 6);
      for (int j = j0; j <= j1; ++j) {
        const uint32_t c = src[k2_channel(kgi, j)];
        const int sh = 6 * j - 32 * d;
        word |= sh >= 0 ? c << sh : c >> (-sh);
      }
      qpack[it] = word;
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < kQTerms; ++k) {
#pragma unroll
      for (int d = 0; d < 6; ++d) bq6[k][d] = (int)qpack[((k * 4 + kg) * GP + gq) * 6 + d];
      bq6[k][6] = 0;
      bq6[k][7] = 0;
      // scale byte t (selected per tile by op_sel): the term's scale for this lane's column
      // block, 2^-127 (contributes nothing) for the others
      uint32_t s = 0;
#pragma unroll
      for (int t = 0; t < NB; ++t) s |= (beta == t ? (uint32_t)(127 + qexp[gq] - 4 * k) : 0u) << (8 * t);
      sreg[k] = (int)s;
    }
  } else {
  // fp16 operand q''[c] = q'[c] * 2^(E - BK*e(c)), E per head so that max|q''| < 2^15
  for (int g = wave; g < G; g += kWaves) {
    const float a0 = qs[g * kHeadDim + lane], a1 = qs[g * kHeadDim + lane + 64];
    float amax = fmaxf(fabsf(a0), fabsf(a1));
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
    const int E = amax > 0.0f ? 14 - ilogbf(amax) : 0;
    float qsum = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = lane + 64 * k;
      const int sh = BK * k_channel_class<BK>(c);
      const uint16_t hbits = f32_to_f16_bits(ldexpf(k ? a1 : a0, E - sh));
      qh[g * kHeadDim + c] = hbits;
      qsum += ldexpf(f16_bits_to_f32(hbits), sh - E);
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) qsum += __shfl_xor(qsum, d);
    if (lane == 0) {
      hconst[2 * g] = qsum;
      hconst[2 * g + 1] = ldexpf(1.0f, 24 - E);
    }
  }
  lds_barrier();
  // B operand of K-step s for this lane (column n = head n % GP, lane group kg), masked per
  // column block: block beta's operand is the lane's own, the others are zero
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 w;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t lo = gq < G ? qh[gq * kHeadDim + k_channel<BK>(s, kg, 2 * jj)] : 0u;
      const uint32_t hi = gq < G ? qh[gq * kHeadDim + k_channel<BK>(s, kg, 2 * jj + 1)] : 0u;
      w[jj] = lo | (hi << 16);
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) bq[bb][s] = (beta == bb) ? w : u32x4{0u, 0u, 0u, 0u};
  }
  }
  const float F = gq < G ? hconst[2 * gq + 1] : 1.0f;                  // score = F * x'
  const float qsf = gq < G ? hconst[2 * gq] / hconst[2 * gq + 1] : 0.0f;


  // per (accumulator a, row r): token u = 4*(a*NB + beta) + r of this lane group
  f32x4 acc_o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc_o[mt] = f32x4{};
  float lsum[A][4], zacc[A][4], nb[A][4];
  int vcls[A][4];                        // BV * class of each held token: P~ carries 2^(S - vcls)
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lsum[a][r] = 0.0f;
      zacc[a][r] = 0.0f;
      nb[a][r] = 0.0f;
      int e = 0;
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
        if (beta == bb) e = v_token_class<BVL>(4 * (a * NB + bb) + r);
      vcls[a][r] = BVL * e;
    }
  // 3-bit values: the high-plane bit of lane-group token u is the subnormal fp16
  // 2^(u % 8) * 2^-24 and weighs 4 (code = low + 4 * high), so its P~ is the low plane's
  // times 4 * 2^(vcls - u % 8); the high words of odd lane groups hold their tokens one
  // byte up in each half
  float hfac[A][4];
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) hfac[a][r] = ldexpf(4.0f, vcls[a][r] - (4 * (a * NB + beta) + r) % 8);
  const int hsh = 8 * (kg & 1);
  // halves of the P.V operand words that carry this lane's tiles (see the P.V step)
  uint32_t bmask[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int t_lo = v_token<BVL>(s, 0) / 4, t_hi = v_token<BVL>(s, 1) / 4;   // same for every jj
    bmask[s] = ((t_lo % NB == beta) ? 0x0000FFFFu : 0u) | ((t_hi % NB == beta) ? 0xFFFF0000u : 0u);
  }
  float m = -__builtin_inff();   // running max of x' for this lane's column
  int S = 30;

  // ---- page walk: compute page i from ring slot i % PIPE, then refill the slot ----
  auto compute = [&](const PageRegs<BK, BV, A>& pr, int i) {
    const int valid_tokens = nseq - (pg0 + i) * kPageTokens;   // >= 1
    const bool partial = valid_tokens < kPageTokens;

    // ---- scores: tile t4 = tokens 16*(n/4) + 4*t4 + n%4 in rows n ----
    f32x4 sacc[A];
#pragma unroll
    for (int a = 0; a < A; ++a) sacc[a] = f32x4{};
    if constexpr (BK != 4) {
      // one 16x16x128 product per tile and fp6 term; the op_sel'd scale byte keeps tile t4
      // out of every column block but t4 % NB
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const uint32_t w0 = pr.k[t4][0], w1 = pr.k[t4][1];
        const v8i av = {(int)(w0 & kFp4CodeMask), (int)((w0 >> 2) & kFp4CodeMask), (int)(w1 & kFp4CodeMask),
                        (int)((w1 >> 2) & kFp4CodeMask), 0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < kQTerms; ++k) sacc[t4 / NB] = mma_fp4_fp6(t4 % NB, av, bq6[k], sacc[t4 / NB], sreg[k]);
        if constexpr (BK == 3) {
          // high plane: operand element (dword d, nibble i) is channel offset
          // 16(d/2) + d%2 + 2i, whose bit sits at 4i + d; shifted to bit 2 of the nibble it
          // is the fp4 value 2 = (4 * bit) / 2, so the two products add to code / 2
          const uint32_t h = pr.kh[t4];
          const v8i ah = {(int)((h << 2) & kFp4HighMask), (int)((h << 1) & kFp4HighMask), (int)(h & kFp4HighMask),
                          (int)((h >> 1) & kFp4HighMask), 0, 0, 0, 0};
#pragma unroll
          for (int k = 0; k < kQTerms; ++k) sacc[t4 / NB] = mma_fp4_fp6(t4 % NB, ah, bq6[k], sacc[t4 / NB], sreg[k]);
        }
      }
    } else
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      uint32_t kw[BK == 2 ? 2 : 4];
#pragma unroll
      for (int e = 0; e < (BK == 2 ? 2 : 4); ++e) kw[e] = pr.k[t4][e];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t w = BK == 2 ? kw[s / 2] : kw[s];
        const uint32_t ws = shifted<BK>(w);
        u32x4 av;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) av[jj] = code_pair<BK>(w, ws, BK == 2 ? 4 * (s % 2) + jj : jj);
        sacc[t4 / NB] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(av), as_half8(bq[t4 % NB][s]),
                                                              sacc[t4 / NB], 0, 0, 0);
      }
    }
    // metadata of the lane's tokens (4 consecutive per tile: 8 bytes each).  The fp16
    // scales and zeros enter the arithmetic as fp16 operands of mixed fma (no conversions).
    float x[A][4];
    u32x2 svp[A], zvp[A];
#pragma unroll
    for (int a = 0; a < A; ++a) {
      // (the 8-byte pair is reinterpreted whole: building half pairs from its two words
      // separately is miscompiled by this toolchain, which then reads only the first word)
      const half4_t sk = __builtin_bit_cast(half4_t, pr.meta[a][0]);
      const half4_t zk = __builtin_bit_cast(half4_t, pr.meta[a][1]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float zq = __builtin_fmaf((float)zk[r], qsf, 0.0f);
        x[a][r] = __builtin_fmaf(sacc[a][r], (float)sk[r], zq);
      }
      svp[a] = pr.meta[a][2];
      zvp[a] = pr.meta[a][3];
    }
    if (partial) {                          // absent tokens: no weight, no garbage scale
#pragma unroll
      for (int a = 0; a < A; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = 16 * kg + 4 * (a * NB + beta) + r < valid_tokens;
          x[a][r] = ok ? x[a][r] : -__builtin_inff();
          const uint32_t keep = ok ? 0xFFFFFFFFu : ((r & 1) ? 0x0000FFFFu : 0xFFFF0000u);
          svp[a][r >> 1] &= keep;
          zvp[a][r >> 1] &= keep;
        }
    }
    // ---- online softmax, per column ----
    float mx = x[0][0];
    uint32_t svm = 0;                      // largest value-scale bit pattern (s_v >= 0)
#pragma unroll
    for (int a = 0; a < A; ++a) {
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[a][r]);
#pragma unroll
      for (int e = 0; e < 2; ++e) svm = max(svm, max(svp[a][e] & 0xFFFFu, svp[a][e] >> 16));
    }
    mx = col_max(mx);
    // Lazy rescaling.  The reference max m of a column moves only when the page's scores
    // exceed it by more than kLag (log2 units), so p = 2^(F(x - m)) <= 2^kLag; S moves
    // only when a value scale would push P~ = p s_v 2^(S - vcls) to 2^15 (fp16 range),
    // and then kSMargin further, so that later pages rarely need it again.  Rescaling is
    // wave-uniform, so an eager rule would run it whenever any of the 16 columns grows.
    constexpr float kLag = 8.0f;
    constexpr int kSMargin = 4;
    // exponent bound of the column's largest value scale: s_v < 2^(ev+1) (fp16 bits;
    // a subnormal scale counts as 2^-15)
    const int svbits = col_max_i((int)svm);
    const int e16 = (svbits >> 10) & 0x1F;
    const int ev = svbits == 0 ? -30 : (e16 == 0 ? -15 : e16 - 15);
    // (3-bit values: the high plane's P~ carries up to 4x more, two bits of headroom)
    const int S_tight = (BV == 3 ? 12 : 14) - (int)kLag - ev;
    const bool need_s = S_tight < S;
    const int S_new = need_s ? S_tight - kSMargin : S;
    const bool need_m = F * (mx - m) > kLag;       // false when the column has no token here
    const float m_new = need_m ? mx : m;
    if (__any(need_m || need_s)) {
      const float alpha = exp2f(F * (m - m_new) + (float)(S_new - S));
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc_o[mt] *= alpha;
#pragma unroll
      for (int a = 0; a < A; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          lsum[a][r] *= alpha;
          zacc[a][r] *= alpha;
          nb[a][r] = (float)(S_new - vcls[a][r]) - F * m_new;
        }
      m = m_new;
      S = S_new;
    }
    float pt[A][4];
#pragma unroll
    for (int a = 0; a < A; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(F, x[a][r], nb[a][r]));
        const half4_t svh = __builtin_bit_cast(half4_t, svp[a]);
        const half4_t zvh = __builtin_bit_cast(half4_t, zvp[a]);
        lsum[a][r] += pe;
        zacc[a][r] = __builtin_fmaf(pe, (float)zvh[r], zacc[a][r]);
        pt[a][r] = __builtin_fmaf(pe, (float)svh[r], 0.0f);
      }

    // ---- P.V: B operand element (s, 2*jj + h) is token u = v_token(s, 2jj+h), i.e. tile
    // b(s, h) = u/4, row jj; the lane feeds only its own tiles, the rest of the operand is 0
    u32x4 bp[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int t_lo = v_token<BVL>(s, 2 * jj) / 4, t_hi = v_token<BVL>(s, 2 * jj + 1) / 4;
        if constexpr (NB == 1) {
          bp[s][jj] = pack_f16x2(pt[t_lo][jj], pt[t_hi][jj]);
        } else {
          // both halves take the held value; a per-lane mask keeps the halves whose tile
          // is this lane's (tile % NB == beta)
          const uint32_t both = pack_f16x2(pt[t_lo / NB][jj], pt[t_hi / NB][jj]);
          bp[s][jj] = both & bmask[s];
        }
      }
#pragma unroll
    for (int rr = 0; rr < (BV != 4 ? 1 : 2); ++rr) {
      const u32x4 va = pr.v[2 * rr], vc = pr.v[2 * rr + 1];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (BV == 4 && s != rr) continue;
          const uint32_t w = (mt >> 2) ? vc[mt & 3] : va[mt & 3];
          const uint32_t ws = shifted<BVL>(w);
          u32x4 av;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) av[jj] = code_pair<BVL>(w, ws, BVL == 2 ? 4 * s + jj : jj);
          acc_o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(av), as_half8(bp[s]), acc_o[mt], 0, 0, 0);
        }
      }
    }
    if constexpr (BV == 3) {
      // high plane: token pair (p, p + 8), p = 4s + jj, sits at bits p and 16 + p of the
      // lane group's (aligned) word, the same pairs as the low plane's operand
      u32x4 bph[2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int t_lo = v_token<2>(s, 2 * jj) / 4, t_hi = v_token<2>(s, 2 * jj + 1) / 4;
          if constexpr (NB == 1) {
            bph[s][jj] = pack_f16x2(pt[t_lo][jj] * hfac[t_lo][jj], pt[t_hi][jj] * hfac[t_hi][jj]);
          } else {
            const uint32_t both = pack_f16x2(pt[t_lo / NB][jj] * hfac[t_lo / NB][jj],
                                             pt[t_hi / NB][jj] * hfac[t_hi / NB][jj]);
            bph[s][jj] = both & bmask[s];
          }
        }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const uint32_t wh = ((mt >> 2) ? pr.vh[1][mt & 3] : pr.vh[0][mt & 3]) >> hsh;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          u32x4 av;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) av[jj] = wh & ((1u << (4 * s + jj)) | (1u << (16 + 4 * s + jj)));
          acc_o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(av), as_half8(bph[s]), acc_o[mt], 0, 0, 0);
        }
      }
    }
  };
  // whole groups of PIPE pages (every path through an iteration issues the same loads, so
  // the compiler's wait for each slot covers that slot's loads only), then the tail
  int i0 = 0;
  for (; i0 + PIPE <= np; i0 += PIPE) {
#pragma unroll
    for (int d = 0; d < PIPE; ++d) {
      if (page_id(i0 + d) >= 0) compute(ring[d], i0 + d);   // an invalid page id contributes nothing
      load(ring[d], i0 + d + PIPE);
    }
  }
#pragma unroll
  for (int d = 0; d < PIPE - 1; ++d)
    if (i0 + d < np && page_id(i0 + d) >= 0) compute(ring[d], i0 + d);

  // ---- column result: m (log2 units), l, o_num = acc * 2^(24-S) + z ----
  float l = 0.0f, z = 0.0f;
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      l += ldexpf(lsum[a][r], vcls[a][r] - S);
      z += ldexpf(zacc[a][r], vcls[a][r] - S);
    }
  l = col_sum(l);
  z = col_sum(z);
  const bool any_page = m != -__builtin_inff();
  const float mlog2 = any_page ? F * m : -__builtin_inff();
  const float oscale = ldexpf(1.0f, 24 - S);
  __syncthreads();
  float (*red_o)[16][kHeadDim] = reinterpret_cast<float (*)[16][kHeadDim]>(smem);
  float (*red_ml)[16][2] = reinterpret_cast<float (*)[16][2]>(smem + kWaves * 16 * kHeadDim * 4);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ch = 4 * (4 * kg + r) + (mt & 3) + 64 * (mt >> 2);
      red_o[wave][n][ch] = __builtin_fmaf(acc_o[mt][r], oscale, z);
    }
  if (kg == 0) {
    red_ml[wave][n][0] = mlog2;
    red_ml[wave][n][1] = any_page ? l : 0.0f;
  }
  __syncthreads();

  // ---- merge the waves and the column blocks of each head ----
  const int hq0 = kvh * G;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kThreads) {
    const int gg = idx / kHeadDim, ch = idx % kHeadDim;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) M = fmaxf(M, red_ml[w][bb * GP + gg][0]);
    float L = 0.0f, O = 0.0f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const int col = bb * GP + gg;
          const float mw = red_ml[w][col][0];
          if (mw != -__builtin_inff()) {
            const float f = exp2f(mw - M);
            L = __builtin_fmaf(red_ml[w][col][1], f, L);
            O = __builtin_fmaf(red_o[w][col][ch], f, O);
          }
        }
    }
    const int hq = hq0 + gg;
    if (p.chunks == 1 && p.win.flush == 0) {
      p.out[((int64_t)b * p.heads_q + hq) * kHeadDim + ch] = L > 0.0f ? O / L : 0.0f;
    } else {
      const int64_t slot = ((int64_t)b * p.heads_q + hq) * p.chunks + chunk;
      p.ws_o[slot * kHeadDim + ch] = O;
      if (ch == 0) {
        p.ws_ml[slot * 2] = M;
        p.ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

__global__ __launch_bounds__(128) void combine_kernel(DecodeParams p) {
  const int64_t row = blockIdx.x;        // b * Hq + hq
  const int ch = threadIdx.x;
  const float* ml = p.ws_ml + row * p.chunks * 2;
  float M = -__builtin_inff();
  for (int c = 0; c < p.chunks; ++c) M = fmaxf(M, ml[2 * c]);
  float L = 0.0f, O = 0.0f;
  if (M != -__builtin_inff()) {
    for (int c = 0; c < p.chunks; ++c) {
      const float mc = ml[2 * c];
      if (mc != -__builtin_inff()) {
        const float f = exp2f(mc - M);
        L = __builtin_fmaf(ml[2 * c + 1], f, L);
        O = __builtin_fmaf(p.ws_o[(row * p.chunks + c) * kHeadDim + ch], f, O);
      }
    }
  }
  p.out[row * kHeadDim + ch] = L > 0.0f ? O / L : 0.0f;
}

template <typename TQ, int BK, int BV>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.chunks, (unsigned)p.heads_kv, (unsigned)p.batch);
  switch (p.gpad) {
    case 4: hipLaunchKernelGGL((decode_kernel<TQ, BK, BV, 4>), grid, dim3(kThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<TQ, BK, BV, 8>), grid, dim3(kThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_kernel<TQ, BK, BV, 16>), grid, dim3(kThreads), 0, stream, p); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.chunks == 1 || p.win.flush > 0) return err;   // windows: merged by the window kernel
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(p.batch * p.heads_q)), dim3(kHeadDim), 0, stream, p);
  return hipGetLastError();
}

template <int BK, int BV>
hipError_t launch_bits(const DecodeParams& p, int q_dtype, hipStream_t stream) {
  switch (q_dtype) {
    case 0: return launch_typed<float, BK, BV>(p, stream);
    case 1: return launch_typed<__bf16, BK, BV>(p, stream);
    default: return launch_typed<_Float16, BK, BV>(p, stream);
  }
}

}  // namespace

int decode_group_pad(int group) { return group <= 4 ? 4 : (group <= 8 ? 8 : 16); }

DecodeSplit decode_split(int batch, int heads_kv, int max_seq_len) {
  const int pages = (max_seq_len + kPageTokens - 1) / kPageTokens;
  const int64_t units = (int64_t)batch * heads_kv;
  // about kResidentWaves waves (one resident round), 4 to 64 pages per wave
  // (a wave's page ids fit one register, one per lane)
  int64_t ppw = (units * pages + kResidentWaves - 1) / kResidentWaves;
  if (ppw < 4) ppw = 4;
  if (ppw > 64) ppw = 64;
  const int64_t waves = pages > 0 ? (pages + ppw - 1) / ppw : 1;
  DecodeSplit s;
  s.pages_per_wave = (int)ppw;
  s.chunks = (int)((waves + kWaves - 1) / kWaves);
  return s;
}

hipError_t launch_decode(const DecodeParams& p, int bits_k, int bits_v, int q_dtype, hipStream_t stream) {
  switch (bits_k * 10 + bits_v) {
    case 22: return launch_bits<2, 2>(p, q_dtype, stream);
    case 23: return launch_bits<2, 3>(p, q_dtype, stream);
    case 24: return launch_bits<2, 4>(p, q_dtype, stream);
    case 32: return launch_bits<3, 2>(p, q_dtype, stream);
    case 33: return launch_bits<3, 3>(p, q_dtype, stream);
    case 34: return launch_bits<3, 4>(p, q_dtype, stream);
    case 42: return launch_bits<4, 2>(p, q_dtype, stream);
    case 43: return launch_bits<4, 3>(p, q_dtype, stream);
    default: return launch_bits<4, 4>(p, q_dtype, stream);
  }
}

}  // namespace kvq
