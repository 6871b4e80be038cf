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
//   scores  S[token][col] = codes_K[token][ch] . q'[ch][col]
//   output  O[ch][col]   += codes_V[ch][token] . P~[token][col]
// Keys of every width use the scaled fp4 x fp6 16x16x128 product: a 2-bit code (or a
// 2-bit slice of a 3- or 4-bit code) in the low bits of an fp4 nibble is the exact value
// code/2, so one AND yields 8 operands; a 4-bit code's high pair weighs 4 through the A
// operand's scale.  q' is carried as fp6 terms with per-term E8M0 scales: three (about 12
// significant bits), and a fourth on pages whose scores are large.
// The P.V product uses 16x16x32 fp16 products: an AND of the packed value word with a
// mask leaves, in each 16-bit half, one code at bit b*e of the mantissa of a subnormal
// fp16, i.e. the exact value code * 2^(b*e) * 2^-24 (codes in the top bits of a half are
// shifted down first); the factor 2^-(b*e) is folded into P~.
// Scale and zero are applied outside the products:
//   score_t = s_t * (q . code_t) + z_t * sum(q)
//   out     = (sum_t p_t s_t code_t + sum_t p_t z_t) / sum_t p_t
// P~ = p s_v 2^(S - b*e) is fp16; the exponent S follows the largest P~ of each page, so the
// tokens that carry the weight keep fp16's full precision whatever their value scales.
//
// Column packing.  The 16 columns hold GP >= G query heads repeated in 16/GP blocks;
// score tile b (16 tokens) only feeds the columns of block b % (16/GP), so one 16x16
// accumulator holds 64 tokens x 4 heads at GP = 4 and every lane's softmax work is
// useful.  A lane (column n = block * GP + head, lane group kg) holds the scores of
// tokens 16*kg + 4*b + r of its tiles b, which are exactly the tokens it must feed to
// the P.V product for column n: no data moves between lanes.  Each column keeps its
// own running max, so the only cross-lane steps per page are over the four lane groups
// of a column; columns of one head are merged once at the end.
#include <atomic>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_encode.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
// Two waves per SIMD: more resident waves measured slower (the SIMD's issue is the limit,
// not latency), and two leave room for a three-page register ring.
constexpr int kWavesPerSimd = 2;
constexpr int kResidentWaves = 256 * 4 * kWavesPerSimd;
// Fewest pages a wave walks when the batch is too small to fill the chip: at batch 1 x 16K
// one page per wave took 20 us (every wave pays the prologue and the merge for one page),
// two to four 14.3-14.9 us, six 15.7-16 us.
constexpr int kMinPagesPerWave = 4;

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

// Token (0..15 within the lane group) of V operand element j at step s, and its class.
template <int BV> __host__ __device__ constexpr int v_token(int s, int j) {
  return BV == 2 ? (4 * s + j / 2) + 8 * (j % 2) : 8 * s + j / 2 + 4 * (j % 2);
}
template <int BV> __host__ __device__ constexpr int v_token_class(int u) {
  return BV == 2 ? pair_class<2>(u % 8) : pair_class<4>((u % 8) % 4);
}

// ---- keys on the scaled fp4 x fp6 matrix-core product (16x16x128) ----
// A 2-bit code c in the low two bits of an fp4 (e2m1) nibble is the exact value c/2, so an
// AND with 0x33333333 turns a packed 2-bit word into 8 fp4 operands (its even codes) and a
// shift plus AND gives the odd ones.  A 4-bit code is two such pairs: the same AND leaves
// bits 0-1 of each code in place and a shift by 2 first gives bits 2-3, whose product
// weighs 4 through the A operand's E8M0 scale.  3-bit codes add their bit-2 plane as the
// fp4 value 2.  Lane group kg reads the channels 32kg .. 32kg+31 of its token's row;
// operand element j of the lane is channel key_channel<BK>(kg, j).  fp4 and fp6 operands of
// this product share one layout (lane group g, element j is contraction index 32g + j),
// and each lane's 32 elements carry their own E8M0 scale.
template <int BK> __host__ __device__ constexpr int key_channel(int kg, int j) {
  return BK == 4 ? 32 * kg + j : 32 * kg + 16 * (j / 16) + 2 * (j % 8) + (j / 8) % 2;
}
constexpr uint32_t kFp4CodeMask = 0x33333333u;
constexpr uint32_t kFp4HighMask = 0x44444444u;   // bit 2 of every nibble: the fp4 value 2
constexpr int kUnitScale = 0x7F7F7F7F;           // E8M0 2^0 in every byte
constexpr int kTimes4Scale = 0x81818181;         // E8M0 2^2 in every byte
// q' is carried as fp6 terms (4 significant bits each, scales 4 binades apart).  Three
// represent it to about 2^-12 of its largest element; a fourth, to about 2^-16, joins the
// products of a page whose largest score (log2 units) exceeds kBigScore in magnitude, where
// a relative score error of 2^-12 would move the softmax weights by more than the
// output's bound allows.
constexpr int kQTerms = 4;
constexpr int kQBase = 3;
constexpr float kBigScore = 24.0f;

typedef int v8i __attribute__((ext_vector_type(8)));
// D = A(fp4, scale sa) . B(fp6 e2m3, scale byte `opsel` of sb) + C; opsel is a constant
// after unrolling.
__device__ __forceinline__ f32x4 mma_fp4_fp6(int opsel, const v8i& a, const v8i& b, f32x4 c, int sb,
                                             int sa = kUnitScale) {
  switch (opsel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 2, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 2, 0, sa, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 2, 0, sa, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 2, 0, sa, 3, sb);
  }
}

typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
// 32 fp32 values to packed fp6 e2m3 (1 sign, 2 exponent bits with bias 1, 3 fraction bits;
// largest 7.5): element 2i of the result (bits 12i .. 12i+5) is a[i] / 2^e, element 2i + 1 is
// b[i] / 2^e, where 2^e is the power of two of `scale`; round to nearest even, saturating
// (checked on the GPU).  Written as inline assembly with an early-clobber result: the
// compiler's builtin for this instruction let the result overlap the second source, which
// the instruction overwrites before reading it.
__device__ __forceinline__ u32x6 fp6_pack32(f32x16 a, f32x16 b, float scale) {
  u32x6 d;
  asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(scale));
  return d;
}
// The inverse at unit scale: element j of the packed fp6 values as fp16 (exact).
typedef _Float16 half32 __attribute__((ext_vector_type(32)));
__device__ __forceinline__ half32 fp6_unpack32_f16(u32x6 c) {
  half32 d;
  asm("v_cvt_scalef32_pk32_f16_fp6 %0, %1, %2" : "=&v"(d) : "v"(c), "v"(1.0f));
  return d;
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

// ---- the query operands: q' = q T^-T (fp32, log2 units) as fp6 terms ----
// One lane's share of them: the fp6 codes of the kQTerms terms for channels key_channel(kg, .)
// of head gq = n % GP (kg = lane / 16), the head's scale exponent e1 and its sums of q' as
// kQBase and kQTerms terms carry them (divided by F = 2: the product with the fp4 codes, of
// value code / 2, gives half of q'.code).
struct QOperands {
  v8i bq6[kQTerms];
  int e1;
  float qsf3, qsf4;
};
constexpr float kF = 2.0f;                 // score = F * x'

// The loads the build needs, issued first so that the page loads queue behind them: this
// thread's q elements and, for lane (quad, cgrp) of wave w, columns j0 .. j0 + 3 (j0 = 32 w
// + 4 quad) of rows 16 cgrp .. 16 cgrp + 15 of T^-T.
template <typename TQ, int GP>
struct QLoads {
  static constexpr int QPER = (GP * kHeadDim + kThreads - 1) / kThreads;  // q elements per thread
  float qreg[QPER];
  f32x4 trow[16];
};
template <typename TQ, int GP>
__device__ __forceinline__ void q_issue_loads(const DecodeParams& p, int b, int kvh, int wave, int lane,
                                              QLoads<TQ, GP>& L) {
  const int G = p.group;
  const TQ* qb = reinterpret_cast<const TQ*>(p.q) + ((int64_t)b * p.heads_q + (int64_t)kvh * G) * kHeadDim;
#pragma unroll
  for (int k = 0; k < QLoads<TQ, GP>::QPER; ++k) {   // rows past the group read row 0 and are zeroed later
    const int idx = (int)threadIdx.x + kThreads * k;
    L.qreg[k] = Elem<TQ>::get(qb, idx < G * kHeadDim ? idx : idx % kHeadDim);
  }
  const int quad = lane & 7, cgrp = lane >> 3;
  const int j0 = 32 * wave + 4 * quad;
  // both candidates live in global memory; saying so keeps these global (not flat) loads,
  // whose completion the compiler counts precisely
  typedef __attribute__((address_space(1))) const f32x4 gf32x4;
  const gf32x4* tsrc = (const gf32x4*)(p.tinv ? p.tinv + (int64_t)kvh * kHeadDim * kHeadDim : kIdentity.v);
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) L.trow[cc] = tsrc[((16 * cgrp + cc) * kHeadDim + j0) / 4];
}

// Builds this lane's operands from the loads (every thread of the 4-wave workgroup calls it:
// it holds three workgroup barriers).  qs: LDS scratch of GP * kQRow floats, q first (rows
// of kHeadDim), then q' (rows of kQRow: each 32-channel group in 33 floats, so that the 16
// (head, group) operands read at once hit distinct banks).
constexpr int kQRow = 4 * 33;
template <typename TQ, int BK, int GP>
__device__ __forceinline__ void q_build(const DecodeParams& p, int wave, int lane, const QLoads<TQ, GP>& L,
                                        float* qs, QOperands& o) {
  const int G = p.group;
  const int kg = lane >> 4, n = lane & 15;
  const int quad = lane & 7, cgrp = lane >> 3;
#pragma unroll
  for (int k = 0; k < QLoads<TQ, GP>::QPER; ++k) {
    const int idx = (int)threadIdx.x + kThreads * k;
    if (idx < GP * kHeadDim) qs[idx] = idx < G * kHeadDim ? L.qreg[k] : 0.0f;
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
        for (int k = 0; k < 4; ++k) a4[k] = __builtin_fmaf(qq[e], L.trow[cc + e][k], a4[k]);
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
  if (cgrp == 0) {
    // channels j0 .. j0 + 3 sit in group j0 / 32 = wave; heads past G read as 0
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int k = 0; k < 4; ++k) qs[g * kQRow + 33 * wave + 4 * quad + k] = g < G ? qacc[g][k] * p.score_scale : 0.0f;
  }
  lds_barrier();
  // q' as fp6 (e2m3) terms t_k with scales 2^(e1 - 4k), e1 per head so that
  // max|q'| 2^-e1 <= 7.5; each term holds the previous remainder to within a quarter of its
  // scale.  Every lane builds its own operand, the channels key_channel(kg, j) of head gq,
  // with the fp6 packing conversion, and converts it back for the remainder.
  const int gq = n % GP;
  // a[i], b[i]: channels key_channel(kg, 2i), key_channel(kg, 2i + 1) (the packing puts
  // a[i] at element 2i and b[i] at 2i + 1), then the remainders
  f32x16 a, b;
  const float* qh = qs + gq * kQRow + 33 * kg;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a[i] = qh[key_channel<BK>(0, 2 * i)];
    b[i] = qh[key_channel<BK>(0, 2 * i + 1)];
    amax = fmaxf(amax, fmaxf(fabsf(a[i]), fabsf(b[i])));
  }
  amax = col_max(amax);                  // over the four lane groups: the whole head
  int e1 = 0;
  if (amax > 0.0f) {
    const int E = ilogbf(amax);
    e1 = ldexpf(amax, 2 - E) <= 7.5f ? E - 2 : E - 1;
  }
  e1 = max(e1, -126 + 4 * (kQTerms - 1));   // the last term's scale stays a normal E8M0 value
  float s3 = 0.0f, s4 = 0.0f;
#pragma unroll
  for (int k = 0; k < kQTerms; ++k) {
    const float scale = ldexpf(1.0f, e1 - 4 * k);
    const u32x6 code = fp6_pack32(a, b, scale);
    const half32 h = fp6_unpack32_f16(code);          // the term's values / scale (exact)
    if (k + 1 < kQTerms) {                            // (the last remainder is not used)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        a[i] = __builtin_fmaf(-(float)h[2 * i], scale, a[i]);
        b[i] = __builtin_fmaf(-(float)h[2 * i + 1], scale, b[i]);
      }
    }
    // the term's sum by a packed fp16 tree: its values are multiples of 1/8 of magnitude at
    // most 7.5, so every partial sum is a multiple of 1/8 below 256 in magnitude, where fp16
    // is exact (steps of 1/8 from 128 to 256)
    half2_t hp[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) hp[i] = half2_t{h[2 * i], h[2 * i + 1]};
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) hp[i] = hp[i] + hp[i + w];
    const float hs = (float)hp[0][0] + (float)hp[0][1];
    if (k < kQBase) s3 += hs * scale;
    s4 += hs * scale;
#pragma unroll
    for (int d = 0; d < 6; ++d) o.bq6[k][d] = (int)code[d];
    o.bq6[k][6] = 0;
    o.bq6[k][7] = 0;
  }
  o.e1 = e1;
  o.qsf3 = gq < G ? col_sum(s3) / kF : 0.0f;
  o.qsf4 = gq < G ? col_sum(s4) / kF : 0.0f;
}

template <typename TQ, int BK, int BV, int GP>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  constexpr int NB = 16 / GP;        // column blocks
  constexpr int A = GP / 4;          // score accumulators (tiles per column)
  constexpr int PIPE = pipe_depth<BK, BV>();
  constexpr int KB = block_bytes(BK), VB = block_bytes(BV);
  constexpr int BVL = low_bits<BV>();   // low-plane width of the values
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= p.batch) {
    // a decode step's append, in the blocks after the decode's: dispatched last, they run in
    // the slots that the first decode workgroups leave while the last ones still walk
    __shared__ float app_part[4][kHeadDim];
    if (p.append_blocks && chunk == 0) {
      if (select_width(p.app) == 3) append_token<TQ, 3, 1>(p.app, b - p.batch, kvh, wave, lane, app_part);
      else append_token<TQ, 0, 1>(p.app, b - p.batch, kvh, wave, lane, app_part);
    }
    return;
  }
  const int kg = lane >> 4, n = lane & 15;
  const int beta = n / GP;           // column block of this lane
  const int G = p.group;

  // merge buffers (per wave: 16 columns x 128 channels in rows of kHeadDim + 1, so that the
  // scattered writes of a half wave reach 32 banks; then 16 x (m, l))
  __shared__ __attribute__((aligned(16))) uint8_t smem[kWaves * 16 * (kHeadDim + 3) * 4];

  // ---- this wave's pages ----
  // with full-precision windows the cache holds the quantized middle positions only
  // a decode step's new token (position seq_len - 1) comes from the step's rows, not the cache
  const bool new_tok = p.knew != nullptr && p.seq_lens[b] > 0;
  const int nseq = min(p.win.flush > 0 ? window_quantized(max(p.seq_lens[b] - p.win_pending, 0), p.win)
                                       : p.seq_lens[b] - (new_tok ? 1 : 0),
                       p.max_pages * kPageTokens);
  const int npages = (nseq + kPageTokens - 1) / kPageTokens;
  const int wv = chunk * kWaves + wave;
  const int pg0 = wv * p.pages_per_wave;
  const int np = max(0, min(pg0 + p.pages_per_wave, npages) - pg0);
  const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;

  // the wave's page ids (at most 128) sit one per lane in two registers; the walk reads
  // them with readlane (its page index is wave-uniform)
  int my_page = -1, my_page2 = -1;         // validated after the prologue loads are out
  if (np > 0) my_page = bt[pg0 + min(lane, np - 1)];
  if (np > 64) my_page2 = bt[pg0 + 64 + min(lane, np - 65)];
  auto page_id = [&](int i) -> int {
    const int lo = __builtin_amdgcn_readlane(my_page, i & 63), hi = __builtin_amdgcn_readlane(my_page2, i & 63);
    return i < 64 ? lo : hi;
  };
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

  // ---- prologue: the query operands ----
  // q and T^-T loads first, then the first pages' loads, so that the arithmetic that builds
  // the operands overlaps the page fetch
  QLoads<TQ, GP> L;
  q_issue_loads<TQ, GP>(p, b, kvh, wave, lane, L);
  my_page = (lane < np && my_page >= 0 && my_page < p.num_pages) ? my_page : -1;
  my_page2 = (lane + 64 < np && my_page2 >= 0 && my_page2 < p.num_pages) ? my_page2 : -1;
  PageRegs<BK, BV, A> ring[PIPE];
#pragma unroll
  for (int d = 0; d < PIPE; ++d) load(ring[d], d);
  __shared__ __attribute__((aligned(16))) float qs[GP * kQRow];
  QOperands qo;
  q_build<TQ, BK, GP>(p, wave, lane, L, qs, qo);
  v8i bq6[kQTerms];
  int sreg[kQTerms];
  constexpr float F = kF;
  const float qsf3 = qo.qsf3, qsf4 = qo.qsf4;
#pragma unroll
  for (int k = 0; k < kQTerms; ++k) {
    bq6[k] = qo.bq6[k];
    // scale byte t (selected per tile by op_sel): the term's scale for this lane's column
    // block, 2^-127 (contributes nothing) for the others
    uint32_t sc = 0;
#pragma unroll
    for (int t = 0; t < NB; ++t) sc |= (beta == t ? (uint32_t)(127 + qo.e1 - 4 * k) : 0u) << (8 * t);
    sreg[k] = (int)sc;
  }

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
  int S = 30;                    // P~ carries 2^(S - vcls)
  int hmax = -128;               // exponent of the lane's largest P~ accumulated so far (units of S)

  // ---- page walk: compute page i from ring slot i % PIPE, then refill the slot ----
  auto compute = [&](const PageRegs<BK, BV, A>& pr, int i) {
    const int valid_tokens = nseq - (pg0 + i) * kPageTokens;   // >= 1
    const bool partial = valid_tokens < kPageTokens;

    // ---- scores: tile t4 = tokens 16*(n/4) + 4*t4 + n%4 in rows n ----
    // one 16x16x128 product per tile, key plane and q' term; the op_sel'd scale byte keeps
    // tile t4 out of every column block but t4 % NB
    f32x4 sacc[A];
#pragma unroll
    for (int a = 0; a < A; ++a) sacc[a] = f32x4{};
    // products of tile t4 with the q' terms K0 .. K0 + NT - 1
    using std::integral_constant;
    auto key_products = [&](int t4, auto k_first, auto k_count) {
      constexpr int K0 = decltype(k_first)::value, NT = decltype(k_count)::value;
      if constexpr (BK == 4) {
        const u32x4 w = pr.k[t4];
        const v8i lo = {(int)(w[0] & kFp4CodeMask), (int)(w[1] & kFp4CodeMask), (int)(w[2] & kFp4CodeMask),
                        (int)(w[3] & kFp4CodeMask), 0, 0, 0, 0};
        const v8i hi = {(int)((w[0] >> 2) & kFp4CodeMask), (int)((w[1] >> 2) & kFp4CodeMask),
                        (int)((w[2] >> 2) & kFp4CodeMask), (int)((w[3] >> 2) & kFp4CodeMask), 0, 0, 0, 0};
#pragma unroll
        for (int k = K0; k < K0 + NT; ++k) {
          sacc[t4 / NB] = mma_fp4_fp6(t4 % NB, lo, bq6[k], sacc[t4 / NB], sreg[k]);
          sacc[t4 / NB] = mma_fp4_fp6(t4 % NB, hi, bq6[k], sacc[t4 / NB], sreg[k], kTimes4Scale);
        }
      } else {
        const uint32_t w0 = pr.k[t4][0], w1 = pr.k[t4][1];
        const v8i av = {(int)(w0 & kFp4CodeMask), (int)((w0 >> 2) & kFp4CodeMask), (int)(w1 & kFp4CodeMask),
                        (int)((w1 >> 2) & kFp4CodeMask), 0, 0, 0, 0};
#pragma unroll
        for (int k = K0; k < K0 + NT; ++k) sacc[t4 / NB] = mma_fp4_fp6(t4 % NB, av, bq6[k], sacc[t4 / NB], sreg[k]);
        if constexpr (BK == 3) {
          // high plane: operand element (dword d, nibble i) is channel offset
          // 16(d/2) + d%2 + 2i, whose bit sits at 4i + d; shifted to bit 2 of the nibble it
          // is the fp4 value 2 = (4 * bit) / 2, so the two products add to code / 2
          const uint32_t h = pr.kh[t4];
          const v8i ah = {(int)((h << 2) & kFp4HighMask), (int)((h << 1) & kFp4HighMask), (int)(h & kFp4HighMask),
                          (int)((h >> 1) & kFp4HighMask), 0, 0, 0, 0};
#pragma unroll
          for (int k = K0; k < K0 + NT; ++k) sacc[t4 / NB] = mma_fp4_fp6(t4 % NB, ah, bq6[k], sacc[t4 / NB], sreg[k]);
        }
      }
    };
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) key_products(t4, integral_constant<int, 0>{}, integral_constant<int, kQBase>{});
    // metadata of the lane's tokens (4 consecutive per tile: 8 bytes each).  The fp16
    // scales and zeros enter the arithmetic as fp16 operands of mixed fma (no conversions).
    // score = s_k * (q' . code) + z_k * sum(q'), with sum(q') as the terms carry it
    float x[A][4];
    u32x2 svp[A], zvp[A];
#pragma unroll
    for (int a = 0; a < A; ++a) {
      svp[a] = pr.meta[a][2];
      zvp[a] = pr.meta[a][3];
    }
    // the lane's largest score (the column's max is reduced only where it is needed)
    auto token_scores = [&](float qsf) {
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
      }
      if (partial) {                        // absent tokens: no weight, no garbage scale
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
      float mx = x[0][0];
#pragma unroll
      for (int a = 0; a < A; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[a][r]);
      return mx;
    };
    float mx = token_scores(qsf3);
    // Large scores take a fourth q' term: a column whose max |score| passes kBigScore / F
    // has a lane whose own max does too (the column max is one of the lanes' maxima, and
    // when it is below -kBigScore / F every lane's is).  A lane without tokens in a partial
    // page has mx = -inf and takes the branch too.
    if (__any(fabsf(mx) > kBigScore / F)) {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) key_products(t4, integral_constant<int, kQBase>{}, integral_constant<int, 1>{});
      mx = token_scores(qsf4);
    }
    // ---- online softmax, per column ----
    // Lazy maximum: the reference max m of a column moves only when the page's scores
    // exceed it by more than kLag (log2 units), so p = 2^(F(x - m)) <= 2^kLag.  Rescaling
    // is wave-uniform, so an eager rule would run it whenever any of the 16 columns grows.
    constexpr float kLag = 8.0f;
    // a column's max passes m + kLag / F exactly when one of its lanes' maxima does
    if (__any(F * (mx - m) > kLag)) {
      const float mxc = col_max(mx);
      const bool need_m = F * (mxc - m) > kLag;   // false when the column has no token here
      const float m_new = need_m ? mxc : m;
      const float alpha = exp2f(F * (m - m_new));
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc_o[mt] *= alpha;
#pragma unroll
      for (int a = 0; a < A; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          lsum[a][r] *= alpha;
          zacc[a][r] *= alpha;
          nb[a][r] = (float)(S - vcls[a][r]) - F * m_new;
        }
      m = m_new;
    }
    float pt[A][4];
    uint32_t pbits = 0;                    // largest P~ of the lane (P~ >= 0: bit patterns order)
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
        pbits = max(pbits, __float_as_uint(pt[a][r]));
      }
    // The P.V operand P~ = p s_v 2^(S - vcls) is fp16.  S follows the tokens that carry the
    // weight: it moves when the column's largest P~ of the page leaves [2^kPtLo, 2^(kPtHi+1)),
    // to 2^kPtTarget, which leaves 2^kLag for later pages' p.  A token whose P~ is below the
    // fp16 normal range then weighs less than 2^-(14 + kPtLo) of the page's largest, and its
    // rounding error is below 2^-(25 + kPtLo) of it.  An upward move is capped so that the
    // largest P~ already accumulated stays below 2^kStateMax in the new units (fp32 state).
    // The page's own sums are already in lsum / zacc: powers of two scale them exactly.
    // (3-bit values: the high plane's P~ carries up to 2^6 more.)
    constexpr int kPtHi = BV == 3 ? 8 : 14;
    constexpr int kPtTarget = kPtHi - (int)kLag - 2;
    constexpr int kPtLo = kPtTarget - 8;
    constexpr int kStateMax = 48;
    // The column's largest P~ leaves the range above when one of its lanes' largest does,
    // and below when every lane of the column that holds weight is below it: a vote of the
    // lanes (column n owns lanes n, n + 16, n + 32, n + 48) decides whether the column's
    // largest is needed at all.  hmax is kept per lane; the column's is the largest of its
    // lanes'.
    const int el = (int)(pbits >> 23) - 127;          // the lane's largest P~ exponent (pbits > 0)
    const uint64_t held = __ballot(pbits != 0u);
    const uint64_t in_range = __ballot(pbits != 0u && el >= kPtLo);
    auto fold = [](uint64_t v) -> uint32_t { v |= v >> 32; v |= v >> 16; return (uint32_t)v & 0xFFFFu; };
    if (__any(pbits != 0u && el > kPtHi) || (fold(held) & ~fold(in_range)) != 0u) {
      const int pcol = col_max_i((int)pbits);
      const int e = (pcol >> 23) - 127;               // exponent of the largest P~ (pcol > 0)
      const bool need_s = pcol != 0 && (e > kPtHi || e < kPtLo);
      if (__any(need_s)) {
        const int hcol = col_max_i(hmax);               // (lane exchanges stay outside divergent code)
        const int d = need_s ? min(kPtTarget - e, kStateMax - hcol) : 0;
        const float f = __builtin_amdgcn_ldexpf(1.0f, d);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) acc_o[mt] *= f;
#pragma unroll
        for (int a = 0; a < A; ++a)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            lsum[a][r] *= f;
            zacc[a][r] *= f;
            pt[a][r] *= f;
            nb[a][r] += (float)d;
          }
        S += d;
        hmax += d;
      }
    }
    hmax = max(hmax, pbits != 0u ? el : -128);

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
  float (*red_o)[16][kHeadDim + 1] = reinterpret_cast<float (*)[16][kHeadDim + 1]>(smem);
  float (*red_ml)[16][2] = reinterpret_cast<float (*)[16][2]>(smem + kWaves * 16 * (kHeadDim + 1) * 4);
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
  // the step's new token joins the merge of chunk 0 as one more part: its score q.k_new
  // (log2 units; q'.k' = q.k, so no transform), weight 1 and value row v_new.  Wave w sums
  // the products of heads w, w + 4, ... over its lanes' channel pairs.
  __shared__ float s_new[16];
  const bool new_part = new_tok && chunk == 0;
  if (new_part) {
    const TQ* krow = reinterpret_cast<const TQ*>(p.knew) + ((int64_t)b * p.heads_kv + kvh) * kHeadDim;
    const float k0 = Elem<TQ>::get(krow, 2 * lane), k1 = Elem<TQ>::get(krow, 2 * lane + 1);
    for (int gg = wave; gg < G; gg += kWaves) {
      const TQ* qrow = reinterpret_cast<const TQ*>(p.q) + ((int64_t)b * p.heads_q + (int64_t)kvh * G + gg) * kHeadDim;
      float d = __builtin_fmaf(Elem<TQ>::get(qrow, 2 * lane), k0, Elem<TQ>::get(qrow, 2 * lane + 1) * k1);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
      if (lane == 0) s_new[gg] = d * p.score_scale;
    }
  }
  __syncthreads();

  // ---- merge the waves and the column blocks of each head ----
  const int hq0 = kvh * G;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kThreads) {
    const int gg = idx / kHeadDim, ch = idx % kHeadDim;
    // every read first, with no branch between them, so that they are all in flight at once
    constexpr int NP = kWaves * NB;
    float mw[NP], lw[NP], ow[NP];
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const int col = bb * GP + gg;
        mw[w * NB + bb] = red_ml[w][col][0];
        lw[w * NB + bb] = red_ml[w][col][1];
        ow[w * NB + bb] = red_o[w][col][ch];
      }
    // the new token's part (chunk 0 of a step: score, weight 1, value; else no part)
    const float m_nt = new_part ? s_new[gg] : -__builtin_inff();
    const float v_nt = new_part
        ? Elem<TQ>::get(reinterpret_cast<const TQ*>(p.vnew) + ((int64_t)b * p.heads_kv + kvh) * kHeadDim, ch)
        : 0.0f;
    float M = m_nt;
#pragma unroll
    for (int k = 0; k < NP; ++k) M = fmaxf(M, mw[k]);
    // a part without tokens (m = -inf) is left out by a select: its other fields are not
    // meaningful (its softmax state never had a finite maximum); a head without any token
    // (M = -inf) keeps L = O = 0
    const float Mf = M == -__builtin_inff() ? 0.0f : M;
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const bool live = mw[k] != -__builtin_inff();
      const float f = __builtin_amdgcn_exp2f(mw[k] - Mf);
      L = live ? __builtin_fmaf(lw[k], f, L) : L;
      O = live ? __builtin_fmaf(ow[k], f, O) : O;
    }
    if (new_part) {
      const float f = __builtin_amdgcn_exp2f(m_nt - Mf);
      L += f;
      O = __builtin_fmaf(v_nt, f, O);
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

// Log-sum-exp merge of the chunks of one (sequence, query head) row: thread = channel.
// Chunks go 64 at a time: each thread's partial outputs of the block are loaded first, then
// the chunks' (max, sum) pairs are staged in LDS by the whole block, so a block costs about
// one memory round trip.  Blocks of chunks merge online.
constexpr int kCombineBlock = 64;
__global__ __launch_bounds__(128) void combine_kernel(DecodeParams p) {
  __shared__ float sml[2 * kCombineBlock];
  const int64_t row = blockIdx.x;        // b * Hq + hq
  const int ch = threadIdx.x;
  const float* ml = p.ws_ml + row * p.chunks * 2;
  const float* po = p.ws_o + row * p.chunks * kHeadDim + ch;
  float M = -__builtin_inff(), L = 0.0f, O = 0.0f;
  for (int c0 = 0; c0 < p.chunks; c0 += kCombineBlock) {
    const int nc = min(kCombineBlock, p.chunks - c0);
    // the block's partial outputs go out first (they do not depend on the maxima), in groups
    // of 8 behind a uniform test, so that one memory round trip covers them all
    float ov[kCombineBlock];
#pragma unroll
    for (int c8 = 0; c8 < kCombineBlock; c8 += 8)
      if (c8 < nc) {
#pragma unroll
        for (int c = c8; c < c8 + 8; ++c) ov[c] = po[(int64_t)(c0 + min(c, nc - 1)) * kHeadDim];
      }
    __syncthreads();
    if (ch < 2 * nc) sml[ch] = ml[2 * c0 + ch];
    __syncthreads();
    float Mb = -__builtin_inff();
    for (int c = 0; c < nc; ++c) Mb = fmaxf(Mb, sml[2 * c]);
    if (Mb == -__builtin_inff()) continue;           // no tokens in these chunks
    const float Mn = fmaxf(M, Mb);
    const float r = M == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    L *= r;
    O *= r;
    M = Mn;
    // a chunk without tokens (m = -inf) is left out by a select
#pragma unroll
    for (int c8 = 0; c8 < kCombineBlock; c8 += 8)
      if (c8 < nc) {
#pragma unroll
        for (int c = c8; c < c8 + 8; ++c) {
          const float mc = sml[2 * min(c, nc - 1)];
          const bool live = c < nc && mc != -__builtin_inff();
          const float f = __builtin_amdgcn_exp2f(mc - M);
          L = live ? __builtin_fmaf(sml[2 * min(c, nc - 1) + 1], f, L) : L;
          O = live ? __builtin_fmaf(ov[c], f, O) : O;
        }
      }
  }
  p.out[row * kHeadDim + ch] = L > 0.0f ? O / L : 0.0f;
}

template <typename TQ, int BK, int BV>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.chunks, (unsigned)p.heads_kv, (unsigned)(p.append_blocks ? 2 * p.batch : p.batch));
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

// ---------------------------------------------------------------------------------
// Scratch of the allocation-free decode.  Host code never passes the array's name to a
// kernel (on the host it only stands in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device, with that device current, and is kept per device.
// ---------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    // concurrent first calls look up the same address; either store is right
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

DecodeSplit decode_split(int batch, int heads_kv, int max_seq_len) {
  const int pages = (max_seq_len + kPageTokens - 1) / kPageTokens;
  const int64_t units = (int64_t)batch * heads_kv;
  // about kResidentWaves waves (one resident round), kMinPagesPerWave to 128 pages per wave
  // (a wave's page ids fit two registers, one per lane; batch 16 x 128K then runs as one
  // round of 4 chunks per sequence instead of two rounds of 8, 3% faster)
  int64_t ppw = (units * pages + kResidentWaves - 1) / kResidentWaves;
  if (ppw < kMinPagesPerWave) ppw = kMinPagesPerWave;
  if (ppw > 128) ppw = 128;
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
