// Read path: one decode step of grouped-query attention over the quantized paged cache.
//
// Method: "WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms" §4.1 (query
// heads of a group share one KV head), §4.2 (query-side compensation q' = q T^-T after
// RoPE; values stay in the folded basis that W_O absorbs); "Spend Bits Where Queries
// Look" (NOVA-KV project page), "Three requirements": the cache is read on every step,
// so per-element read work is paid over the whole cache.
//
// Design (gfx950, wave64).  Grid (chunk, KV head, sequence), 4 waves per workgroup; each
// wave walks a contiguous run of pages with an online softmax, the workgroup merges its
// four waves, and a second kernel merges chunks when a sequence is split.
//
// Both contractions run on the matrix cores as 16x16x32 fp16 products with fp32
// accumulation, with the query heads of the group as the N = 16 columns:
//   scores  S[token][head] = codes_K[token][ch] . q''[ch][head]
//   output  O[ch][head]   += codes_V[ch][token] . P~[token][head]
// Codes are never converted arithmetically: an AND of the packed word with a mask
// leaves, in each 16-bit half, one code at bit b*e of the mantissa of a subnormal fp16,
// i.e. the exact value code * 2^(b*e) * 2^-24.  Codes in the top bits of a half are
// shifted down first.  The factor 2^-(b*e) is folded into the other operand (q'' per
// channel, P~ per token), so one AND yields two operands.  Scale and zero are applied
// outside the products:
//   score_t = s_t * (q . code_t) + z_t * sum(q)
//   out     = (sum_t p_t s_t code_t + sum_t p_t z_t) / sum_t p_t
// The token order inside a score tile is chosen so that each lane's score accumulators
// hold exactly the tokens that lane feeds to the P.V product; no shuffles are needed.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxGroup = 16;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half8 as_half8(u32x4 w) { return __builtin_bit_cast(half8, w); }

// Position class e of the code pair p of a word (the fp16 mantissa bit offset is b*e).
template <int B> __host__ __device__ constexpr int pair_class(int p) {
  return B == 2 ? (p <= 4 ? p : p - 5) : (p <= 1 ? p : p - 2);
}
template <int B> constexpr int num_classes() { return B == 2 ? 5 : 2; }

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

__device__ __forceinline__ float lo_f16(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w)[0]; }
__device__ __forceinline__ float hi_f16(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w)[1]; }

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  half2_t h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float wave_max16(float v) {  // over lanes l, l^16, l^32, l^48
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float wave_sum16(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
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

template <int BK, int BV, typename TQ>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  constexpr int kCodeBytesK = code_bytes(BK), kCodeBytesV = code_bytes(BV);
  constexpr int NCV = num_classes<BV>();
  const int chunk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = p.group;
  const int hq0 = kvh * G;

  __shared__ float qs[kMaxGroup][kHeadDim];
  __shared__ uint16_t qh[kMaxGroup][kHeadDim];
  __shared__ float hconst[kMaxGroup][2];
  __shared__ float red_o[kWaves][kMaxGroup][kHeadDim];
  __shared__ float red_ml[kWaves][kMaxGroup][2];

  // ---- query compensation q' = q T^-T, scaled to log2 units ----
  const TQ* qb = reinterpret_cast<const TQ*>(p.q) + ((int64_t)b * p.heads_q + hq0) * kHeadDim;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256) qs[idx / kHeadDim][idx % kHeadDim] = Elem<TQ>::get(qb, idx);
  __syncthreads();
  float qv[(kMaxGroup * kHeadDim) / 256];
  {
    const float* ti = p.tinv ? p.tinv + (int64_t)kvh * kHeadDim * kHeadDim : nullptr;
    int r = 0;
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256, ++r) {
      const int g = idx / kHeadDim, j = idx % kHeadDim;
      float acc = 0.0f;
      if (ti) {
        for (int c = 0; c < kHeadDim; ++c) acc = __builtin_fmaf(qs[g][c], ti[c * kHeadDim + j], acc);
      } else {
        acc = qs[g][j];
      }
      qv[r] = acc * p.score_scale;
    }
    __syncthreads();
    r = 0;
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256, ++r) qs[idx / kHeadDim][idx % kHeadDim] = qv[r];
    __syncthreads();
  }
  // fp16 operand q''[c] = q'[c] * 2^(E - BK*e(c)), E per head so that max|q''| < 2^15
  for (int g = wave; g < G; g += kWaves) {
    const float a0 = qs[g][lane], a1 = qs[g][lane + 64];
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
      qh[g][c] = hbits;
      qsum += ldexpf(f16_bits_to_f32(hbits), sh - E);
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) qsum += __shfl_xor(qsum, d);
    if (lane == 0) {
      hconst[g][0] = qsum;
      hconst[g][1] = ldexpf(1.0f, 24 - E);
    }
  }
  __syncthreads();

  const int kg = lane >> 4, i16 = lane & 15;
  const int g = i16;                       // head column of this lane
  const bool gvalid = g < G;
  u32x4 bq[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t lo = gvalid ? qh[g][k_channel<BK>(s, kg, 2 * jj)] : 0u;
      const uint32_t hi = gvalid ? qh[g][k_channel<BK>(s, kg, 2 * jj + 1)] : 0u;
      bq[s][jj] = lo | (hi << 16);
    }
  const float F = gvalid ? hconst[g][1] : 1.0f;             // score = F * x'
  const float qsf = gvalid ? hconst[g][0] / hconst[g][1] : 0.0f;

  // ---- walk this wave's pages ----
  const int n = min(p.seq_lens[b], p.max_pages * kPageTokens);
  const int npages = (n + kPageTokens - 1) / kPageTokens;
  const int wv = chunk * kWaves + wave;
  const int pg0 = wv * p.pages_per_wave;
  const int pg1 = min(pg0 + p.pages_per_wave, npages);

  f32x4 acc_o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc_o[mt] = f32x4{};
  float lsum[NCV], zacc[NCV];
#pragma unroll
  for (int e = 0; e < NCV; ++e) { lsum[e] = 0.0f; zacc[e] = 0.0f; }
  float m = -__builtin_inff();   // running max of x' for this lane's head
  int S = 30;                    // P~ = p * s_v * 2^(S - BV*e)

  const int64_t kstride = (int64_t)block_bytes(BK), vstride = (int64_t)block_bytes(BV);
  const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;

  for (int pg = pg0; pg < pg1; ++pg) {
    const int64_t page = bt[pg];
    if (page < 0 || page >= p.num_pages) continue;   // invalid page id: contributes nothing
    const uint8_t* kb = p.kpool + (page * p.heads_kv + kvh) * kstride;
    const uint8_t* vb = p.vpool + (page * p.heads_kv + kvh) * vstride;

    // K codes for the four 16-token tiles
    uint32_t kw[4][BK == 2 ? 2 : 4];
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
      const int tok = 16 * (i16 >> 2) + 4 * b4 + (i16 & 3);
      if constexpr (BK == 2) {
        u32x2 w = *reinterpret_cast<const u32x2*>(kb + tok * 32 + kg * 8);
        kw[b4][0] = w[0]; kw[b4][1] = w[1];
      } else {
        u32x4 w = *reinterpret_cast<const u32x4*>(kb + tok * 64 + kg * 16);
        kw[b4][0] = w[0]; kw[b4][1] = w[1]; kw[b4][2] = w[2]; kw[b4][3] = w[3];
      }
    }
    // metadata of tokens 16kg .. 16kg+15 (two fp16 per word)
    const u32x4* kmeta = reinterpret_cast<const u32x4*>(kb + kCodeBytesK);
    const u32x4* vmeta = reinterpret_cast<const u32x4*>(vb + kCodeBytesV);
    u32x4 sk0 = kmeta[2 * kg], sk1 = kmeta[2 * kg + 1];
    u32x4 zk0 = kmeta[8 + 2 * kg], zk1 = kmeta[8 + 2 * kg + 1];
    u32x4 sv0 = vmeta[2 * kg], sv1 = vmeta[2 * kg + 1];
    u32x4 zv0 = vmeta[8 + 2 * kg], zv1 = vmeta[8 + 2 * kg + 1];
    // V codes: word rows of this lane group's tokens, channels 4*i16.. and 64+4*i16..
    u32x4 vw[BV == 2 ? 1 : 2][2];
#pragma unroll
    for (int r = 0; r < (BV == 2 ? 1 : 2); ++r) {
      const int row = BV == 2 ? kg : 2 * kg + r;
      const u32x4* vrow = reinterpret_cast<const u32x4*>(vb + row * kHeadDim * 4);
      vw[r][0] = vrow[i16];
      vw[r][1] = vrow[16 + i16];
    }
    auto word8 = [](const u32x4& a, const u32x4& c, int w) -> uint32_t { return w < 4 ? a[w] : c[w - 4]; };

    // ---- scores ----
    float x[16];
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
      f32x4 acc = f32x4{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t w = BK == 2 ? kw[b4][s / 2] : kw[b4][s];
        const uint32_t ws = shifted<BK>(w);
        u32x4 a;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) a[jj] = code_pair<BK>(w, ws, BK == 2 ? 4 * (s % 2) + jj : jj);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(a), as_half8(bq[s]), acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = 4 * b4 + r;
        const uint32_t skw = word8(sk0, sk1, u / 2), zkw = word8(zk0, zk1, u / 2);
        const float sk = (u & 1) ? hi_f16(skw) : lo_f16(skw);
        const float zk = (u & 1) ? hi_f16(zkw) : lo_f16(zkw);
        x[u] = __builtin_fmaf(acc[r], sk, zk * qsf);
      }
    }
    const int valid_tokens = n - pg * kPageTokens;   // >= 1
    const bool partial = valid_tokens < kPageTokens;
    if (partial) {
#pragma unroll
      for (int u = 0; u < 16; ++u) x[u] = (16 * kg + u < valid_tokens) ? x[u] : -__builtin_inff();
    }

    // ---- online softmax ----
    float mx = x[0];
#pragma unroll
    for (int u = 1; u < 16; ++u) mx = fmaxf(mx, x[u]);
    mx = wave_max16(mx);
    u16x2 svm = __builtin_bit_cast(u16x2, sv0[0]);
#pragma unroll
    for (int w = 1; w < 8; ++w) svm = __builtin_elementwise_max(svm, __builtin_bit_cast(u16x2, word8(sv0, sv1, w)));
    int svmax = max((int)svm[0], (int)svm[1]);
    if (partial) {
      svmax = 0;
      for (int u = 0; u < 16; ++u) {
        const uint32_t svw = word8(sv0, sv1, u / 2);
        const int bits16 = (u & 1) ? (int)(svw >> 16) : (int)(svw & 0xFFFFu);
        svmax = (16 * kg + u < valid_tokens) ? max(svmax, bits16) : svmax;
      }
    }
    svmax = max(svmax, __shfl_xor(svmax, 16));
    svmax = max(svmax, __shfl_xor(svmax, 32));
    const int s_page = svmax >= 0x400 ? 14 - ((svmax >> 10) - 15) : 29;
    const int S_new = min(S, s_page);
    const float m_new = fmaxf(m, mx);
    if (__any(m_new > m || S_new != S)) {
      const float alpha = exp2f(F * (m - m_new) + (float)(S_new - S));
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc_o[mt] *= alpha;
#pragma unroll
      for (int e = 0; e < NCV; ++e) { lsum[e] *= alpha; zacc[e] *= alpha; }
      m = m_new;
      S = S_new;
    }
    float nb[NCV];
#pragma unroll
    for (int e = 0; e < NCV; ++e) nb[e] = (float)(S - BV * e) - F * m;
    float pt[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = v_token_class<BV>(u);
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(F, x[u], nb[e]));
      const uint32_t svw = word8(sv0, sv1, u / 2), zvw = word8(zv0, zv1, u / 2);
      const float sv = (u & 1) ? hi_f16(svw) : lo_f16(svw);
      const float zv = (u & 1) ? hi_f16(zvw) : lo_f16(zvw);
      if (partial && !(16 * kg + u < valid_tokens)) {
        pt[u] = 0.0f;
      } else {
        lsum[e] += pe;
        zacc[e] = __builtin_fmaf(pe, zv, zacc[e]);
        pt[u] = pe * sv;
      }
    }

    // ---- P.V ----
    u32x4 bp[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) bp[s][jj] = pack_f16x2(pt[v_token<BV>(s, 2 * jj)], pt[v_token<BV>(s, 2 * jj + 1)]);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t w = BV == 2 ? vw[0][mt >> 2][mt & 3] : vw[s][mt >> 2][mt & 3];
        const uint32_t ws = shifted<BV>(w);
        u32x4 a;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) a[jj] = code_pair<BV>(w, ws, BV == 2 ? 4 * s + jj : jj);
        acc_o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(a), as_half8(bp[s]), acc_o[mt], 0, 0, 0);
      }
    }
  }

  // ---- wave result: m (log2 units), l, o_num = acc * 2^(24-S) + z ----
  float l = 0.0f, z = 0.0f;
#pragma unroll
  for (int e = 0; e < NCV; ++e) {
    l += ldexpf(lsum[e], BV * e - S);
    z += ldexpf(zacc[e], BV * e - S);
  }
  l = wave_sum16(l);
  z = wave_sum16(z);
  const float mlog2 = (pg1 > pg0) ? F * m : -__builtin_inff();
  const float oscale = ldexpf(1.0f, 24 - S);
  if (gvalid) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ch = 4 * (4 * kg + r) + (mt & 3) + 64 * (mt >> 2);
        red_o[wave][g][ch] = __builtin_fmaf(acc_o[mt][r], oscale, z);
      }
    if (kg == 0) {
      red_ml[wave][g][0] = mlog2;
      red_ml[wave][g][1] = (pg1 > pg0) ? l : 0.0f;
    }
  }
  __syncthreads();

  // ---- merge the four waves; write the result or the chunk partial ----
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256) {
    const int gg = idx / kHeadDim, ch = idx % kHeadDim;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_ml[w][gg][0]);
    float L = 0.0f, O = 0.0f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = red_ml[w][gg][0];
        if (mw != -__builtin_inff()) {
          const float f = exp2f(mw - M);
          L = __builtin_fmaf(red_ml[w][gg][1], f, L);
          O = __builtin_fmaf(red_o[w][gg][ch], f, O);
        }
      }
    }
    const int hq = hq0 + gg;
    if (p.chunks == 1) {
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

template <int BK, int BV>
hipError_t launch_bits(const DecodeParams& p, int q_dtype, hipStream_t stream) {
  dim3 grid((unsigned)p.chunks, (unsigned)p.heads_kv, (unsigned)p.batch);
  dim3 block(256);
  switch (q_dtype) {
    case 0: hipLaunchKernelGGL((decode_kernel<BK, BV, float>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((decode_kernel<BK, BV, __bf16>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_kernel<BK, BV, _Float16>), grid, block, 0, stream, p); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.chunks == 1) return err;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(p.batch * p.heads_q)), dim3(kHeadDim), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

DecodeSplit decode_split(int batch, int heads_kv, int max_seq_len) {
  const int pages = (max_seq_len + kPageTokens - 1) / kPageTokens;
  const int64_t units = (int64_t)batch * heads_kv;
  // about 8192 waves in flight over the chip, at least 4 pages per wave
  int64_t ppw = (units * pages + 8191) / 8192;
  if (ppw < 4) ppw = 4;
  if (ppw > 256) ppw = 256;
  const int64_t waves = pages > 0 ? (pages + ppw - 1) / ppw : 1;
  DecodeSplit s;
  s.pages_per_wave = (int)ppw;
  s.chunks = (int)((waves + kWaves - 1) / kWaves);
  return s;
}

hipError_t launch_decode(const DecodeParams& p, int bits_k, int bits_v, int q_dtype, hipStream_t stream) {
  if (bits_k == 2 && bits_v == 2) return launch_bits<2, 2>(p, q_dtype, stream);
  if (bits_k == 2 && bits_v == 4) return launch_bits<2, 4>(p, q_dtype, stream);
  if (bits_k == 4 && bits_v == 2) return launch_bits<4, 2>(p, q_dtype, stream);
  return launch_bits<4, 4>(p, q_dtype, stream);
}

}  // namespace kvq
