// Full-precision cache windows: the read half (attention over the window positions,
// merged with the quantized partials) and the prefill of the windows.
//
// Method: "WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms" §4.4 (the first
// S_sink and the newest S_keep positions stay in full precision; the middle positions are
// quantized in batches of S_flush; new positions are read at full precision by their step
// before the batches they make eligible are quantized) and §4.5 (the windows are a small
// fraction of the sequence).
//
// window_kernel: grid (KV head, sequence), 4 waves.  The window keys are stored before
// the key transform, so their scores use the plain query.  Scores and softmax in fp32,
// log2 units (the query is scaled by sm_scale * log2 e), tile by tile with a running max
// per head.  The result (max, sum, unnormalised output) is merged with the partials that
// decode_kernel wrote to the workspace for the quantized positions, and the output is
// written.  In a decode step the kernel also stores the new position's key and value in
// the window row (it reads them for the scores from the step's inputs, not from there).
//
// window_store_kernel: the full-precision positions of a packed batch of fresh prompts
// into their window rows (the middle positions go through the append kernels).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWinWaves = 4;
constexpr int kWinThreads = 64 * kWinWaves;

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a row; every lane of the row gets the same value.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror: the other quad of the half row
  v += dpp<0x140>(v);   // row_mirror: the other half row
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d);
  return v;
}

// Eight consecutive elements as raw 16-byte words, converted to fp32 when used.
template <typename T> struct Raw8 {
  u32x4 w[sizeof(T) / 2];
};
template <typename T> __device__ __forceinline__ Raw8<T> load8(const T* p) {
  Raw8<T> r;
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 2); ++k) r.w[k] = reinterpret_cast<const u32x4*>(p)[k];
  return r;
}
template <typename T> __device__ __forceinline__ Raw8<T> zero8() {
  Raw8<T> r;
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 2); ++k) r.w[k] = u32x4{0u, 0u, 0u, 0u};
  return r;
}
__device__ __forceinline__ void to_f32(const Raw8<float>& r, float (&o)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = __uint_as_float(r.w[e / 4][e % 4]);
}
__device__ __forceinline__ void to_f32(const Raw8<__bf16>& r, float (&o)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = __uint_as_float(r.w[0][e] << 16);
    o[2 * e + 1] = __uint_as_float(r.w[0][e] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void to_f32(const Raw8<_Float16>& r, float (&o)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = f16_bits_to_f32(r.w[0][e] & 0xFFFFu);
    o[2 * e + 1] = f16_bits_to_f32(r.w[0][e] >> 16);
  }
}

// Tile: 4 waves x 4 rows of 16 lanes x NI tokens; lane (row tg, column) holds channels
// 8*column .. +7 of token (wave*NI + i)*4 + tg of the tile.
template <typename T, int GP>
__global__ __launch_bounds__(kWinThreads) void window_kernel(DecodeParams p, WindowParams w) {
  constexpr int NI = sizeof(T) == 4 ? 4 : 8;
  constexpr int kTile = kWinWaves * 4 * NI;
  constexpr int HW = GP / kWinWaves;           // heads per wave in the softmax update
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tg = lane >> 4, col = lane & 15, c0 = 8 * col;
  const int G = p.group;
  const WindowShape ws = p.win;

  __shared__ __attribute__((aligned(16))) float qs[GP][kHeadDim];
  __shared__ float sp[GP][kTile];              // scores, then weights
  __shared__ float alpha_s[GP];
  __shared__ float ml_s[GP][2];
  __shared__ __attribute__((aligned(16))) float red[kWinWaves][GP][kHeadDim];

  // ---- the window positions of this sequence ----
  // (as decode_kernel: at most max_pages pages of quantized positions; a length beyond
  // what the cache and the ring can hold reads the newest keep + flush positions)
  const int len = max(p.seq_lens[b], 0);
  const int nq = min(window_quantized(max(len - p.win_pending, 0), ws), p.max_pages * kPageTokens);
  const int ns = min(len, ws.sink);                                   // sink positions 0 .. ns-1
  const int nr = min(max(len - ws.sink - nq, 0), ws.keep + ws.flush);  // then the newest nr
  const int row = w.win_rows ? w.win_rows[b] : b;
  const bool row_ok = row >= 0 && row < w.rows;
  const int nf = row_ok ? ns + nr : 0;
  const bool has_new = w.k_new != nullptr && len >= 1 && row_ok;
  const int64_t tstride = (int64_t)p.heads_kv * kHeadDim;   // elements per window slot
  const int64_t rbase = (int64_t)(row_ok ? row : 0) * window_width(ws) * tstride + (int64_t)kvh * kHeadDim;
  const T* kw = reinterpret_cast<const T*>(w.kwin) + rbase;
  const T* vw = reinterpret_cast<const T*>(w.vwin) + rbase;
  const int64_t nrow = ((int64_t)b * p.heads_kv + kvh) * kHeadDim;
  const T* kn = has_new ? reinterpret_cast<const T*>(w.k_new) + nrow : nullptr;
  const T* vn = has_new ? reinterpret_cast<const T*>(w.v_new) + nrow : nullptr;

  // ---- the step's new position into its window slot ----
  if (has_new && wave < 2) {
    T* dst = reinterpret_cast<T*>(wave == 0 ? w.kwin : w.vwin) + rbase + window_slot(len - 1, ws) * tstride;
    const T* src = wave == 0 ? kn : vn;
    dst[2 * lane] = src[2 * lane];
    dst[2 * lane + 1] = src[2 * lane + 1];
  }

  // ---- every load of the first phase goes out before any wait: the query heads, the
  // quantized partials' first chunk (the merge's inputs, written by the decode launch before
  // this one) and the first tile's window rows ----
  constexpr int NQ = GP * kHeadDim / kWinThreads;     // query elements and merge outputs per thread
  const T* qb = reinterpret_cast<const T*>(p.q) + ((int64_t)b * p.heads_q + (int64_t)kvh * G) * kHeadDim;
  float qv[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int idx = threadIdx.x + j * kWinThreads;
    const float x = Elem<T>::get(qb, min(idx, G * kHeadDim - 1));   // in range for every lane
    qv[j] = idx < G * kHeadDim ? x : 0.0f;
  }
  // chunk 0 of merge output idx = threadIdx.x + j * threads (at 16 query heads per KV head the
  // registers that would hold them, and the first tile, through the query staging cost
  // occupancy: those load at the merge and in the tile loop)
  constexpr bool kPre = GP <= 8;
  constexpr int NP = kPre ? NQ : 1;
  float pm0[NP], pl0[NP], po0[NP];
  auto load_chunk0 = [&](int j, float& m0, float& l0, float& o0) {
    const int idx = threadIdx.x + j * kWinThreads;
    const int64_t prow = (int64_t)b * p.heads_q + (int64_t)kvh * G + min(idx / kHeadDim, G - 1);
    m0 = p.ws_ml[prow * p.chunks * 2];
    l0 = p.ws_ml[prow * p.chunks * 2 + 1];
    o0 = p.ws_o[prow * p.chunks * kHeadDim + idx % kHeadDim];
  };
  if constexpr (kPre) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) load_chunk0(j, pm0[j], pl0[j], po0[j]);
  }
  Raw8<T> kr[NI], vr[NI];
  bool ok[NI];
  // ring slot of the first recent position (uniform): recent position len - nr + r sits r
  // slots later, wrapped once at most (r < nr <= keep + flush), so no token needs a division
  const int ring = ws.keep + ws.flush;
  const int srec = ws.sink + max(len - nr - ws.sink, 0) % ring;
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = t0 + (wave * NI + i) * 4 + tg;
      ok[i] = t < nf;
      if (ok[i]) {
        const int r = t - ns;
        const int pos = t < ns ? t : len - nr + r;
        const bool fresh = has_new && pos == len - 1;
        const int wrapped = srec + r >= ws.sink + ring ? srec + r - ring : srec + r;
        // 32-bit element offsets within the row (a row spans window_width * heads_kv * 128
        // elements)
        const uint32_t off = fresh ? (uint32_t)c0 : (uint32_t)(t < ns ? t : wrapped) * (uint32_t)tstride + c0;
        kr[i] = load8<T>((fresh ? kn : kw) + off);
        vr[i] = load8<T>((fresh ? vn : vw) + off);
      } else {
        kr[i] = zero8<T>();
        vr[i] = zero8<T>();
      }
    }
  };
  if constexpr (kPre) load_tile(0);
  // ---- query heads of the group, scaled to log2 units ----
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int idx = threadIdx.x + j * kWinThreads;
    qs[idx / kHeadDim][idx % kHeadDim] = qv[j] * p.score_scale;
  }

  float o[GP][8];
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[g][c] = 0.0f;
  float mrun[HW], lrun[HW];
#pragma unroll
  for (int k = 0; k < HW; ++k) {
    mrun[k] = -__builtin_inff();
    lrun[k] = 0.0f;
  }
  __syncthreads();

  for (int t0 = 0; t0 < nf; t0 += kTile) {
    if (!kPre || t0 > 0) load_tile(t0);
    // scores: lane column g keeps head g's score of its row's token
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kf[8];
      to_f32(kr[i], kf);
      float mine = -__builtin_inff();
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (g < G) {
          const f32x4 qa = *reinterpret_cast<const f32x4*>(&qs[g][c0]);
          const f32x4 qc = *reinterpret_cast<const f32x4*>(&qs[g][c0 + 4]);
          float d = 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e) d = __builtin_fmaf(qa[e], kf[e], d);
#pragma unroll
          for (int e = 0; e < 4; ++e) d = __builtin_fmaf(qc[e], kf[4 + e], d);
          d = row_sum16(d);
          mine = col == g ? d : mine;
        }
      }
      if (col < G) sp[col][(wave * NI + i) * 4 + tg] = ok[i] ? mine : -__builtin_inff();
    }
    __syncthreads();
    // running max and sum of heads wave, wave + 4, ...; the tile's weights replace its scores
#pragma unroll
    for (int k = 0; k < HW; ++k) {
      const int g = wave + kWinWaves * k;
      if (g < G) {
        float s[kTile / 64];
        float mx = -__builtin_inff();
#pragma unroll
        for (int u = 0; u < kTile / 64; ++u) {
          s[u] = sp[g][lane + 64 * u];
          mx = fmaxf(mx, s[u]);
        }
        mx = wave_max(mx);                        // finite: the tile's first token exists
        const float mnew = fmaxf(mrun[k], mx);
        const float alpha = exp2f(mrun[k] - mnew);
        float sum = 0.0f;
#pragma unroll
        for (int u = 0; u < kTile / 64; ++u) {
          const float e = exp2f(s[u] - mnew);
          sp[g][lane + 64 * u] = e;
          sum += e;
        }
        lrun[k] = __builtin_fmaf(lrun[k], alpha, wave_sum(sum));
        mrun[k] = mnew;
        if (lane == 0) alpha_s[g] = alpha;
      }
    }
    __syncthreads();
    // P.V
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      if (g < G) {
        const float a = alpha_s[g];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[g][c] *= a;
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[8];
      to_f32(vr[i], vf);
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (g < G) {
          const float pw = sp[g][(wave * NI + i) * 4 + tg];
#pragma unroll
          for (int c = 0; c < 8; ++c) o[g][c] = __builtin_fmaf(pw, vf[c], o[g][c]);
        }
      }
    }
    __syncthreads();                              // sp is rewritten by the next tile
  }

  // ---- sum the four rows of each wave, then the waves ----
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (g < G) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float v = o[g][c];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        o[g][c] = v;
      }
      if (tg == 0) {
        *reinterpret_cast<f32x4*>(&red[wave][g][c0]) = f32x4{o[g][0], o[g][1], o[g][2], o[g][3]};
        *reinterpret_cast<f32x4*>(&red[wave][g][c0 + 4]) = f32x4{o[g][4], o[g][5], o[g][6], o[g][7]};
      }
    }
  }
#pragma unroll
  for (int k = 0; k < HW; ++k) {
    const int g = wave + kWinWaves * k;
    if (g < G && lane == 0) {
      ml_s[g][0] = mrun[k];
      ml_s[g][1] = lrun[k];
    }
  }
  __syncthreads();

  // ---- merge with the quantized partials and write the output ----
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int idx = threadIdx.x + j * kWinThreads;
    if (idx >= G * kHeadDim) break;
    const int g = idx / kHeadDim, ch = idx % kHeadDim;
    const int64_t prow = (int64_t)b * p.heads_q + (int64_t)kvh * G + g;
    const float* ml = p.ws_ml + prow * p.chunks * 2;
    float m0, l0, o0;
    if constexpr (kPre) {
      m0 = pm0[j];
      l0 = pl0[j];
      o0 = po0[j];
    } else {
      load_chunk0(j, m0, l0, o0);
    }
    const float mw = ml_s[g][0];
    float M = fmaxf(mw, m0);
    for (int c = 1; c < p.chunks; ++c) M = fmaxf(M, ml[2 * c]);
    float L = 0.0f, O = 0.0f;
    if (M != -__builtin_inff()) {
      if (mw != -__builtin_inff()) {
        const float f = exp2f(mw - M);
        L = ml_s[g][1] * f;
        O = (((red[0][g][ch] + red[1][g][ch]) + red[2][g][ch]) + red[3][g][ch]) * f;
      }
      if (m0 != -__builtin_inff()) {
        const float f = exp2f(m0 - M);
        L = __builtin_fmaf(l0, f, L);
        O = __builtin_fmaf(o0, f, O);
      }
      for (int c = 1; c < p.chunks; ++c) {
        const float mc = ml[2 * c];
        if (mc != -__builtin_inff()) {
          const float f = exp2f(mc - M);
          L = __builtin_fmaf(ml[2 * c + 1], f, L);
          O = __builtin_fmaf(p.ws_o[(prow * p.chunks + c) * kHeadDim + ch], f, O);
        }
      }
    }
    p.out[prow * kHeadDim + ch] = L > 0.0f ? O / L : 0.0f;
  }
}

// Grid (window slot candidates, sequences): workgroup (t, b) copies the key and value of
// the t-th full-precision position of fresh prompt b (sink positions first, then the
// newest ones) from the packed prompt rows into b's window row.
template <typename T>
__global__ __launch_bounds__(256) void window_store_kernel(WindowStoreParams p) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int beg = p.cu_seqlens[b], len = p.cu_seqlens[b + 1] - beg;
  const int nq = window_quantized(len, p.win);
  const int ns = min(len, p.win.sink), nr = max(len - p.win.sink - nq, 0);
  const int row = p.win_rows ? p.win_rows[b] : b;
  if (t >= ns + nr || row < 0 || row >= p.rows) return;
  const int pos = t < ns ? t : p.win.sink + nq + (t - ns);
  if (beg < 0 || (int64_t)beg + pos >= p.n) return;              // outside the packed rows
  const int64_t n_el = (int64_t)p.heads * kHeadDim;                // elements of one position
  const int64_t src = ((int64_t)beg + pos) * n_el;
  const int64_t dst = ((int64_t)row * window_width(p.win) + window_slot(pos, p.win)) * n_el;
  const int words = (int)(n_el * (int64_t)sizeof(T) / 16);
  for (int c = threadIdx.x; c < 2 * words; c += 256) {
    const bool is_v = c >= words;
    const int cc = is_v ? c - words : c;
    const u32x4* s = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(is_v ? p.v : p.k) + src) + cc;
    u32x4* d = reinterpret_cast<u32x4*>(reinterpret_cast<T*>(is_v ? p.vwin : p.kwin) + dst) + cc;
    *d = *s;
  }
}

template <typename T>
hipError_t launch_window_typed(const DecodeParams& p, const WindowParams& w, hipStream_t stream) {
  const dim3 grid((unsigned)p.heads_kv, (unsigned)p.batch), block(kWinThreads);
  switch (p.gpad) {
    case 4: hipLaunchKernelGGL((window_kernel<T, 4>), grid, block, 0, stream, p, w); break;
    case 8: hipLaunchKernelGGL((window_kernel<T, 8>), grid, block, 0, stream, p, w); break;
    default: hipLaunchKernelGGL((window_kernel<T, 16>), grid, block, 0, stream, p, w); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_store_typed(const WindowStoreParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)window_width(p.win), (unsigned)p.batch), block(256);
  hipLaunchKernelGGL((window_store_kernel<T>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_window(const DecodeParams& p, const WindowParams& w, int q_dtype, hipStream_t stream) {
  switch (q_dtype) {
    case 0: return launch_window_typed<float>(p, w, stream);
    case 1: return launch_window_typed<__bf16>(p, w, stream);
    default: return launch_window_typed<_Float16>(p, w, stream);
  }
}

hipError_t launch_window_store(const WindowStoreParams& p, int dtype, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_store_typed<float>(p, stream);
    case 1: return launch_store_typed<__bf16>(p, stream);
    default: return launch_store_typed<_Float16>(p, stream);
  }
}

}  // namespace kvq
