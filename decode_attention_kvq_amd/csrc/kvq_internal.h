// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct AppendParams {
  const void* k;
  const void* v;
  const int64_t* slots;
  const void* t;          // [H][128][128] or null
  uint8_t* kpool;
  uint8_t* vpool;
  int64_t n;
  int64_t num_pages;
  int heads;
  int bits_k, bits_v;
  int quant_k, quant_v;   // 0 percentile, 1 rms
  int ilo, ihi;           // percentile order-statistic positions (0..127)
  float flo, fhi;         // interpolation weights
  float alpha_k, alpha_v;
};

// Width of the insertion networks that hold every order statistic the percentile clip
// needs (positions ilo, ilo+1, ihi, ihi+1 of 128); 0 means a full sort.
__host__ __device__ inline int select_width(const AppendParams& p) {
  constexpr int kHeadDim = 128;
  if (p.quant_k != 0 && p.quant_v != 0) return 3;
  auto reach = [](int r) { return r < kHeadDim / 2 ? r + 1 : kHeadDim - r; };
  const int rs[4] = {p.ilo, p.ilo + 1 < kHeadDim ? p.ilo + 1 : kHeadDim - 1, p.ihi,
                     p.ihi + 1 < kHeadDim ? p.ihi + 1 : kHeadDim - 1};
  int need = 0;
  for (int r : rs) need = reach(r) > need ? reach(r) : need;
  return need <= 3 ? 3 : (need <= 8 ? 8 : 0);
}


struct DecodeParams {
  const uint8_t* kpool;
  const uint8_t* vpool;
  const void* q;
  const float* tinv;      // [Hkv][128][128] or null
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* out;             // [B][Hq][128]
  float* ws_o;            // [B][Hq][chunks][128]
  float* ws_ml;           // [B][Hq][chunks][2]
  int batch, heads_q, heads_kv, group;
  int gpad;               // query heads per KV head rounded up to 4, 8 or 16
  int max_pages;          // row stride of block_table
  int64_t num_pages;      // pages in each pool (page ids outside are skipped)
  int pages_per_wave;
  int chunks;             // workgroups per (sequence, KV head)
  float score_scale;      // sm_scale * log2(e)
};

struct DequantParams {
  const uint8_t* pool;
  const int64_t* slots;
  float* out;
  int64_t n;
  int64_t num_pages;
  int heads;
  int bits;
  int which;
};

// Kernel launchers; return hipSuccess or the launch error.
hipError_t launch_append(const AppendParams& p, int in_dtype, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int bits_k, int bits_v, int q_dtype,
                         hipStream_t stream);
hipError_t launch_dequant(const DequantParams& p, hipStream_t stream);

// Split of a decode launch, a function of the shapes only.
struct DecodeSplit {
  int pages_per_wave;
  int chunks;
};
DecodeSplit decode_split(int batch, int heads_kv, int max_seq_len);
int decode_group_pad(int group);

}  // namespace kvq
