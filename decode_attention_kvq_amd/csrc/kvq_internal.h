// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Full-precision cache windows: positions [0, sink) and the newest positions of a sequence
// stay in full precision; a position from `sink` on is eligible once `keep` newer ones
// exist, and eligible positions are quantized in batches of `flush`, oldest first, as soon
// as `flush` of them wait.  The paged cache holds quantized position p at index p - sink.
// The full-precision positions live in a window row of sink + keep + flush slots: the sink
// at slots [0, sink), every later position p in the ring slot sink + (p - sink) % (keep + flush).
struct WindowShape {
  int sink, keep, flush;   // flush == 0: no window
};

// Quantized positions of a sequence of `len` positions once every waiting batch has been
// quantized (positions sink .. sink + result - 1).
__host__ __device__ inline int window_quantized(int len, const WindowShape& w) {
  const int e = len - w.sink - w.keep;
  return e >= w.flush ? e / w.flush * w.flush : 0;
}
__host__ __device__ inline int window_slot(int pos, const WindowShape& w) {
  return pos < w.sink ? pos : w.sink + (pos - w.sink) % (w.keep + w.flush);
}
__host__ __device__ inline int window_width(const WindowShape& w) { return w.sink + w.keep + w.flush; }

// Where the append kernels find a token's cache slot and source row.
enum SlotMode {
  kSlotsGiven = 0,      // slot = slots[i], source row i of k / v
  kSlotsPrefill = 1,    // windowed prefill: token i is position i - cu_seqlens[b] of sequence b
                        // (source row i); middle positions go to index position - sink
  kSlotsFlush = 2,      // window flush of a decode step: token i is batch entry i % flush of
                        // sequence i / flush; source rows are window slots (k / v = the windows)
};

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
  // slot modes other than kSlotsGiven
  int slot_mode;
  WindowShape win;
  const int32_t* cu_seqlens;   // [batch + 1] (prefill)
  const int32_t* seq_lens;     // [batch] (flush: lengths after the step)
  const int32_t* block_table;  // [batch][max_pages]
  const int32_t* win_rows;     // [batch] window row of each sequence, or null (row b)
  int batch, max_pages, num_rows;
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
  // full-precision windows (win.flush == 0: none): the cache holds the quantized middle
  // positions only, window_quantized(seq_len - win_pending) of them; the partial results
  // always go to the workspace, and the window kernel merges them
  WindowShape win;
  int win_pending;
  // a decode step's new tokens, [B][Hkv][128] of the query's type (null: none): position
  // seq_len - 1 of each non-empty sequence takes part from these rows at full precision, and
  // the cache supplies positions [0, seq_len - 1)
  const void* knew;
  const void* vnew;
  // a decode step: append_blocks = 1 adds batch z-blocks to the grid, and block
  // (0, h, batch + i) appends token i of `app` for KV head h (blocks (c > 0, h, batch + i)
  // of a split decode do nothing); this launch never reads what they write: the new tokens
  // take part from knew / vnew
  int append_blocks;
  AppendParams app;
};

// The window half of a windowed decode: attention over the full-precision positions, the
// merge with the quantized partials, and (decode step) the store of the new token.
struct WindowParams {
  void* kwin;             // [rows][sink + keep + flush][Hkv][128] of the query dtype
  void* vwin;
  const int32_t* win_rows;
  int rows;
  const void* k_new;      // [B][Hkv][128] or null: the step's new token (position seq_len - 1)
  const void* v_new;
};

// Prefill of the windows: copies the full-precision positions of each sequence from the
// packed prompt rows into its window row.
struct WindowStoreParams {
  const void* k;
  const void* v;
  void* kwin;
  void* vwin;
  const int32_t* cu_seqlens;
  const int32_t* win_rows;
  int64_t n;              // packed prompt rows
  int rows, batch, heads;
  WindowShape win;
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
hipError_t launch_window(const DecodeParams& p, const WindowParams& w, int q_dtype, hipStream_t stream);
hipError_t launch_window_store(const WindowStoreParams& p, int dtype, hipStream_t stream);

constexpr int kSmallAppendMaxTokens = 512;    // batches of up to this many tokens take the small path

// Split of a decode launch, a function of the shapes only.
struct DecodeSplit {
  int pages_per_wave;
  int chunks;
};
DecodeSplit decode_split(int batch, int heads_kv, int max_seq_len);
int decode_group_pad(int group);

// The allocation-free decode's partial outputs: a file-scope device array of this many bytes
// on every GPU the library runs on.  decode_scratch returns its address on the current
// device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace kvq
