// C ABI of the kvq library: host-side validation, then kernel dispatch on the caller's
// stream.  Nothing here allocates or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <string>

#include "../../include/kvq.h"
#include "kvq_internal.h"

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status s, const char* msg) {
  g_last_error = msg;
  return s;
}

kvq_status check_cache(const kvq_cache_desc* c, bool need_k, bool need_v) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache descriptor is null");
  if (c->head_dim != 128) return fail(KVQ_ERR_UNSUPPORTED, "head_dim must be 128");
  if (c->page_size != 64) return fail(KVQ_ERR_UNSUPPORTED, "page_size must be 64");
  if (c->num_kv_heads < 1) return fail(KVQ_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (c->num_kv_heads > 65535) return fail(KVQ_ERR_UNSUPPORTED, "num_kv_heads must be <= 65535");
  if (c->bits_k < 2 || c->bits_k > 4 || c->bits_v < 2 || c->bits_v > 4)
    return fail(KVQ_ERR_UNSUPPORTED, "bits_k and bits_v must be 2, 3 or 4");
  if (c->num_pages < 0) return fail(KVQ_ERR_INVALID_ARG, "num_pages must be >= 0");
  if (need_k && !c->k_pages) return fail(KVQ_ERR_INVALID_ARG, "k_pages is null");
  if (need_v && !c->v_pages) return fail(KVQ_ERR_INVALID_ARG, "v_pages is null");
  return KVQ_OK;
}

kvq_status check_quantizer(int q, float alpha, float p_lo, float p_hi) {
  if (q == KVQ_Q_PERCENTILE) {
    if (!(std::isfinite(p_lo) && std::isfinite(p_hi) && p_lo >= 0.0f && p_lo <= p_hi && p_hi <= 1.0f))
      return fail(KVQ_ERR_INVALID_ARG, "percentiles must satisfy 0 <= p_lo <= p_hi <= 1");
    return KVQ_OK;
  }
  if (q == KVQ_Q_RMS) {
    if (!(std::isfinite(alpha) && alpha > 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "alpha must be > 0");
    return KVQ_OK;
  }
  return fail(KVQ_ERR_INVALID_ARG, "unknown quantizer");
}

// Linear-interpolation percentile position over 128 sorted values.
void percentile_position(float p, int* i, float* f) {
  const double rank = (double)p * 127.0;
  int ii = (int)std::floor(rank);
  if (ii < 0) ii = 0;
  float ff = (float)(rank - (double)ii);
  if (ii >= 127) { ii = 127; ff = 0.0f; }
  *i = ii;
  *f = ff;
}

bool valid_dtype(int d) { return d == KVQ_F32 || d == KVQ_BF16 || d == KVQ_F16; }

kvq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KVQ_OK;
  g_last_error = std::string("HIP error: ") + hipGetErrorString(e);
  return KVQ_ERR_HIP;
}

// Workspace: only when sequences are split over several workgroups, the partial outputs
// and their (max, sum) pairs.
struct WorkspaceLayout {
  size_t o_bytes, ml_bytes, total;
};

WorkspaceLayout workspace_layout(int batch, int heads_q, int chunks, bool always = false) {
  WorkspaceLayout w{0, 0, 0};
  if (batch <= 0 || chunks < 1 || (chunks == 1 && !always)) return w;
  const size_t rows = (size_t)batch * heads_q * chunks;
  w.o_bytes = (rows * 128 * sizeof(float) + 255) & ~(size_t)255;
  w.ml_bytes = (rows * 2 * sizeof(float) + 255) & ~(size_t)255;
  w.total = w.o_bytes + w.ml_bytes;
  return w;
}

kvq::AppendParams append_params(const kvq_cache_desc* cache, const void* k, const void* v, const int64_t* slots,
                                int64_t n_tokens, const void* t_k) {
  kvq::AppendParams p{};
  p.k = k; p.v = v; p.slots = slots; p.t = t_k;
  p.kpool = static_cast<uint8_t*>(cache->k_pages);
  p.vpool = static_cast<uint8_t*>(cache->v_pages);
  p.n = n_tokens; p.num_pages = cache->num_pages; p.heads = cache->num_kv_heads;
  p.bits_k = cache->bits_k; p.bits_v = cache->bits_v;
  p.quant_k = cache->quant_k; p.quant_v = cache->quant_v;
  percentile_position(cache->p_lo, &p.ilo, &p.flo);
  percentile_position(cache->p_hi, &p.ihi, &p.fhi);
  p.alpha_k = cache->alpha_k; p.alpha_v = cache->alpha_v;
  return p;
}

// Longest quantized run the decode split is sized for (windows: the sink is never quantized).
int split_length(int max_seq_len, const kvq::WindowShape* win) {
  return win ? (max_seq_len > win->sink ? max_seq_len - win->sink : 0) : max_seq_len;
}

// Checks and fills the decode launch; shared by the plain and windowed decodes.  With
// windows (win non-null) the partial results always go to the workspace.
kvq_status decode_params(const kvq_cache_desc* cache, const void* q, kvq_dtype q_dtype, int32_t batch,
                         int32_t num_q_heads, const float* t_k_inv_t, const int32_t* block_table,
                         int32_t max_pages, const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                         float* out, void* workspace, size_t workspace_bytes, kvq::DecodeParams* pp,
                         const kvq::WindowShape* win = nullptr) {
  if (batch < 0) return fail(KVQ_ERR_INVALID_ARG, "batch must be >= 0");
  kvq_status s = check_cache(cache, batch > 0, batch > 0);
  if (s != KVQ_OK) return s;
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads != 0)
    return fail(KVQ_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  const int group = num_q_heads / cache->num_kv_heads;
  if (group > 16) return fail(KVQ_ERR_UNSUPPORTED, "at most 16 query heads per KV head");
  if (!valid_dtype(q_dtype)) return fail(KVQ_ERR_INVALID_ARG, "unknown query dtype");
  if (max_seq_len < 0 || max_pages < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len and max_pages must be >= 0");
  if ((int64_t)max_pages * 64 < (int64_t)split_length(max_seq_len, win))
    return fail(KVQ_ERR_INVALID_ARG, win ? "max_pages*64 must cover max_seq_len - sink"
                                         : "max_pages*64 must cover max_seq_len");
  if (!std::isfinite(sm_scale)) return fail(KVQ_ERR_INVALID_ARG, "sm_scale must be finite");
  if (batch == 0) return KVQ_OK;
  if (batch > 65535) return fail(KVQ_ERR_UNSUPPORTED, "batch must be <= 65535");
  if (!q || !block_table || !seq_lens || !out)
    return fail(KVQ_ERR_INVALID_ARG, "q, block_table, seq_lens and out must be non-null");
  const kvq::DecodeSplit sp = kvq::decode_split(batch, cache->num_kv_heads, split_length(max_seq_len, win));
  const WorkspaceLayout wl = workspace_layout(batch, num_q_heads, sp.chunks, win != nullptr);
  if (wl.total > 0 && (!workspace || workspace_bytes < wl.total))
    return fail(KVQ_ERR_WORKSPACE, win ? "workspace smaller than kvq_window_workspace_bytes()"
                                       : "workspace smaller than kvq_decode_workspace_bytes()");
  if (cache->num_pages < 1) return fail(KVQ_ERR_INVALID_ARG, "num_pages must be >= 1");
  kvq::DecodeParams& p = *pp;
  p = kvq::DecodeParams{};
  p.kpool = static_cast<const uint8_t*>(cache->k_pages);
  p.vpool = static_cast<const uint8_t*>(cache->v_pages);
  p.q = q; p.tinv = t_k_inv_t; p.block_table = block_table; p.seq_lens = seq_lens; p.out = out;
  char* ws = static_cast<char*>(workspace);
  p.ws_o = wl.o_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  p.ws_ml = wl.ml_bytes ? reinterpret_cast<float*>(ws + wl.o_bytes) : nullptr;
  p.batch = batch; p.heads_q = num_q_heads; p.heads_kv = cache->num_kv_heads; p.group = group;
  p.gpad = kvq::decode_group_pad(group);
  p.max_pages = max_pages; p.num_pages = cache->num_pages; p.pages_per_wave = sp.pages_per_wave; p.chunks = sp.chunks;
  p.score_scale = sm_scale * 1.4426950408889634f;
  if (win) p.win = *win;
  return KVQ_OK;
}

size_t elem_bytes(kvq_dtype d) { return d == KVQ_F32 ? 4 : 2; }

// Checks a window descriptor; fills the shape.
kvq_status check_window(const kvq_cache_desc* cache, const kvq_window_desc* w, bool need_data,
                        kvq::WindowShape* shape) {
  if (!w) return fail(KVQ_ERR_INVALID_ARG, "window descriptor is null");
  if (w->sink < 0 || w->keep < 0 || w->flush < 1)
    return fail(KVQ_ERR_INVALID_ARG, "window sizes must satisfy sink >= 0, keep >= 0, flush >= 1");
  if ((int64_t)w->sink + w->keep + w->flush > KVQ_WINDOW_MAX_SLOTS)
    return fail(KVQ_ERR_UNSUPPORTED, "sink + keep + flush exceeds KVQ_WINDOW_MAX_SLOTS");
  // the window kernel addresses a row's elements with 32-bit offsets
  if (cache && ((int64_t)w->sink + w->keep + w->flush) * cache->num_kv_heads * 128 > 0xFFFFFFFFLL)
    return fail(KVQ_ERR_UNSUPPORTED, "(sink + keep + flush) * num_kv_heads * 128 must be < 2^32");
  if (!valid_dtype(w->dtype)) return fail(KVQ_ERR_INVALID_ARG, "unknown window dtype");
  if (w->num_rows < 0) return fail(KVQ_ERR_INVALID_ARG, "num_rows must be >= 0");
  if (need_data && (w->num_rows < 1 || !w->k_win || !w->v_win))
    return fail(KVQ_ERR_INVALID_ARG, "window tensors must be non-null with num_rows >= 1");
  *shape = kvq::WindowShape{w->sink, w->keep, w->flush};
  return KVQ_OK;
}

}  // namespace

extern "C" {

size_t kvq_block_bytes(int32_t bits) {
  if (bits < 2 || bits > 4) return 0;
  return (size_t)(64 * 128 * bits / 8 + 4 * 64);
}

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

kvq_status kvq_quantize_append(const kvq_cache_desc* cache, const void* k, const void* v,
                               kvq_dtype in_dtype, int64_t n_tokens, const int64_t* slot_mapping,
                               const void* t_k, kvq_dtype t_dtype, void* stream) {
  g_last_error.clear();
  if (n_tokens < 0) return fail(KVQ_ERR_INVALID_ARG, "n_tokens must be >= 0");
  kvq_status s = check_cache(cache, n_tokens > 0, n_tokens > 0);
  if (s != KVQ_OK) return s;
  if ((s = check_quantizer(cache->quant_k, cache->alpha_k, cache->p_lo, cache->p_hi)) != KVQ_OK) return s;
  if ((s = check_quantizer(cache->quant_v, cache->alpha_v, cache->p_lo, cache->p_hi)) != KVQ_OK) return s;
  if (!valid_dtype(in_dtype)) return fail(KVQ_ERR_INVALID_ARG, "unknown input dtype");
  if (t_k && t_dtype != in_dtype) return fail(KVQ_ERR_UNSUPPORTED, "t_dtype must equal in_dtype");
  if (n_tokens == 0) return KVQ_OK;
  if (!k || !v || !slot_mapping) return fail(KVQ_ERR_INVALID_ARG, "k, v and slot_mapping must be non-null");
  if ((n_tokens + 127) / 128 > 0x7FFFFFFFLL) return fail(KVQ_ERR_UNSUPPORTED, "too many tokens");
  const kvq::AppendParams p = append_params(cache, k, v, slot_mapping, n_tokens, t_k);
  return hip_status(kvq::launch_append(p, (int)in_dtype, static_cast<hipStream_t>(stream)));
}

size_t kvq_decode_workspace_bytes(const kvq_cache_desc* cache, int32_t batch, int32_t num_q_heads,
                                  int32_t max_seq_len) {
  if (!cache || cache->num_kv_heads < 1 || batch <= 0 || num_q_heads < 1 || max_seq_len < 0) return 0;
  const kvq::DecodeSplit sp = kvq::decode_split(batch, cache->num_kv_heads, max_seq_len);
  return workspace_layout(batch, num_q_heads, sp.chunks).total;
}

size_t kvq_decode_step_workspace_bytes(const kvq_cache_desc* cache, int32_t batch, int32_t num_q_heads,
                                       int32_t max_seq_len) {
  return kvq_decode_workspace_bytes(cache, batch, num_q_heads, max_seq_len);
}

kvq_status kvq_decode_attn(const kvq_cache_desc* cache, const void* q, kvq_dtype q_dtype, int32_t batch,
                           int32_t num_q_heads, const float* t_k_inv_t, const int32_t* block_table,
                           int32_t max_pages, const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                           float* out, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  kvq::DecodeParams p;
  kvq_status s = decode_params(cache, q, q_dtype, batch, num_q_heads, t_k_inv_t, block_table, max_pages, seq_lens,
                               max_seq_len, sm_scale, out, workspace, workspace_bytes, &p);
  if (s != KVQ_OK || batch == 0) return s;
  return hip_status(kvq::launch_decode(p, cache->bits_k, cache->bits_v, (int)q_dtype,
                                       static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_attn_noalloc(const kvq_cache_desc* cache, const void* q, kvq_dtype q_dtype,
                                   int32_t batch, int32_t num_q_heads, const float* t_k_inv_t,
                                   const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                                   int32_t max_seq_len, float sm_scale, float* out, void* stream) {
  g_last_error.clear();
  const size_t need = kvq_decode_workspace_bytes(cache, batch, num_q_heads, max_seq_len);
  if (need > kvq::kNoAllocScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof msg, "these sizes need %zu bytes of partial outputs; the allocation-free "
                  "decode holds %zu (KVQ_NOALLOC_SCRATCH_BYTES)", need, kvq::kNoAllocScratchBytes);
    return fail(KVQ_ERR_WORKSPACE, msg);
  }
  void* scratch = nullptr;
  if (need > 0) {
    // the scratch address is the current device's: the stream must belong to it
    int cur = 0;
    kvq_status s = hip_status(hipGetDevice(&cur));
    if (s != KVQ_OK) return s;
    if (stream) {
      hipDevice_t sd = 0;
      if ((s = hip_status(hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd))) != KVQ_OK) return s;
      if (sd != cur) return fail(KVQ_ERR_INVALID_ARG, "stream belongs to another device than the current one");
    }
    if ((s = hip_status(kvq::decode_scratch(&scratch))) != KVQ_OK) return s;
  }
  kvq::DecodeParams p;
  kvq_status s = decode_params(cache, q, q_dtype, batch, num_q_heads, t_k_inv_t, block_table, max_pages, seq_lens,
                               max_seq_len, sm_scale, out, scratch, scratch ? kvq::kNoAllocScratchBytes : 0, &p);
  if (s != KVQ_OK || batch == 0) return s;
  return hip_status(kvq::launch_decode(p, cache->bits_k, cache->bits_v, (int)q_dtype,
                                       static_cast<hipStream_t>(stream)));
}

kvq_status kvq_decode_step(const kvq_cache_desc* cache, const void* q, const void* k_new, const void* v_new,
                           kvq_dtype dtype, int32_t batch, int32_t num_q_heads, const int64_t* new_slots,
                           const void* t_k, kvq_dtype t_dtype, const float* t_k_inv_t,
                           const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                           int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  kvq::DecodeParams p;
  kvq_status s = decode_params(cache, q, dtype, batch, num_q_heads, t_k_inv_t, block_table, max_pages, seq_lens,
                               max_seq_len, sm_scale, out, workspace, workspace_bytes, &p);
  if (s != KVQ_OK) return s;
  if ((s = check_quantizer(cache->quant_k, cache->alpha_k, cache->p_lo, cache->p_hi)) != KVQ_OK) return s;
  if ((s = check_quantizer(cache->quant_v, cache->alpha_v, cache->p_lo, cache->p_hi)) != KVQ_OK) return s;
  if (t_k && t_dtype != dtype) return fail(KVQ_ERR_UNSUPPORTED, "t_dtype must equal dtype");
  if (batch == 0) return KVQ_OK;
  if (!k_new || !v_new || !new_slots) return fail(KVQ_ERR_INVALID_ARG, "k_new, v_new and new_slots must be non-null");
  // The new token of each sequence takes part in the attention from k_new / v_new at full
  // precision (the decode reads positions [0, seq_len - 1) from the cache), and its codes
  // are written for later steps by an append that the decode does not wait for: the decode
  // masks position seq_len - 1 out of the last page it loads.  The append runs in the
  // decode's own launch, in blocks after the decode's: dispatched last, they take the slots
  // that the first decode workgroups leave while the last ones still walk their pages.  (A
  // batch too large for the grid appends in a launch of its own first.)
  const kvq::AppendParams a = append_params(cache, k_new, v_new, new_slots, batch, t_k);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  p.knew = k_new;
  p.vnew = v_new;
  if (batch <= 32767) {
    p.app = a;
    p.append_blocks = 1;
  } else if ((s = hip_status(kvq::launch_append(a, (int)dtype, st))) != KVQ_OK) {
    return s;
  }
  return hip_status(kvq::launch_decode(p, cache->bits_k, cache->bits_v, (int)dtype, st));
}

kvq_status kvq_dequant(const kvq_cache_desc* cache, int32_t which, const int64_t* slots, int64_t n_tokens,
                       float* out, void* stream) {
  g_last_error.clear();
  if (which != 0 && which != 1) return fail(KVQ_ERR_INVALID_ARG, "which must be 0 (keys) or 1 (values)");
  if (n_tokens < 0) return fail(KVQ_ERR_INVALID_ARG, "n_tokens must be >= 0");
  kvq_status s = check_cache(cache, n_tokens > 0 && which == 0, n_tokens > 0 && which == 1);
  if (s != KVQ_OK) return s;
  if (n_tokens == 0) return KVQ_OK;
  if (!slots || !out) return fail(KVQ_ERR_INVALID_ARG, "slots and out must be non-null");
  if ((n_tokens * cache->num_kv_heads * 32 + 255) / 256 > 0x7FFFFFFFLL)
    return fail(KVQ_ERR_UNSUPPORTED, "too many tokens");
  kvq::DequantParams p{};
  p.pool = static_cast<const uint8_t*>(which == 0 ? cache->k_pages : cache->v_pages);
  p.slots = slots; p.out = out; p.n = n_tokens; p.num_pages = cache->num_pages;
  p.heads = cache->num_kv_heads;
  p.bits = which == 0 ? cache->bits_k : cache->bits_v;
  p.which = which;
  return hip_status(kvq::launch_dequant(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" {

size_t kvq_window_bytes(const kvq_cache_desc* cache, const kvq_window_desc* win) {
  if (!cache || !win || cache->num_kv_heads < 1 || win->num_rows < 0 || win->sink < 0 || win->keep < 0 ||
      win->flush < 1 || !valid_dtype(win->dtype))
    return 0;
  return (size_t)win->num_rows * (size_t)(win->sink + win->keep + win->flush) * (size_t)cache->num_kv_heads * 128 *
         elem_bytes(win->dtype);
}

kvq_status kvq_window_prefill(const kvq_cache_desc* cache, const kvq_window_desc* win, const void* k, const void* v,
                              int32_t batch, const int32_t* cu_seqlens, int64_t n_tokens,
                              const int32_t* block_table, int32_t max_pages, const int32_t* win_rows,
                              const void* t_k, void* stream) {
  g_last_error.clear();
  if (batch < 0 || n_tokens < 0 || max_pages < 0)
    return fail(KVQ_ERR_INVALID_ARG, "batch, n_tokens and max_pages must be >= 0");
  kvq::WindowShape shape;
  kvq_status s = check_window(cache, win, batch > 0 && n_tokens > 0, &shape);
  if (s != KVQ_OK) return s;
  if ((s = check_cache(cache, n_tokens > 0, n_tokens > 0)) != KVQ_OK) return s;
  if ((s = check_quantizer(cache->quant_k, cache->alpha_k, cache->p_lo, cache->p_hi)) != KVQ_OK) return s;
  if ((s = check_quantizer(cache->quant_v, cache->alpha_v, cache->p_lo, cache->p_hi)) != KVQ_OK) return s;
  if (batch == 0 || n_tokens == 0) return KVQ_OK;
  if (batch > 65535) return fail(KVQ_ERR_UNSUPPORTED, "batch must be <= 65535");
  if (n_tokens > 0x7FFFFFFFLL) return fail(KVQ_ERR_UNSUPPORTED, "n_tokens must fit in int32");
  if (!k || !v || !cu_seqlens || !block_table)
    return fail(KVQ_ERR_INVALID_ARG, "k, v, cu_seqlens and block_table must be non-null");
  if (max_pages < 1) return fail(KVQ_ERR_INVALID_ARG, "max_pages must be >= 1");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  kvq::WindowStoreParams ws{};
  ws.k = k; ws.v = v; ws.kwin = win->k_win; ws.vwin = win->v_win; ws.cu_seqlens = cu_seqlens;
  ws.win_rows = win_rows; ws.n = n_tokens; ws.rows = win->num_rows; ws.batch = batch;
  ws.heads = cache->num_kv_heads; ws.win = shape;
  if ((s = hip_status(kvq::launch_window_store(ws, (int)win->dtype, st))) != KVQ_OK) return s;
  kvq::AppendParams a = append_params(cache, k, v, nullptr, n_tokens, t_k);
  a.slot_mode = kvq::kSlotsPrefill;
  a.win = shape; a.cu_seqlens = cu_seqlens; a.block_table = block_table; a.win_rows = win_rows;
  a.batch = batch; a.max_pages = max_pages; a.num_rows = win->num_rows;
  return hip_status(kvq::launch_append(a, (int)win->dtype, st));
}

size_t kvq_window_workspace_bytes(const kvq_cache_desc* cache, const kvq_window_desc* win, int32_t batch,
                                  int32_t num_q_heads, int32_t max_seq_len) {
  if (!cache || !win || cache->num_kv_heads < 1 || batch <= 0 || num_q_heads < 1 || max_seq_len < 0 ||
      win->sink < 0)
    return 0;
  const kvq::WindowShape shape{win->sink, win->keep, win->flush};
  const kvq::DecodeSplit sp = kvq::decode_split(batch, cache->num_kv_heads, split_length(max_seq_len, &shape));
  return workspace_layout(batch, num_q_heads, sp.chunks, true).total;
}

kvq_status kvq_window_decode_attn(const kvq_cache_desc* cache, const kvq_window_desc* win, const void* q,
                                  int32_t batch, int32_t num_q_heads, const float* t_k_inv_t,
                                  const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                                  const int32_t* win_rows, int32_t max_seq_len, float sm_scale, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  kvq::WindowShape shape;
  kvq_status s = check_window(cache, win, batch > 0, &shape);
  if (s != KVQ_OK) return s;
  kvq::DecodeParams p;
  s = decode_params(cache, q, win->dtype, batch, num_q_heads, t_k_inv_t, block_table, max_pages, seq_lens,
                    max_seq_len, sm_scale, out, workspace, workspace_bytes, &p, &shape);
  if (s != KVQ_OK || batch == 0) return s;
  p.win_pending = 0;
  kvq::WindowParams w{win->k_win, win->v_win, win_rows, win->num_rows, nullptr, nullptr};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = hip_status(kvq::launch_decode(p, cache->bits_k, cache->bits_v, (int)win->dtype, st))) != KVQ_OK) return s;
  return hip_status(kvq::launch_window(p, w, (int)win->dtype, st));
}

kvq_status kvq_window_decode_step(const kvq_cache_desc* cache, const kvq_window_desc* win, const void* q,
                                  const void* k_new, const void* v_new, int32_t batch, int32_t num_q_heads,
                                  const void* t_k, const float* t_k_inv_t, const int32_t* block_table,
                                  int32_t max_pages, const int32_t* seq_lens, const int32_t* win_rows,
                                  int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  kvq::WindowShape shape;
  kvq_status s = check_window(cache, win, batch > 0, &shape);
  if (s != KVQ_OK) return s;
  kvq::DecodeParams p;
  s = decode_params(cache, q, win->dtype, batch, num_q_heads, t_k_inv_t, block_table, max_pages, seq_lens,
                    max_seq_len, sm_scale, out, workspace, workspace_bytes, &p, &shape);
  if (s != KVQ_OK) return s;
  if ((s = check_quantizer(cache->quant_k, cache->alpha_k, cache->p_lo, cache->p_hi)) != KVQ_OK) return s;
  if ((s = check_quantizer(cache->quant_v, cache->alpha_v, cache->p_lo, cache->p_hi)) != KVQ_OK) return s;
  if (batch == 0) return KVQ_OK;
  if (!k_new || !v_new) return fail(KVQ_ERR_INVALID_ARG, "k_new and v_new must be non-null");
  if ((int64_t)batch * shape.flush > 0x7FFFFFFFLL) return fail(KVQ_ERR_UNSUPPORTED, "batch * flush too large");
  // stream order: the quantized partials, the window (which stores the new position and
  // merges), then the batches the new positions made eligible are quantized
  p.win_pending = 1;
  kvq::WindowParams w{win->k_win, win->v_win, win_rows, win->num_rows, k_new, v_new};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = hip_status(kvq::launch_decode(p, cache->bits_k, cache->bits_v, (int)win->dtype, st))) != KVQ_OK) return s;
  if ((s = hip_status(kvq::launch_window(p, w, (int)win->dtype, st))) != KVQ_OK) return s;
  kvq::AppendParams a = append_params(cache, win->k_win, win->v_win, nullptr, (int64_t)batch * shape.flush, t_k);
  a.slot_mode = kvq::kSlotsFlush;
  a.win = shape; a.seq_lens = seq_lens; a.block_table = block_table; a.win_rows = win_rows;
  a.batch = batch; a.max_pages = max_pages; a.num_rows = win->num_rows;
  return hip_status(kvq::launch_append(a, (int)win->dtype, st));
}

}  // extern "C"
