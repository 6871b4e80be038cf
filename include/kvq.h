/*
 * kvq.h -- C ABI of the quantized KV-cache library for AMD Instinct MI355X (gfx950).
 *
 * Two operations, as the method's pages state the problem:
 *   write path  -- "WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms",
 *                  §4.2 (dense per-KV-head key transform applied after RoPE; the value
 *                  transform is folded into W_V/W_O offline, so values arrive already
 *                  transformed), §4.3 (QuEST: one group = one token's d channels,
 *                  RMS-based clip) and §5.3 (OSCAR-style percentile-clipped affine
 *                  codes); "Spend Bits Where Queries Look" (NOVA-KV project page),
 *                  "Three requirements" (paged cache, same number of bits per token)
 *                  and its online-inference figure (encode once when written).
 *   read path   -- same pages: query-side compensation q' = q T^-T (§4.2), decode
 *                  inside attention on every step (NOVA-KV "Three requirements": read
 *                  cost is paid over the whole cache each step), grouped-query
 *                  attention (§4.1); the output stays in the transformed value basis
 *                  that W_O absorbs (§4.2).
 *
 * Conventions for every entry point
 *   - Pointers marked "device" are HIP device memory owned by the caller; the library
 *     never allocates, frees or keeps them.  "stream" is a hipStream_t (NULL = the
 *     default stream).  Work is enqueued asynchronously; the call returns when it is
 *     enqueued.  Device-side faults surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; a non-OK status
 *     means nothing was enqueued.  kvq_last_error() then returns a message for the
 *     calling thread.
 *   - Shapes are fixed by the layout: head_dim 128, page_size 64 tokens, 2-, 3- or 4-bit
 *     codes.  Other values return KVQ_ERR_UNSUPPORTED.
 *   - Floating-point inputs must be finite.
 *
 * Page layout (the ABI of k_pages / v_pages).  A pool is [num_pages][num_kv_heads]
 * blocks of kvq_block_bytes(bits) bytes; the block of (page p, KV head h) starts at
 * pool + (p*num_kv_heads + h)*kvq_block_bytes(bits).  Token slot s lives in page
 * s/64 at offset o = s%64.  A block holds, in order:
 *   codes   64*128*bits/8 bytes of little-endian 32-bit words, R = 32/bits codes a word
 *           keys:   word o*(128/R) + c/R,  bits (c%R)*bits   (token-major rows)
 *           values: word (o/R)*128 + c,    bits (o%R)*bits   (a word holds R
 *                   consecutive tokens of one channel c)
 *   scales  64 fp16 (token o at byte 2*o of this section)
 *   zeros   64 fp16 (token o at byte 2*o of this section)
 * 3-bit codes ("WUSH-KV" §5.1 evaluates 2, 3 and 4 bits) are two bit planes in the
 * 3072-byte code section: bytes 0..2047 hold bits 0-1 of every code laid out exactly as
 * a 2-bit code section; bytes 2048..3071 (words 512..767) hold bit 2:
 *           keys:   word 512 + o*4 + c/32, channel offset u = c%32 at bit
 *                   4*((u%16)/2) + 2*(u/16) + u%2
 *           values: word 512 + (o/32)*128 + c, token offset t = o%32 at bit
 *                   t%8 + 16*((t/8)%2) + 8*(t/16)
 * A dequantized element is fma(code, scale, zero) in fp32.  2-bit blocks are 2304 bytes
 * (2.25 bits per element), 3-bit blocks 3328 bytes (3.25), 4-bit blocks 4352 bytes (4.25).
 *
 * Quantizer of one group x[0..127] (one token of one KV head):
 *   percentile: lo, hi = linear-interpolated order statistics at p_lo, p_hi
 *               (rank p*127 formed in double, weight f rounded to float,
 *               v = fmaf(f, s[i+1] - s[i], s[i]) + 0.0f over the sorted values s)
 *   rms:        lo = -alpha*r, hi = +alpha*r, r = sqrtf(sum(x^2)/128) with the fp32
 *               sum taken by one pairwise tree over the 128 channels (at stride 64,
 *               32, ..., 1, element c < stride adds element c + stride)
 *   then        s = (hi - lo)/L (L = 2^bits - 1), scale = fp16(s), zero = fp16(lo)
 *               (both saturated to +-65504, round to nearest even),
 *               r = scale == 0 ? 0 : 1/scale, code = clamp(rint((x - zero)*r), 0, L).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1,   /* null pointer, negative size, inconsistent shapes */
  KVQ_ERR_UNSUPPORTED = -2,   /* valid but not implemented: head_dim, bits, dtype pair */
  KVQ_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
  KVQ_ERR_HIP = -4            /* a HIP call failed while enqueueing */
} kvq_status;

typedef enum kvq_dtype { KVQ_F32 = 0, KVQ_BF16 = 1, KVQ_F16 = 2 } kvq_dtype;

typedef enum kvq_quantizer {
  KVQ_Q_PERCENTILE = 0,  /* OSCAR-style percentile-clipped affine (WUSH-KV §5.3) */
  KVQ_Q_RMS = 1          /* QuEST-style RMS-clipped symmetric levels (WUSH-KV §4.3) */
} kvq_quantizer;

/* Geometry and quantizer settings of one layer's paged cache. */
typedef struct kvq_cache_desc {
  int32_t num_kv_heads;   /* >= 1 */
  int32_t head_dim;       /* must be 128 */
  int32_t page_size;      /* must be 64 */
  int32_t bits_k;         /* 2, 3 or 4 */
  int32_t bits_v;         /* 2, 3 or 4 */
  int32_t quant_k;        /* kvq_quantizer for keys */
  int32_t quant_v;        /* kvq_quantizer for values */
  float p_lo, p_hi;       /* percentile quantizer: 0 <= p_lo <= p_hi <= 1 */
  float alpha_k, alpha_v; /* rms quantizer clip multipliers, > 0 */
  int64_t num_pages;      /* pages in each pool */
  void* k_pages;          /* device, [num_pages][num_kv_heads][kvq_block_bytes(bits_k)] */
  void* v_pages;          /* device, [num_pages][num_kv_heads][kvq_block_bytes(bits_v)] */
} kvq_cache_desc;

/* Bytes of one (page, KV head) block for 2-, 3- or 4-bit codes; 0 for other widths. */
size_t kvq_block_bytes(int32_t bits);

/* Write path: transform, clip, quantize and pack n_tokens new tokens.
 *   k, v          device, [n_tokens][num_kv_heads][128] of in_dtype; keys post-RoPE,
 *                 values already in the folded (transformed) basis.
 *   slot_mapping  device, [n_tokens] int64; slot of each token.  Slots must be
 *                 distinct; a slot < 0 or >= num_pages*64 is skipped (nothing written).
 *   t_k           device, [num_kv_heads][128][128] row-major, k' = k . T_K; or NULL for
 *                 the identity.  t_dtype must equal in_dtype.  Batches of up to 512
 *                 tokens transform with fp32 fused multiply-adds (four partial sums over
 *                 32 rows of T, added in order); larger bf16/f16 batches use the matrix
 *                 cores with fp32 accumulation, f32 batches fp32 arithmetic.
 * Bits of a block not belonging to the written tokens are preserved, so tokens may be
 * appended one at a time into partly filled pages. */
kvq_status kvq_quantize_append(const kvq_cache_desc* cache, const void* k, const void* v,
                               kvq_dtype in_dtype, int64_t n_tokens,
                               const int64_t* slot_mapping, const void* t_k,
                               kvq_dtype t_dtype, void* stream);

/* Workspace bytes kvq_decode_attn needs for these sizes.  Non-zero only when the sizes
 * make the launch split each sequence over several workgroups (few sequences, long
 * contexts): the workspace then holds the partial outputs that a merge step combines. */
size_t kvq_decode_workspace_bytes(const kvq_cache_desc* cache, int32_t batch,
                                  int32_t num_q_heads, int32_t max_seq_len);

/* Workspace bytes of kvq_decode_step: the step needs no more than its decode, so this equals
 * kvq_decode_workspace_bytes() (0 for invalid arguments). */
size_t kvq_decode_step_workspace_bytes(const kvq_cache_desc* cache, int32_t batch,
                                       int32_t num_q_heads, int32_t max_seq_len);

/* Read path: one decode step of grouped-query attention over the quantized cache.
 *   q            device, [batch][num_q_heads][128] of q_dtype (post-RoPE queries);
 *                num_q_heads must be a multiple of num_kv_heads, at most 16 query
 *                heads per KV head; query head g reads KV head g/(num_q_heads/num_kv_heads).
 *   t_k_inv_t    device, [num_kv_heads][128][128] fp32 row-major, q' = q . T_K^-T; NULL
 *                when keys were written without a transform.
 *   block_table  device, [batch][max_pages] int32 page ids; entries past a sequence's
 *                last page are not read; a page id outside [0, num_pages) contributes
 *                nothing (its tokens are skipped).
 *   seq_lens     device, [batch] int32, 0 <= seq_lens[b] <= max_seq_len <= 64*max_pages
 *                (max_seq_len sizes the split over workgroups: a seq_lens[b] above it is
 *                not fully read; reads never go past 64*max_pages positions).
 *   sm_scale     softmax scale (1/sqrt(128) for standard attention).
 *   out          device, [batch][num_q_heads][128] fp32, in the transformed value basis;
 *                an empty sequence gives zeros.
 *   workspace    device scratch of at least kvq_decode_workspace_bytes(...) bytes (may be
 *                NULL when that is 0); its content on entry does not matter.  Calls that
 *                share a workspace must be ordered (same stream). */
kvq_status kvq_decode_attn(const kvq_cache_desc* cache, const void* q, kvq_dtype q_dtype,
                           int32_t batch, int32_t num_q_heads, const float* t_k_inv_t,
                           const int32_t* block_table, int32_t max_pages,
                           const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                           float* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Allocation-free kvq_decode_attn, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.  Arguments
 * and results are those of kvq_decode_attn without the workspace.  The partial outputs of
 * sequences split over several workgroups go to a device array of KVQ_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on, until the process ends; the call makes
 * no allocation.  Sizes for which kvq_decode_workspace_bytes() exceeds it return
 * KVQ_ERR_WORKSPACE before anything is enqueued.  The call runs on the current device and
 * `stream` must belong to it (KVQ_ERR_INVALID_ARG otherwise).  Every call on one GPU shares
 * that GPU's array, which keeps the last call's contents (nothing needs clearing: every
 * partial is written before it is read): calls that can overlap on one GPU (streams with no
 * ordering between them) race, and must not be made. */
enum { KVQ_NOALLOC_SCRATCH_BYTES = 32 << 20 };
kvq_status kvq_decode_attn_noalloc(const kvq_cache_desc* cache, const void* q, kvq_dtype q_dtype,
                                   int32_t batch, int32_t num_q_heads, const float* t_k_inv_t,
                                   const int32_t* block_table, int32_t max_pages,
                                   const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                                   float* out, void* stream);

/* One decode step with the step's new tokens, in the order "WUSH-KV: KV Cache Quantization
 * with Data-Adaptive Transforms" §4.4 gives a new entry: it first takes part in attention
 * at full precision, and is quantized into the cache afterwards.  For every sequence b with
 * seq_lens[b] > 0, position seq_lens[b]-1 is the new token: sequence b is read as by
 * kvq_decode_attn over positions [0, seq_lens[b]-1) of the cache plus the new token's own
 * key and value (k_new, v_new, unquantized; its score is q . k_new, which equals
 * q' . k' under the key transform); and the new token's key and value (all KV heads) are
 * encoded exactly as kvq_quantize_append encodes them and written at new_slots[b], for
 * later steps.  The write path is [W] §4.2/§4.3, the read path §4.1/§4.2.  The decode does
 * not wait for the append (it gives position seq_lens[b]-1 of the cache no weight): the
 * append runs in the decode's own launch, in workgroups after the decode's (a batch above
 * 32767 appends in a launch of its own first).  All launches are on `stream`.
 *   q, k_new, v_new  device, [batch][num_q_heads][128] and [batch][num_kv_heads][128] of
 *                 dtype (post-RoPE query and key; the value in the folded basis).
 *   new_slots     device, [batch] int64: the slot of position seq_lens[b]-1 of sequence b
 *                 (page block_table[b][(seq_lens[b]-1)/64], offset (seq_lens[b]-1)%64);
 *                 < 0 or >= num_pages*64: nothing is written for that sequence (it still
 *                 attends to its new token).  The slot must not be one that any sequence
 *                 reads in this call (positions [0, seq_lens-1) of the block tables): the
 *                 append may run while the decode reads.
 *   t_k           as in kvq_quantize_append (t_dtype must equal dtype); t_k_inv_t,
 *                 block_table, seq_lens, max_seq_len, sm_scale, out as in kvq_decode_attn.
 *   workspace     device scratch, owned by the caller, of at least
 *                 kvq_decode_workspace_bytes() bytes (KVQ_ERR_WORKSPACE otherwise).
 * The written bytes equal those of kvq_quantize_append for the same new tokens. */
kvq_status kvq_decode_step(const kvq_cache_desc* cache, const void* q, const void* k_new,
                           const void* v_new, kvq_dtype dtype, int32_t batch,
                           int32_t num_q_heads, const int64_t* new_slots, const void* t_k,
                           kvq_dtype t_dtype, const float* t_k_inv_t,
                           const int32_t* block_table, int32_t max_pages,
                           const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                           float* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Dequantize cached tokens: which = 0 keys (transformed basis), 1 values.
 *   slots  device, [n_tokens] int64 (< 0 or >= num_pages*64: the output rows are left
 *          untouched)
 *   out    device, [n_tokens][num_kv_heads][128] fp32, fma(code, scale, zero). */
kvq_status kvq_dequant(const kvq_cache_desc* cache, int32_t which, const int64_t* slots,
                       int64_t n_tokens, float* out, void* stream);

/* ---------------------------------------------------------------------------------
 * Full-precision cache windows ("WUSH-KV: KV Cache Quantization with Data-Adaptive
 * Transforms" §4.4; §4.5 for their size).  The first `sink` positions and the newest
 * positions of a sequence stay in full precision.  A position p >= sink is eligible once
 * `keep` newer positions exist; eligible positions are quantized, oldest first, in batches
 * of `flush` as soon as `flush` of them wait.  Hence, once every waiting batch has been
 * quantized, a sequence of L positions has
 *     Q(L) = flush * floor((L - sink - keep) / flush)   (0 when L - sink - keep < flush)
 * quantized positions sink .. sink+Q-1, held in the paged cache at index p - sink
 * (page block_table[b][(p - sink)/64], offset (p - sink)%64); positions 0 .. sink-1 and
 * sink+Q .. L-1 are read in full precision.  A decode step reads its new position in full
 * precision and quantizes the batch it makes eligible after its attention.
 *
 * Window tensors (k_win, v_win): device, [num_rows][sink + keep + flush][num_kv_heads][128]
 * of `dtype`, caller-owned.  Sequence b uses row win_rows[b] (row b when win_rows is NULL;
 * a row outside [0, num_rows) gives it no full-precision positions and nothing is written
 * there).  The sequences of one call must use distinct rows (a decode step writes them).
 * Position p < sink is slot p; a later position p is slot sink + (p - sink) % (keep + flush).  Keys are stored as given (post-RoPE, before the key
 * transform), so their scores use the plain query; values in the folded basis as given.
 * Queries, new keys and values, prompts and T_K are all of `dtype`.
 * --------------------------------------------------------------------------------- */
/* Largest sink + keep + flush; also (sink + keep + flush) * num_kv_heads * 128 < 2^32 (the
 * elements of one row), else KVQ_ERR_UNSUPPORTED. */
enum { KVQ_WINDOW_MAX_SLOTS = 65535 };

typedef struct kvq_window_desc {
  int32_t sink;           /* S_sink >= 0 */
  int32_t keep;           /* S_keep >= 0 */
  int32_t flush;          /* S_flush >= 1 */
  int32_t num_rows;       /* window rows (sequences in flight) */
  kvq_dtype dtype;        /* element type of the windows and of every activation passed */
  void* k_win;            /* device, see above */
  void* v_win;
} kvq_window_desc;

/* Bytes of one window tensor (k_win or v_win); 0 for an invalid descriptor. */
size_t kvq_window_bytes(const kvq_cache_desc* cache, const kvq_window_desc* win);

/* Prefill of fresh prompts into a windowed cache: after the call, prompt b of length
 * L = cu_seqlens[b+1] - cu_seqlens[b] is in the state above with Q(L) quantized positions
 * (written exactly as kvq_quantize_append writes them, T_K applied) and its other
 * positions in window row win_rows[b].
 *   k, v          device, [n_tokens][num_kv_heads][128] of win->dtype, the prompts packed
 *                 back to back; cu_seqlens device [batch+1] int32 offsets (cu_seqlens[0] = 0,
 *                 non-decreasing, cu_seqlens[batch] <= n_tokens).
 *   block_table   device, [batch][max_pages] int32 (cache index j of sequence b in page
 *                 block_table[b][j/64]; an index past max_pages pages is not written).
 *   t_k           device, [num_kv_heads][128][128] of win->dtype, or NULL (identity).
 * Two kernels in stream order (window store, quantize-append). */
kvq_status kvq_window_prefill(const kvq_cache_desc* cache, const kvq_window_desc* win,
                              const void* k, const void* v, int32_t batch,
                              const int32_t* cu_seqlens, int64_t n_tokens,
                              const int32_t* block_table, int32_t max_pages,
                              const int32_t* win_rows, const void* t_k, void* stream);

/* Workspace bytes of kvq_window_decode_attn / kvq_window_decode_step for these sizes
 * (always non-zero for batch >= 1: the quantized partials are merged with the window). */
size_t kvq_window_workspace_bytes(const kvq_cache_desc* cache, const kvq_window_desc* win,
                                  int32_t batch, int32_t num_q_heads, int32_t max_seq_len);

/* Read path over a windowed cache: attention of q over all seq_lens[b] positions, Q(L)
 * quantized (read as by kvq_decode_attn, with q . T_K^-T) and the rest from the window
 * with q; one softmax over both.  Arguments as in kvq_decode_attn, q of win->dtype, except
 * that block_table covers the quantized positions only: max_pages*64 >= max_seq_len - sink.
 * The state read is the one after every waiting batch was quantized (after a prefill or a
 * decode step).  Two kernels: quantized partials, then window attention and merge. */
kvq_status kvq_window_decode_attn(const kvq_cache_desc* cache, const kvq_window_desc* win,
                                  const void* q, int32_t batch, int32_t num_q_heads,
                                  const float* t_k_inv_t, const int32_t* block_table,
                                  int32_t max_pages, const int32_t* seq_lens,
                                  const int32_t* win_rows, int32_t max_seq_len,
                                  float sm_scale, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* One decode step over a windowed cache.  seq_lens[b] = L counts the new position L-1,
 * whose key and value are k_new[b], v_new[b] ([batch][num_kv_heads][128] of win->dtype).
 * In stream order: attention over the state with Q(L-1) quantized positions and the new
 * position in full precision (the new key and value are stored in the window); then, if
 * Q(L) > Q(L-1), the batch of positions sink+Q(L-1) .. sink+Q(L)-1 is quantized from the
 * window into the paged cache (with t_k, as kvq_quantize_append).  Other arguments as in
 * kvq_window_decode_attn.  Kernels: quantized partials, window attention and merge (which
 * stores the new position), flush.  The flush covers batch*flush candidate positions;
 * workgroups whose positions have nothing to quantize return at once. */
kvq_status kvq_window_decode_step(const kvq_cache_desc* cache, const kvq_window_desc* win,
                                  const void* q, const void* k_new, const void* v_new,
                                  int32_t batch, int32_t num_q_heads, const void* t_k,
                                  const float* t_k_inv_t, const int32_t* block_table,
                                  int32_t max_pages, const int32_t* seq_lens,
                                  const int32_t* win_rows, int32_t max_seq_len,
                                  float sm_scale, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

const char* kvq_status_string(kvq_status status);

/* Message describing the calling thread's last non-OK status ("" if none). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
