"""Python binding of the kvq C ABI for torch tensors.

Argument marshalling only: tensors supply device pointers, the current torch stream
supplies the hipStream_t, and every step of the computation runs in the HIP kernels of
libkvq.so.  Function names follow the C entry points (kvq_quantize_append,
kvq_decode_attn, kvq_decode_step, kvq_dequant, and the full-precision window calls
kvq_window_prefill, kvq_window_decode_attn, kvq_window_decode_step).
"""
from __future__ import annotations

import ctypes as C
import math

import torch

from ._lib import KvqCacheDesc, KvqWindowDesc, check, load

HEAD_DIM = 128
PAGE_TOKENS = 64
QUANTIZERS = {"percentile": 0, "rms": 1}
_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


def block_bytes(bits: int) -> int:
    n = int(load().kvq_block_bytes(bits))
    if n == 0:
        raise ValueError("bits must be 2, 3 or 4")
    return n


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _shape(t, name, *dims):
    """Raises ValueError unless t (when given) has exactly the shape dims (None: any size).
    Runs before anything reaches the library: a short tensor would be read past its end on
    the device."""
    if t is None:
        return
    if t.dim() != len(dims) or any(d is not None and s != d for s, d in zip(t.shape, dims)):
        want = "[" + ", ".join("*" if d is None else str(d) for d in dims) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")


def _dev(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")


class KVCache:
    """One layer's paged, packed K and V pools ([num_pages, kv_heads, block_bytes] uint8)."""

    def __init__(self, num_pages: int, num_kv_heads: int, bits_k: int = 2, bits_v: int = 2,
                 quant_k: str = "percentile", quant_v: str = "percentile", p_lo: float = 0.01,
                 p_hi: float = 0.99, alpha_k: float = 2.83, alpha_v: float = 2.83,
                 device="cuda", k_pages=None, v_pages=None):
        self.num_pages, self.num_kv_heads = num_pages, num_kv_heads
        self.bits_k, self.bits_v = bits_k, bits_v
        self.quant_k, self.quant_v = quant_k, quant_v
        self.p_lo, self.p_hi, self.alpha_k, self.alpha_v = p_lo, p_hi, alpha_k, alpha_v
        shape_k = (num_pages, num_kv_heads, block_bytes(bits_k))
        shape_v = (num_pages, num_kv_heads, block_bytes(bits_v))
        self.k_pages = torch.zeros(shape_k, dtype=torch.uint8, device=device) if k_pages is None else k_pages
        self.v_pages = torch.zeros(shape_v, dtype=torch.uint8, device=device) if v_pages is None else v_pages
        _shape(self.k_pages, "k_pages", *shape_k)
        _shape(self.v_pages, "v_pages", *shape_v)
        _dev(self.k_pages, "k_pages", torch.uint8)
        _dev(self.v_pages, "v_pages", torch.uint8)

    def desc(self) -> KvqCacheDesc:
        return KvqCacheDesc(self.num_kv_heads, HEAD_DIM, PAGE_TOKENS, self.bits_k, self.bits_v,
                            QUANTIZERS[self.quant_k], QUANTIZERS[self.quant_v], self.p_lo, self.p_hi,
                            self.alpha_k, self.alpha_v, self.num_pages, self.k_pages.data_ptr(),
                            self.v_pages.data_ptr())


def kvq_quantize_append(cache: KVCache, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                        t_k: torch.Tensor | None = None, stream=None) -> None:
    """k, v: [n, kv_heads, 128] (f32/bf16/f16); slot_mapping: [n] int64; t_k: [kv_heads,128,128]."""
    H = cache.num_kv_heads
    _shape(k, "k", None, H, HEAD_DIM)
    n = k.shape[0]
    _shape(v, "v", n, H, HEAD_DIM); _shape(slot_mapping, "slot_mapping", n)
    _shape(t_k, "t_k", H, HEAD_DIM, HEAD_DIM)
    _dev(k, "k"); _dev(v, "v", k.dtype); _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(t_k, "t_k", k.dtype)
    d = cache.desc()
    check(load().kvq_quantize_append(C.byref(d), _ptr(k), _ptr(v), _DTYPES[k.dtype], n,
                                     _ptr(slot_mapping), _ptr(t_k), _DTYPES[k.dtype], _stream(stream)))


def decode_workspace_bytes(cache: KVCache, batch: int, num_q_heads: int, max_seq_len: int) -> int:
    d = cache.desc()
    return int(load().kvq_decode_workspace_bytes(C.byref(d), batch, num_q_heads, max_seq_len))


def decode_step_workspace_bytes(cache: KVCache, batch: int, num_q_heads: int, max_seq_len: int) -> int:
    """Workspace bytes of kvq_decode_step: the same as decode_workspace_bytes (the step's
    append runs in the decode's own launch and needs no workspace)."""
    d = cache.desc()
    return int(load().kvq_decode_step_workspace_bytes(C.byref(d), batch, num_q_heads, max_seq_len))


def _read_shapes(cache, q, block_table, seq_lens, t_k_inv_t, out, win_rows=None):
    """Shape checks shared by the read calls; returns (B, Hq)."""
    H = cache.num_kv_heads
    _shape(q, "q", None, None, HEAD_DIM)
    B, Hq = q.shape[0], q.shape[1]
    if Hq % H != 0:
        raise ValueError(f"q has {Hq} heads, not a multiple of the cache's {H} KV heads")
    _shape(block_table, "block_table", B, None); _shape(seq_lens, "seq_lens", B)
    _shape(win_rows, "win_rows", B)
    _shape(t_k_inv_t, "t_k_inv_t", H, HEAD_DIM, HEAD_DIM); _shape(out, "out", B, Hq, HEAD_DIM)
    return B, Hq


def kvq_decode_attn(cache: KVCache, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                    max_seq_len: int, t_k_inv_t: torch.Tensor | None = None, sm_scale: float | None = None,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """q: [B, Hq, 128]; block_table: [B, max_pages] int32; seq_lens: [B] int32.
    Returns out [B, Hq, 128] fp32 in the transformed value basis."""
    B, Hq = _read_shapes(cache, q, block_table, seq_lens, t_k_inv_t, out)
    _dev(q, "q"); _dev(block_table, "block_table", torch.int32); _dev(seq_lens, "seq_lens", torch.int32)
    _dev(t_k_inv_t, "t_k_inv_t", torch.float32)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    need = decode_workspace_bytes(cache, B, Hq, max_seq_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = cache.desc()
    check(load().kvq_decode_attn(C.byref(d), _ptr(q), _DTYPES[q.dtype], B, Hq, _ptr(t_k_inv_t),
                                 _ptr(block_table), block_table.shape[1], _ptr(seq_lens), max_seq_len,
                                 float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def kvq_decode_attn_noalloc(cache: KVCache, q: torch.Tensor, block_table: torch.Tensor,
                            seq_lens: torch.Tensor, max_seq_len: int, out: torch.Tensor,
                            t_k_inv_t: torch.Tensor | None = None, sm_scale: float | None = None,
                            stream=None) -> torch.Tensor:
    """kvq_decode_attn without a workspace, for callers that cannot allocate: `out`
    [B, Hq, 128] fp32 is the caller's; the split partials use the library's device array
    (KVQ_NOALLOC_SCRATCH_BYTES per GPU).  Calls that can overlap on one GPU race."""
    B, Hq = _read_shapes(cache, q, block_table, seq_lens, t_k_inv_t, out)
    _dev(q, "q"); _dev(block_table, "block_table", torch.int32); _dev(seq_lens, "seq_lens", torch.int32)
    _dev(t_k_inv_t, "t_k_inv_t", torch.float32); _dev(out, "out", torch.float32)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    d = cache.desc()
    check(load().kvq_decode_attn_noalloc(C.byref(d), _ptr(q), _DTYPES[q.dtype], B, Hq, _ptr(t_k_inv_t),
                                         _ptr(block_table), block_table.shape[1], _ptr(seq_lens), max_seq_len,
                                         float(sm_scale), _ptr(out), _stream(stream)))
    return out


def kvq_decode_step(cache: KVCache, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    new_slots: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                    max_seq_len: int, t_k: torch.Tensor | None = None,
                    t_k_inv_t: torch.Tensor | None = None, sm_scale: float | None = None,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """One decode step: each sequence's new token (k_new, v_new: [B, kv_heads, 128]; position
    seq_lens[b]-1) takes part in the attention at full precision beside positions
    [0, seq_lens[b]-1) of the cache, and is quantized into the cache at new_slots[b] ([B]
    int64) for later steps.  Returns out."""
    B, Hq = _read_shapes(cache, q, block_table, seq_lens, t_k_inv_t, out)
    H = cache.num_kv_heads
    _shape(k_new, "k_new", B, H, HEAD_DIM); _shape(v_new, "v_new", B, H, HEAD_DIM)
    _shape(new_slots, "new_slots", B); _shape(t_k, "t_k", H, HEAD_DIM, HEAD_DIM)
    _dev(q, "q"); _dev(k_new, "k_new", q.dtype); _dev(v_new, "v_new", q.dtype)
    _dev(new_slots, "new_slots", torch.int64); _dev(t_k, "t_k", q.dtype)
    _dev(block_table, "block_table", torch.int32); _dev(seq_lens, "seq_lens", torch.int32)
    _dev(t_k_inv_t, "t_k_inv_t", torch.float32)
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    need = decode_step_workspace_bytes(cache, B, Hq, max_seq_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = cache.desc()
    check(load().kvq_decode_step(C.byref(d), _ptr(q), _ptr(k_new), _ptr(v_new), _DTYPES[q.dtype], B, Hq,
                                 _ptr(new_slots), _ptr(t_k), _DTYPES[q.dtype], _ptr(t_k_inv_t),
                                 _ptr(block_table), block_table.shape[1], _ptr(seq_lens), max_seq_len,
                                 float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def kvq_dequant(cache: KVCache, which: int, slots: torch.Tensor, out: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """which = 0 keys, 1 values; slots: [n] int64 -> [n, kv_heads, 128] fp32."""
    _shape(slots, "slots", None)
    n = slots.shape[0]
    _shape(out, "out", n, cache.num_kv_heads, HEAD_DIM)
    _dev(slots, "slots", torch.int64)
    if out is None:
        out = torch.zeros((n, cache.num_kv_heads, HEAD_DIM), dtype=torch.float32, device=slots.device)
    _dev(out, "out", torch.float32)
    d = cache.desc()
    check(load().kvq_dequant(C.byref(d), which, _ptr(slots), n, _ptr(out), _stream(stream)))
    return out


# --------------------------------------------------------------------------------------
# Full-precision cache windows ("WUSH-KV" §4.4)
# --------------------------------------------------------------------------------------

class Window:
    """Full-precision window rows of one layer: k_win, v_win [num_rows, sink+keep+flush,
    kv_heads, 128] of `dtype` (the dtype of every activation passed with them)."""

    def __init__(self, cache: KVCache, num_rows: int, sink: int, keep: int, flush: int,
                 dtype=torch.bfloat16, device="cuda", k_win=None, v_win=None):
        self.sink, self.keep, self.flush, self.num_rows, self.dtype = sink, keep, flush, num_rows, dtype
        shape = (num_rows, sink + keep + flush, cache.num_kv_heads, HEAD_DIM)
        self.k_win = torch.zeros(shape, dtype=dtype, device=device) if k_win is None else k_win
        self.v_win = torch.zeros(shape, dtype=dtype, device=device) if v_win is None else v_win
        _shape(self.k_win, "k_win", *shape)
        _shape(self.v_win, "v_win", *shape)
        _dev(self.k_win, "k_win", dtype)
        _dev(self.v_win, "v_win", dtype)

    def desc(self) -> KvqWindowDesc:
        return KvqWindowDesc(self.sink, self.keep, self.flush, self.num_rows, _DTYPES[self.dtype],
                             self.k_win.data_ptr(), self.v_win.data_ptr())


def kvq_window_prefill(cache: KVCache, win: Window, k: torch.Tensor, v: torch.Tensor,
                       cu_seqlens: torch.Tensor, block_table: torch.Tensor,
                       win_rows: torch.Tensor | None = None, t_k: torch.Tensor | None = None,
                       stream=None) -> None:
    """Fresh prompts packed as k, v [n, kv_heads, 128] with offsets cu_seqlens [B+1] int32."""
    H = cache.num_kv_heads
    _shape(k, "k", None, H, HEAD_DIM)
    _shape(v, "v", k.shape[0], H, HEAD_DIM)
    _shape(cu_seqlens, "cu_seqlens", None)
    if cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens has shape [0], expected [batch + 1]")
    _shape(block_table, "block_table", cu_seqlens.shape[0] - 1, None)
    _shape(win_rows, "win_rows", cu_seqlens.shape[0] - 1); _shape(t_k, "t_k", H, HEAD_DIM, HEAD_DIM)
    _dev(k, "k", win.dtype); _dev(v, "v", win.dtype); _dev(cu_seqlens, "cu_seqlens", torch.int32)
    _dev(block_table, "block_table", torch.int32); _dev(win_rows, "win_rows", torch.int32)
    _dev(t_k, "t_k", win.dtype)
    n = k.shape[0]
    B = cu_seqlens.shape[0] - 1
    d, w = cache.desc(), win.desc()
    check(load().kvq_window_prefill(C.byref(d), C.byref(w), _ptr(k), _ptr(v), B, _ptr(cu_seqlens), n,
                                    _ptr(block_table), block_table.shape[1], _ptr(win_rows), _ptr(t_k),
                                    _stream(stream)))


def window_workspace_bytes(cache: KVCache, win: Window, batch: int, num_q_heads: int, max_seq_len: int) -> int:
    d, w = cache.desc(), win.desc()
    return int(load().kvq_window_workspace_bytes(C.byref(d), C.byref(w), batch, num_q_heads, max_seq_len))


def _window_out_ws(cache, win, q, max_seq_len, out, workspace):
    B, Hq, _ = q.shape
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32)
    need = window_workspace_bytes(cache, win, B, Hq, max_seq_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return out, workspace, ws_bytes


def kvq_window_decode_attn(cache: KVCache, win: Window, q: torch.Tensor, block_table: torch.Tensor,
                           seq_lens: torch.Tensor, max_seq_len: int, win_rows: torch.Tensor | None = None,
                           t_k_inv_t: torch.Tensor | None = None, sm_scale: float | None = None,
                           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                           stream=None) -> torch.Tensor:
    """Attention over a windowed cache (state after every waiting batch was quantized)."""
    B, Hq = _read_shapes(cache, q, block_table, seq_lens, t_k_inv_t, out, win_rows)
    _dev(q, "q", win.dtype); _dev(block_table, "block_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32); _dev(win_rows, "win_rows", torch.int32)
    _dev(t_k_inv_t, "t_k_inv_t", torch.float32)
    out, workspace, ws_bytes = _window_out_ws(cache, win, q, max_seq_len, out, workspace)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    d, w = cache.desc(), win.desc()
    check(load().kvq_window_decode_attn(C.byref(d), C.byref(w), _ptr(q), B, Hq, _ptr(t_k_inv_t),
                                        _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                        _ptr(win_rows), max_seq_len, float(sm_scale), _ptr(out),
                                        _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def kvq_window_decode_step(cache: KVCache, win: Window, q: torch.Tensor, k_new: torch.Tensor,
                           v_new: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                           max_seq_len: int, win_rows: torch.Tensor | None = None,
                           t_k: torch.Tensor | None = None, t_k_inv_t: torch.Tensor | None = None,
                           sm_scale: float | None = None, out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode step: seq_lens [B] counts the new position, whose key and value are
    k_new, v_new [B, kv_heads, 128]; attention, then the flush of the batch it made eligible."""
    B, Hq = _read_shapes(cache, q, block_table, seq_lens, t_k_inv_t, out, win_rows)
    H = cache.num_kv_heads
    _shape(k_new, "k_new", B, H, HEAD_DIM); _shape(v_new, "v_new", B, H, HEAD_DIM)
    _shape(t_k, "t_k", H, HEAD_DIM, HEAD_DIM)
    _dev(q, "q", win.dtype); _dev(k_new, "k_new", win.dtype); _dev(v_new, "v_new", win.dtype)
    _dev(block_table, "block_table", torch.int32); _dev(seq_lens, "seq_lens", torch.int32)
    _dev(win_rows, "win_rows", torch.int32); _dev(t_k, "t_k", win.dtype)
    _dev(t_k_inv_t, "t_k_inv_t", torch.float32)
    out, workspace, ws_bytes = _window_out_ws(cache, win, q, max_seq_len, out, workspace)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    d, w = cache.desc(), win.desc()
    check(load().kvq_window_decode_step(C.byref(d), C.byref(w), _ptr(q), _ptr(k_new), _ptr(v_new), B, Hq,
                                        _ptr(t_k), _ptr(t_k_inv_t), _ptr(block_table), block_table.shape[1],
                                        _ptr(seq_lens), _ptr(win_rows), max_seq_len, float(sm_scale),
                                        _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out
