"""CPU oracle for the quantized-KV-cache hot path (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  It is independent of the HIP library: it shares no code
with it and imports nothing from it.  The arithmetic lives in ``kvq_oracle.c``
(plain C, built with gcc ``-O2 -ffp-contract=off``); this module builds it, loads
it with ctypes and wraps it for numpy arrays.  ``wush.py`` holds the fp64
calibration reference.

Parity status of each function is stated in its docstring.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

HEAD_DIM = 128
PAGE_TOKENS = 64
PERCENTILE = 0
RMS = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i64, i32, f32, f64 = C.c_int64, C.c_int, C.c_float, C.c_double
        L.oracle_f32_to_f16.restype = C.c_uint16
        L.oracle_f32_to_f16.argtypes = [f32]
        L.oracle_f16_to_f32.restype = f32
        L.oracle_f16_to_f32.argtypes = [C.c_uint16]
        L.oracle_f32_to_f16_array.argtypes = [P, P, i64]
        L.oracle_f16_to_f32_array.argtypes = [P, P, i64]
        L.oracle_transform_keys.argtypes = [P, P, i64, i32, P]
        L.oracle_percentile_position.argtypes = [f32, i32, P, P]
        L.oracle_clip_percentile.argtypes = [P, i32, f32, f32, P, P]
        L.oracle_clip_rms.argtypes = [P, i32, f32, P, P]
        L.oracle_quantize_group.argtypes = [P, i32, i32, f32, f32, P, P, P]
        L.oracle_quantize_rows.argtypes = [P, i64, i32, i32, f32, f32, f32, P, P, P, P, P]
        L.oracle_block_bytes.restype = i64
        L.oracle_block_bytes.argtypes = [i32]
        L.oracle_pack_token.argtypes = [P, i32, i32, i32, P, C.c_uint16, C.c_uint16]
        L.oracle_unpack_token.argtypes = [P, i32, i32, i32, P, P, P]
        L.oracle_append.restype = i32
        L.oracle_append.argtypes = [P, P, i64, i32, i32, i32, i32, i32, f32, f32, f32, f32,
                                    P, P, P, i64, P]
        L.oracle_dequant.argtypes = [P, i32, i32, i32, P, i64, P]
        L.oracle_decode_attention.argtypes = [P, P, i32, i32, i32, P, i32, i32, P, P, i32, P,
                                              f64, P, P]
        L.oracle_window_quantized.restype = i64
        L.oracle_window_quantized.argtypes = [i64, i32, i32, i32]
        L.oracle_window_attention.argtypes = [P, P, i32, i32, i32, P, i32, i32, P, P, i32, P, i32,
                                              i32, i32, i32, P, P, i64, f64, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# --------------------------------------------------------------------------- fp16

def f32_to_f16_bits(x) -> np.ndarray:
    """IEEE binary16 bits of fp32 values, round to nearest even (written from the format)."""
    x = _f32(x)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_f16_array(_p(x), _p(out), x.size)
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_f16_to_f32_array(_p(h), _p(out), h.size)
    return out


# --------------------------------------------------------------------------- O1-O4

def transform_keys(k, t) -> np.ndarray:
    """O1: k' = k . T per KV head, fp64 accumulation rounded to fp32.

    k: [n, H, 128]; t: [H, 128, 128] or None.  Pinned by the query-compensation identity
    (q T^-T).(k T) = q.k and by T = I reducing to a copy.
    """
    k = _f32(k)
    n, H, d = k.shape
    out = np.empty_like(k)
    tt = None if t is None else _f32(t)
    lib().oracle_transform_keys(_p(k), _p(tt), n, H, _p(out))
    return out


def percentile_position(p: float, n: int = HEAD_DIM):
    """(i, f) for an fp32 percentile p: rank = fp64(p) * (n-1), f rounded to fp32."""
    i = C.c_int()
    f = C.c_float()
    lib().oracle_percentile_position(p, n, C.byref(i), C.byref(f))
    return i.value, f.value


def quantize_rows(x, bits: int, quantizer: int = PERCENTILE, p_lo: float = 0.01,
                  p_hi: float = 0.99, alpha: float = 2.83):
    """O2-O4 on each row of x [rows, 128]: returns (codes u8, scale f16 bits, zero f16 bits,
    lo, hi).  Pinned by numpy.percentile, the RMS closed form, code range, the half-step
    error bound and brute-force nearest-level search (tests/test_oracle_quant.py)."""
    x = _f32(x).reshape(-1, HEAD_DIM)
    rows = x.shape[0]
    codes = np.empty((rows, HEAD_DIM), np.uint8)
    s = np.empty(rows, np.uint16)
    z = np.empty(rows, np.uint16)
    lo = np.empty(rows, np.float32)
    hi = np.empty(rows, np.float32)
    lib().oracle_quantize_rows(_p(x), rows, bits, quantizer, p_lo, p_hi, alpha,
                               _p(codes), _p(s), _p(z), _p(lo), _p(hi))
    return codes, s, z, lo, hi


# --------------------------------------------------------------------------- O5-O7

def block_bytes(bits: int) -> int:
    return int(lib().oracle_block_bytes(bits))


def new_pool(num_pages: int, kv_heads: int, bits: int, fill=None, rng=None) -> np.ndarray:
    """A host page pool [num_pages, kv_heads, block_bytes] of uint8."""
    shape = (num_pages, kv_heads, block_bytes(bits))
    if rng is not None:
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.full(shape, 0 if fill is None else fill, np.uint8)


def pack_token(block: np.ndarray, which: int, bits: int, o: int, codes, scale_h, zero_h):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    assert block.flags.c_contiguous and block.dtype == np.uint8
    lib().oracle_pack_token(_p(block), which, bits, o, _p(codes), int(scale_h), int(zero_h))


def unpack_token(block: np.ndarray, which: int, bits: int, o: int):
    codes = np.empty(HEAD_DIM, np.uint8)
    s = C.c_uint16()
    z = C.c_uint16()
    block = np.ascontiguousarray(block, dtype=np.uint8)
    lib().oracle_unpack_token(_p(block), which, bits, o, _p(codes), C.byref(s), C.byref(z))
    return codes, s.value, z.value


def append(k_pool, v_pool, k, v, slots, t_k=None, bits_k=2, bits_v=2,
           quant_k=PERCENTILE, quant_v=PERCENTILE, p_lo=0.01, p_hi=0.99,
           alpha_k=2.83, alpha_v=2.83):
    """Write path (O1-O5) into host pools, in place."""
    k = _f32(k)
    v = _f32(v)
    n, H, _ = k.shape
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    tt = None if t_k is None else _f32(t_k)
    assert k_pool.shape[1] == H and k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    rc = lib().oracle_append(_p(k_pool), _p(v_pool), k_pool.shape[0], H, bits_k, bits_v,
                             quant_k, quant_v, p_lo, p_hi, alpha_k, alpha_v,
                             _p(k), _p(v), _p(tt), n, _p(slots))
    if rc != 0:
        raise ValueError("slot out of range")


def dequant(pool, which: int, bits: int, slots) -> np.ndarray:
    """O6: fp32 [n, H, 128] = fma(code, scale, zero)."""
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    H = pool.shape[1]
    out = np.zeros((slots.shape[0], H, HEAD_DIM), np.float32)
    lib().oracle_dequant(_p(pool), which, H, bits, _p(slots), slots.shape[0], _p(out))
    return out


def decode_attention(k_pool, v_pool, q, block_table, seq_lens, t_inv_t=None, bits_k=2,
                     bits_v=2, sm_scale=None, return_lse=False):
    """O7: exact two-pass softmax attention over the dequantized cache, fp64 output.

    q: [B, Hq, 128]; block_table: [B, max_pages] int32; seq_lens: [B] int32.
    Pinned against torch fp64 scaled_dot_product_attention on the dequantized tensors and
    closed-form special cases (tests/test_oracle_attention.py)."""
    q = _f32(q)
    B, Hq, _ = q.shape
    H = k_pool.shape[1]
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    tt = None if t_inv_t is None else _f32(t_inv_t)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(HEAD_DIM)
    out = np.zeros((B, Hq, HEAD_DIM), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    lib().oracle_decode_attention(_p(k_pool), _p(v_pool), H, bits_k, bits_v, _p(q), B, Hq,
                                  _p(tt), _p(bt), bt.shape[1], _p(sl), float(sm_scale),
                                  _p(out), _p(lse))
    return (out, lse) if return_lse else out


def decode_step(k_pool, v_pool, q, block_table, seq_lens, k_new, v_new, t_inv_t=None, bits_k=2,
                bits_v=2, sm_scale=None):
    """A decode step whose new token takes part at full precision ([W] §4.4: a new entry is
    used for attention before it is quantized), fp64 output.

    For each sequence b with L = seq_lens[b] > 0: softmax attention over positions
    [0, L - 1) dequantized from the cache (as decode_attention, with the compensated query)
    and the new token's own key k_new[b] and value v_new[b] ([B, H, 128]); the new token's
    score is sm_scale q . k_new, the product that q' . k' gives under the key transform.
    Rows of sequences with L = 0 are 0.  Pinned against torch fp64 attention over the
    cache's dequantized keys and values followed by the new row, with and without a key
    transform (tests/test_oracle_attention.py)."""
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out_q, lse_q = decode_attention(k_pool, v_pool, q, block_table, np.maximum(sl - 1, 0).astype(np.int32),
                                    t_inv_t=t_inv_t, bits_k=bits_k, bits_v=bits_v, sm_scale=sm_scale,
                                    return_lse=True)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(HEAD_DIM)
    q64 = _f32(q).astype(np.float64)
    kn = _f32(k_new).astype(np.float64)
    vn = _f32(v_new).astype(np.float64)
    B, Hq, _ = q64.shape
    G = Hq // k_pool.shape[1]
    out = np.zeros((B, Hq, HEAD_DIM), np.float64)
    for b in range(B):
        if sl[b] <= 0:
            continue
        for hq in range(Hq):
            s = float(sm_scale) * float(q64[b, hq] @ kn[b, hq // G])
            m = max(s, float(lse_q[b, hq]))
            w_cache = np.exp(lse_q[b, hq] - m)          # 0 when the cache part is empty
            w_new = np.exp(s - m)
            out[b, hq] = (w_cache * out_q[b, hq] + w_new * vn[b, hq // G]) / (w_cache + w_new)
    return out


def window_quantized(length: int, sink: int, keep: int, flush: int) -> int:
    """Full-precision windows ([W] §4.4): positions quantized once a sequence has grown to
    `length` and every waiting batch of `flush` eligible positions has been quantized.
    Pinned by hand-worked cases and invariants (tests/test_oracle_window.py)."""
    return int(lib().oracle_window_quantized(int(length), int(sink), int(keep), int(flush)))


def window_attention(k_pool, v_pool, q, block_table, seq_lens, k_fp, v_fp, sink, keep, flush,
                     pending=0, t_inv_t=None, bits_k=2, bits_v=2, sm_scale=None, return_lse=False):
    """Attention over a windowed cache ([W] §4.4), fp64 output.

    Positions sink .. sink+Q-1 are read dequantized from the paged cache at index
    position - sink (with the compensated query); every other position reads k_fp / v_fp
    [B, fp_len, H, 128] (the stored full-precision values) with the plain query.
    Q = window_quantized(seq_len - pending).  Pinned against decode_attention when every
    position is quantized, against plain softmax attention when none is, and against
    torch fp64 attention over keys mapped back to the original basis when mixed
    (tests/test_oracle_window.py)."""
    q = _f32(q)
    B, Hq, _ = q.shape
    H = k_pool.shape[1]
    kf = _f32(k_fp)
    vf = _f32(v_fp)
    assert kf.shape[0] == B and kf.shape[2] == H and vf.shape == kf.shape
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    assert int(sl.max(initial=0)) <= kf.shape[1]
    tt = None if t_inv_t is None else _f32(t_inv_t)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(HEAD_DIM)
    out = np.zeros((B, Hq, HEAD_DIM), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    lib().oracle_window_attention(_p(k_pool), _p(v_pool), H, bits_k, bits_v, _p(q), B, Hq, _p(tt),
                                  _p(bt), bt.shape[1], _p(sl), int(pending), int(sink), int(keep),
                                  int(flush), _p(kf), _p(vf), kf.shape[1], float(sm_scale),
                                  _p(out), _p(lse))
    return (out, lse) if return_lse else out
