"""Shared helpers of the GPU parity tests (host side only)."""
from __future__ import annotations

import numpy as np

import oracle


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per (sequence, query head) row: max_j |got - ref| / max_j |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def pool_codes(pool: np.ndarray, which: int, bits: int, slots):
    """Codes, scale bits and zero bits of the given slots, read with the oracle's unpacker."""
    H = pool.shape[1]
    codes = np.zeros((len(slots), H, 128), np.uint8)
    s = np.zeros((len(slots), H), np.uint16)
    z = np.zeros((len(slots), H), np.uint16)
    for i, slot in enumerate(slots):
        p, o = divmod(int(slot), 64)
        for h in range(H):
            c, si, zi = oracle.unpack_token(pool[p, h], which, bits, o)
            codes[i, h], s[i, h], z[i, h] = c, si, zi
    return codes, s, z


def f16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in fp16 ulps between two arrays of fp16 bit patterns (same sign assumed
    when both are non-zero)."""
    def ordered(x):
        x = x.astype(np.int64)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a) - ordered(b))


def describe_mismatch(got: np.ndarray, ref: np.ndarray, limit: int = 8) -> str:
    idx = np.argwhere(got != ref)
    lines = [f"{len(idx)} of {got.size} differ"]
    for k in idx[:limit]:
        k = tuple(int(t) for t in k)
        lines.append(f"  at {k}: got {got[k]!r} ref {ref[k]!r}")
    return "\n".join(lines)


def rms_order_rows():
    """Two groups whose fp32 sum of squares depends on the order of the additions, worked
    by hand for the one 128-wide pairwise tree (stride 64, 32, ..., 1: element i < stride
    adds element i + stride).  Squares are exact; in [2^24, 2^25) fp32 numbers are 2 apart,
    so 2^24 + 1 rounds (tie to even) to 2^24.

    Row A: x[0] = 4096 (square 2^24), x[64..127] = 1.
      stride 64: s0 = 2^24 + 1 -> 2^24; s1..s63 = 1
      stride 32: s0 = 2^24 + 1 -> 2^24; s1..s31 = 2
      stride 16, 8, 4, 2, 1: s0 gains 2, 4, 8, 16, 32 exactly -> 2^24 + 62.
    (Summing each 64-channel half first and then the halves gives 2^24 + 64; a running
    sum from channel 0 gives 2^24.)
    Row B: x[0] = 4096, x[32..63] = x[96..127] = 1.
      stride 64: s0 = 2^24; s32..s63 = 2
      stride 32: s0 = 2^24 + 2; s1..s31 = 2
      stride 16, 8, 4, 2, 1: s0 gains 2, 4, 8, 16, 32 -> 2^24 + 64.
    (Halves first: 2^24 + 62.)
    Returns the rows and their sums of squares."""
    a = np.zeros(128, np.float32)
    a[0] = 4096.0
    a[64:] = 1.0
    b = np.zeros(128, np.float32)
    b[0] = 4096.0
    b[32:64] = 1.0
    b[96:] = 1.0
    return np.stack([a, b]), np.array([2.0 ** 24 + 62, 2.0 ** 24 + 64], np.float32)


def _threads(n_tasks: int) -> int:
    import os
    return max(1, min(16, os.cpu_count() or 1, n_tasks))


def oracle_append_sequence(k_pool, v_pool, k, v, slots, **kw):
    """oracle.append of one sequence's tokens (slots in position order, 64 to a page) in
    page-aligned chunks on worker threads: each chunk writes whole pages no other chunk
    touches, and the oracle call releases the GIL."""
    from concurrent.futures import ThreadPoolExecutor
    n = len(slots)
    step = 64 * max(1, -(-n // 64) // 64)
    chunks = [(a, min(a + step, n)) for a in range(0, n, step)]
    with ThreadPoolExecutor(_threads(len(chunks))) as ex:
        list(ex.map(lambda c: oracle.append(k_pool, v_pool, k[c[0]:c[1]], v[c[0]:c[1]], slots[c[0]:c[1]], **kw),
                    chunks))


def oracle_decode_sequence(k_pool, v_pool, q, pages, seq_len, t_inv_t=None, **kw):
    """oracle.decode_attention of one sequence (q [Hq, 128], its pages in order), one KV head
    per worker thread; returns [Hq, 128] fp64."""
    from concurrent.futures import ThreadPoolExecutor
    H = k_pool.shape[1]
    G = q.shape[0] // H
    kp = k_pool[pages]
    vp = v_pool[pages]
    bt = np.arange(len(pages), dtype=np.int32)[None]
    seq = np.array([seq_len], np.int32)

    def head(h):
        ti = None if t_inv_t is None else t_inv_t[h:h + 1]
        return oracle.decode_attention(np.ascontiguousarray(kp[:, h:h + 1]), np.ascontiguousarray(vp[:, h:h + 1]),
                                       q[None, h * G:(h + 1) * G], bt, seq, t_inv_t=ti, **kw)[0]
    with ThreadPoolExecutor(_threads(H)) as ex:
        return np.concatenate(list(ex.map(head, range(H))), axis=0)


def oracle_step_sequence(k_pool, v_pool, q, pages, seq_len, k_new, v_new, t_inv_t=None, **kw):
    """oracle.decode_step of one sequence (q [Hq, 128], its pages in order, its new token's
    rows k_new, v_new [H, 128]), one KV head per worker thread; returns [Hq, 128] fp64."""
    from concurrent.futures import ThreadPoolExecutor
    H = k_pool.shape[1]
    G = q.shape[0] // H
    kp = k_pool[pages]
    vp = v_pool[pages]
    bt = np.arange(len(pages), dtype=np.int32)[None]
    seq = np.array([seq_len], np.int32)

    def head(h):
        ti = None if t_inv_t is None else t_inv_t[h:h + 1]
        return oracle.decode_step(np.ascontiguousarray(kp[:, h:h + 1]), np.ascontiguousarray(vp[:, h:h + 1]),
                                  q[None, h * G:(h + 1) * G], bt, seq, k_new[None, h:h + 1], v_new[None, h:h + 1],
                                  t_inv_t=ti, **kw)[0]
    with ThreadPoolExecutor(_threads(H)) as ex:
        return np.concatenate(list(ex.map(head, range(H))), axis=0)


def pool_scales_zeros(pool: np.ndarray, bits: int, slots):
    """fp16 bit patterns of the scale and zero of every (slot, KV head): [n, H] each, read
    straight from the block layout (64 scales, then 64 zeros, after the code section)."""
    slots = np.asarray(slots, np.int64)
    cb = 64 * 128 * bits // 8
    p, o = slots // 64, slots % 64
    meta = pool[:, :, cb:cb + 256].view(np.uint16)           # [pages, H, 128]
    return meta[p, :, o], meta[p, :, 64 + o]


# Scale/zero one fp16 ulp apart: the fraction of groups allowed.  The GPU accumulates k . T
# in fp32 on the matrix cores, the oracle in fp64 with one rounding; the two differ by about
# one fp32 ulp on part of the elements, and a fraction of the clip bounds then round to fp16
# on either side of a boundary.  Measured over whole 16K-token sequences (131,072 groups):
# 4.6e-5 to 1.07e-4, so the bound is twice the 1e-4 first aimed at.
SCALE_ZERO_RATE = 2e-4


def rare_event_bound(n: int, rate: float = SCALE_ZERO_RATE) -> float:
    """Largest count of independent rare events (a scale or zero one fp16 ulp away because
    the GPU's fp32 transform sum and the oracle's fp64 sum round to fp16 on either side of a
    boundary) that n groups show with more than 99.9% probability when the true rate is
    `rate`: the Poisson mean plus three standard deviations, plus one.  Tests over a few
    thousand groups use it; tests over the 131,072 or more groups of a full 16K sequence
    assert the rate itself."""
    lam = rate * n
    return lam + 3.0 * lam ** 0.5 + 1.0
