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
