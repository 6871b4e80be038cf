"""Seeded random configurations of the write path against the oracle: batch sizes on both sides
of the small/tile boundary with ragged tails, 1 to 8 KV heads, every bit-width pair, both
quantizers, all three input types, and slot layouts that mix aligned runs, scattered slots,
skipped tokens and runs that start mid-word.  Without a transform the pools must be
bit-exact; with one (16-bit inputs on the matrix cores) the stage-B bounds apply."""
import zlib

import numpy as np
import pytest
import torch

from decode_attention_kvq_amd import calib, synth
from helpers import describe_mismatch, f16_ulp_distance, pool_codes, rare_event_bound
from test_gpu_append import _inputs, _run_both

pytestmark = pytest.mark.gpu

BITS = [(2, 2), (4, 4), (2, 4), (4, 2), (3, 3), (3, 2), (2, 3), (4, 3), (3, 4)]
QUANTS = [("percentile", "percentile"), ("rms", "rms"), ("percentile", "rms"), ("rms", "percentile")]
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _slots(rng, n, num_pages, kind):
    if kind == "aligned":
        return np.arange(n, dtype=np.int64) + 64 * int(rng.integers(0, 3))
    if kind == "offset":                 # a contiguous run that starts inside a word
        return np.arange(n, dtype=np.int64) + int(rng.integers(1, 31))
    s = rng.permutation(num_pages * 64)[:n].astype(np.int64)
    s[rng.random(n) < 0.05] = -1         # skipped tokens
    return s


def _case(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.choice([int(rng.integers(1, 512)), int(rng.integers(513, 2600))]))
    H = int(rng.integers(1, 9))
    bits = BITS[int(rng.integers(len(BITS)))]
    quant = QUANTS[int(rng.integers(len(QUANTS)))]
    dtype = ["f32", "bf16", "f16"][int(rng.integers(3))]
    kind = ["aligned", "offset", "scattered"][int(rng.integers(3))]
    with_t = dtype != "f32" and bool(rng.integers(2))
    return rng, n, H, bits, quant, dtype, kind, with_t


@pytest.mark.parametrize("seed", range(24))
def test_random_write_path_configuration(seed):
    rng, n, H, bits, quant, dtype, kind, with_t = _case(zlib.crc32(b"append-random-%d" % seed))
    num_pages = (n + 64) // 64 + 3
    k, v = _inputs(n, H, rng, dtype=dtype, config=1 if with_t else 0)
    slots = _slots(rng, n, num_pages, kind)
    t = None
    if with_t:
        ts = []
        for h in range(H):
            kc, qc = synth.calibration_set(1, h % 8, 4)
            ts.append(calib.calibrate_key_transform(kc, qc)[0])
        t = np.stack(ts)
        if dtype == "f16":
            t = t.astype(np.float16).astype(np.float32)
    gk, gv, ok, ov = _run_both(k, v, slots, num_pages, H, bits, quant, rng, t=t,
                               torch_dtype=TORCH[dtype])
    info = (n, H, bits, quant, dtype, kind, with_t)
    assert np.array_equal(gv, ov), (info, describe_mismatch(gv, ov))
    if t is None:
        assert np.array_equal(gk, ok), (info, describe_mismatch(gk, ok))
        return
    live = slots[slots >= 0]
    gc, gs, gz = pool_codes(gk, 0, bits[0], live)
    oc, os_, oz = pool_codes(ok, 0, bits[0], live)
    assert np.sum(gc != oc) <= max(2, 1e-4 * gc.size), (info, np.sum(gc != oc))
    bad = (gs != os_) | (gz != oz)
    assert np.sum(bad) <= rare_event_bound(bad.size), (info, np.sum(bad))
    assert np.all(f16_ulp_distance(gs, os_) <= 1) and np.all(f16_ulp_distance(gz, oz) <= 1), info
