"""Seeded random configurations of the decode step (kvq_decode_step) against the oracle: 1 to
12 sequences of ragged lengths (empty: no new token; page-partial; split over several
workgroups, with the chunks' partials merged after the launch), 1 to 4
KV heads, group sizes 1 to 16, every bit-width pair, both quantizers, the three input types,
with and without a key transform, shuffled pages.  The oracle writes every position but the
last; the step attends to the last one (a new token per sequence) at full precision and
appends it.
  * values, and keys without a transform, are written exactly as the oracle appends them;
  * the output is within 2e-3 per row of the oracle's step, and a split step given exactly
    the decode's workspace by the caller writes and returns the same bits."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from decode_attention_kvq_amd import api
from helpers import describe_mismatch, row_rel_err
from test_gpu_step import _gpu, _setup

pytestmark = pytest.mark.gpu

BITS = [(2, 2), (4, 4), (2, 4), (4, 2), (3, 3), (3, 2), (2, 3), (4, 3), (3, 4)]
QUANTS = [("percentile", "percentile"), ("rms", "rms"), ("percentile", "rms"), ("rms", "percentile")]


def _case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 13))
    H = int(rng.integers(1, 5))
    G = int(rng.integers(1, 17))
    bits = BITS[int(rng.integers(len(BITS)))]
    quant = QUANTS[int(rng.integers(len(QUANTS)))]
    dtype = ["f32", "bf16", "f16"][int(rng.integers(3))]
    with_t = bool(rng.integers(2))
    kinds = rng.integers(0, 4, size=B)
    lens = np.where(kinds == 0, 0, np.where(kinds == 1, rng.integers(1, 64, size=B),
                    np.where(kinds == 2, rng.integers(64, 1200, size=B), rng.integers(1200, 6000, size=B))))
    return rng, B, H, G, bits, quant, dtype, with_t, [int(x) for x in lens]


@pytest.mark.parametrize("seed", range(16))
def test_random_step_configuration(seed):
    rng, B, H, G, bits, quant, dtype, with_t, lens = _case(zlib.crc32(b"step-random-%d" % seed))
    if max(lens) == 0:
        lens[0] = 1
    info = (B, H, G, bits, quant, dtype, with_t, lens)
    print(info, flush=True)
    s = _setup(rng, B, H, G, lens, bits, quant, dtype, with_t)
    out, kf, vf = _gpu(s, H, bits, quant, dtype, lens, fused=True)
    # the oracle: its own append of the new tokens into the same starting cache, then decode
    kp, vp = s["kp"].copy(), s["vp"].copy()
    oracle.append(kp, vp, s["knew"], s["vnew"], s["new_slots"], t_k=s["t"], **s["kw"])
    assert np.array_equal(vf, vp), (info, describe_mismatch(vf, vp))
    if not with_t:
        assert np.array_equal(kf, kp), (info, describe_mismatch(kf, kp))
    ref = oracle.decode_step(kp, vp, s["q"], s["bt"], np.array(lens, np.int32), s["knew"], s["vnew"],
                             t_inv_t=s["tinv"], bits_k=bits[0], bits_v=bits[1])
    empty = np.array(lens) == 0
    assert np.all(out[empty] == 0), info
    err = row_rel_err(out[~empty], ref[~empty])
    assert err.max() <= 2e-3, (info, float(err.max()))
    # a split decode with a workspace the caller sizes exactly
    cache = api.KVCache(s["P"], H, bits[0], bits[1], quant[0], quant[1])
    split = api.decode_workspace_bytes(cache, B, H * G, max(lens)) > 0
    if split:
        out_m, km, vm = _gpu(s, H, bits, quant, dtype, lens, fused=True, min_workspace=True)
        assert np.array_equal(kf, km) and np.array_equal(vf, vm), info
        assert np.array_equal(out, out_m), (info, float(np.abs(out - out_m).max()))
