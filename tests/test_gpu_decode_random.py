"""Seeded random configurations of the read path against the oracle: 1 to 12 sequences of
ragged lengths (empty, page-partial, split over several workgroups), 1 to 4 KV heads, every
group size from 1 to 16 (the padded column blocks of 4, 8 and 16), every bit-width pair,
both quantizers, the three query types, with and without a key transform, shuffled pages.
Stage C: the oracle writes the cache, the GPU decodes it; 2e-3 max relative error per row."""
import zlib

import numpy as np
import pytest

import oracle
from decode_attention_kvq_amd import synth
from helpers import row_rel_err
from test_gpu_decode import TOL, _gpu_decode, _oracle_cache, _transforms

pytestmark = pytest.mark.gpu

BITS = [(2, 2), (4, 4), (2, 4), (4, 2), (3, 3), (3, 2), (2, 3), (4, 3), (3, 4)]
QUANTS = [("percentile", "percentile"), ("rms", "rms"), ("percentile", "rms")]


def _case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 13))
    H = int(rng.integers(1, 5))
    G = int(rng.integers(1, 17))
    bits = BITS[int(rng.integers(len(BITS)))]
    quant = QUANTS[int(rng.integers(len(QUANTS)))]
    q_dtype = ["f32", "bf16", "f16"][int(rng.integers(3))]
    with_t = bool(rng.integers(2))
    kinds = rng.integers(0, 4, size=B)
    seq = np.where(kinds == 0, 0, np.where(kinds == 1, rng.integers(1, 64, size=B),
                   np.where(kinds == 2, rng.integers(64, 1200, size=B), rng.integers(1200, 6000, size=B))))
    return rng, B, H, G, bits, quant, q_dtype, with_t, seq.astype(np.int32)


@pytest.mark.parametrize("seed", range(24))
def test_random_read_path_configuration(seed):
    rng, B, H, G, bits, quant, q_dtype, with_t, seq = _case(zlib.crc32(b"decode-random-%d" % seed))
    info = (B, H, G, bits, quant, q_dtype, with_t, seq.tolist())
    t = tinv = None
    if with_t:
        t, tinv = _transforms(1, H, G)
    kp, vp, bt = _oracle_cache(rng, B, H, np.maximum(seq, 1), bits, t=t, quant=quant)
    q = synth.to_dtype(rng.standard_normal((B, H * G, 128)).astype(np.float32) * 2.0, q_dtype)
    got = _gpu_decode(kp, vp, q, bt, seq, bits, tinv=tinv, q_dtype=q_dtype, max_seq_len=int(max(seq.max(), 1)))
    ref = oracle.decode_attention(kp, vp, q, bt, seq, t_inv_t=tinv, bits_k=bits[0], bits_v=bits[1])
    empty = seq == 0
    assert np.all(got[empty] == 0), info
    if np.any(~empty):
        err = row_rel_err(got[~empty], ref[~empty])
        assert err.max() <= TOL, (info, float(err.max()))
