"""Synthetic attention-stage error study: the relative squared L2 error of q.k, of the
softmax and of the attention output when the keys are cached with the RMS-clipped
(QuEST-style) quantizer after the identity (I), a random rotation (R), the normalised
Hadamard transform (H) or the WUSH transform, at 2, 3 and 4 bits ("WUSH-KV", §5.1-§5.2 and
their Figs. 1-2, which compare the same transforms on the same three stages of one
attention layer).  Stand-in data: the Sigma-model keys and queries of one Qwen3-8B-shaped
KV head (4 query heads), calibration from independent draws; values unquantized, so the
output error is the keys'.  Encoding through the oracle (fp16 scale/zero, RNE codes).

Checks the direction the pages report: WUSH gives the smallest error at every stage and
width; every transform's error falls as bits are added.  `PYTHONPATH=. python tests/test_error_study.py`
prints the table.
"""
import numpy as np
import pytest

import oracle
from decode_attention_kvq_amd import calib, synth

D, G, N, NQ, CONFIG, HEAD = 128, 4, 2048, 128, 1, 0
ALPHA = 2.83


def _transforms():
    kc, qc = synth.calibration_set(CONFIG, HEAD, G)
    rng = np.random.default_rng(2024)
    return {"I": np.eye(D), "R": synth.haar_orthogonal(D, rng), "H": calib.sylvester_hadamard(D),
            "WUSH": calib.wush(*calib.key_statistics(kc, qc))}


def _softmax(s):
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def _rel(a, b):
    return float(np.sum((a - b) ** 2) / np.sum(b ** 2))


def study(bits_list=(2, 3, 4)):
    k = synth.keys(CONFIG, HEAD, N, offset_seed=11).astype(np.float64)
    v = synth.values(CONFIG, HEAD, N, offset_seed=11).astype(np.float64)
    q = np.concatenate([synth.queries(CONFIG, HEAD * G + g, NQ, offset_seed=11) for g in range(G)]).astype(np.float64)
    s = q @ k.T / np.sqrt(D)
    p = _softmax(s)
    o = p @ v
    rows = {}
    for name, t in _transforms().items():
        kt = (k @ t).astype(np.float32)
        for bits in bits_list:
            c, sh, zh, _, _ = oracle.quantize_rows(kt, bits, oracle.RMS, alpha=ALPHA)
            kq = c * oracle.f16_bits_to_f32(sh)[:, None].astype(np.float64) + \
                oracle.f16_bits_to_f32(zh)[:, None].astype(np.float64)
            sq = (q @ np.linalg.inv(t).T) @ kq.T / np.sqrt(D)
            pq = _softmax(sq)
            rows[(name, bits)] = (_rel(sq, s), _rel(pq, p), _rel(pq @ v, o))
    return rows


@pytest.fixture(scope="module")
def rows():
    return study()


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("stage", [0, 1, 2])
def test_wush_has_the_smallest_error(rows, bits, stage):
    errs = {name: rows[(name, bits)][stage] for name in ("I", "R", "H", "WUSH")}
    assert errs["WUSH"] == min(errs.values()), errs


@pytest.mark.parametrize("name", ["I", "R", "H", "WUSH"])
def test_error_falls_with_bits(rows, name):
    for stage in range(3):
        e2, e3, e4 = (rows[(name, b)][stage] for b in (2, 3, 4))
        assert e2 > e3 > e4, (name, stage, e2, e3, e4)


if __name__ == "__main__":
    r = study()
    print("| transform | bits | q.k | softmax | output |")
    print("|---|---|---|---|---|")
    for (name, bits), (a, b, c) in r.items():
        print(f"| {name} | {bits} | {a:.3e} | {b:.3e} | {c:.3e} |")
