"""Pins of the oracle's full-precision windows ("WUSH-KV" §4.4): the quantization policy and
attention over a cache whose sink and newest positions stay in full precision."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kvq_amd import synth


# Worked by hand for S_sink = 2, S_keep = 3, S_flush = 4: positions 0-1 are the sink; at
# length x the eligible positions are 2 .. x-4 (x - 5 of them), so the first batch
# (positions 2-5) goes at x = 9, the next (6-9) at x = 13, then 10-13 at x = 17.
HAND = {0: 0, 1: 0, 5: 0, 8: 0, 9: 4, 12: 4, 13: 8, 16: 8, 17: 12, 20: 12}


@pytest.mark.parametrize("length,expected", sorted(HAND.items()))
def test_quantized_count_worked_example(length, expected):
    assert oracle.window_quantized(length, 2, 3, 4) == expected


def _chunked_growth(chunks, sink, keep, flush):
    """Brute force with explicit position sets: append each chunk, then quantize the oldest
    `flush` eligible positions while at least `flush` of them wait."""
    quantized, n = set(), 0
    for c in chunks:
        n += c
        while True:
            waiting = sorted(p for p in range(sink, n - keep) if p not in quantized)
            if len(waiting) < flush:
                break
            quantized.update(waiting[:flush])
    return n, quantized


@pytest.mark.parametrize("sink,keep,flush", [(0, 0, 1), (0, 0, 64), (4, 0, 8), (0, 16, 8), (3, 5, 7),
                                             (32, 64, 64), (1, 1, 2)])
def test_quantized_count_matches_chunked_brute_force(sink, keep, flush):
    rng = np.random.default_rng(sink * 1000 + keep * 10 + flush)
    for _ in range(6):
        chunks = rng.integers(1, 40, size=rng.integers(1, 8)).tolist()
        n, qset = _chunked_growth(chunks, sink, keep, flush)
        nq = oracle.window_quantized(n, sink, keep, flush)
        assert qset == set(range(sink, sink + nq)), (chunks, nq)


@pytest.mark.parametrize("sink,keep,flush", [(0, 0, 1), (2, 3, 4), (32, 64, 64), (5, 0, 16), (0, 9, 3)])
def test_quantized_count_invariants(sink, keep, flush):
    prev = 0
    for n in range(0, 400):
        nq = oracle.window_quantized(n, sink, keep, flush)
        assert nq % flush == 0 and nq - prev in (0, flush)
        if nq:
            assert keep <= n - sink - nq < keep + flush
        else:
            assert n < sink + keep + flush
        prev = nq


# --------------------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------------------

def _setup(rng, B, H, G, lens, sink, keep, flush, bits=(2, 2), t=None):
    """Oracle-written pools holding every middle position (index position - sink) and the
    full-precision history of every position."""
    fp_len = max(lens)
    pps = max(1, -(-max(max(lens) - sink, 1) // 64))
    num_pages = B * pps + 2
    kp = oracle.new_pool(num_pages, H, bits[0], rng=rng)
    vp = oracle.new_pool(num_pages, H, bits[1], rng=rng)
    bt = synth.shuffled_block_table(B, pps, num_pages, rng)
    k_fp = rng.standard_normal((B, fp_len, H, 128)).astype(np.float32)
    v_fp = rng.standard_normal((B, fp_len, H, 128)).astype(np.float32)
    k_fp[..., :4] *= 6.0                    # a few outlier channels
    for b, L in enumerate(lens):
        nmid = max(L - sink, 0)
        j = np.arange(nmid)
        slots = bt[b, j // 64].astype(np.int64) * 64 + j % 64
        oracle.append(kp, vp, k_fp[b, sink:L], v_fp[b, sink:L], slots, t_k=t, bits_k=bits[0], bits_v=bits[1])
    q = rng.standard_normal((B, H * G, 128)).astype(np.float32)
    return kp, vp, bt, k_fp, v_fp, q


def _torch_reference(kp, vp, bt, k_fp, v_fp, q, lens, sink, keep, flush, pending, t_inv_t, bits):
    """Attention with every quantized key mapped back to the original basis
    (k^ = dequant(k') T^-1), so the plain query applies to every position."""
    B, Hq, _ = q.shape
    H = kp.shape[1]
    G = Hq // H
    out = np.zeros((B, Hq, 128))
    for b, L in enumerate(lens):
        nq = oracle.window_quantized(max(L - pending, 0), sink, keep, flush)
        K = k_fp[b, :L].astype(np.float64).copy()
        V = v_fp[b, :L].astype(np.float64).copy()
        if nq:
            j = np.arange(nq)
            slots = bt[b, j // 64].astype(np.int64) * 64 + j % 64
            kq = oracle.dequant(kp, 0, bits[0], slots).astype(np.float64)
            if t_inv_t is not None:
                kq = np.einsum("nhc,hjc->nhj", kq, t_inv_t.astype(np.float64))   # k' (T^-T)^T = k' T^-1
            K[sink:sink + nq] = kq
            V[sink:sink + nq] = oracle.dequant(vp, 1, bits[1], slots)
        for hq in range(Hq):
            h = hq // G
            qt = torch.from_numpy(q[b, hq].astype(np.float64))[None, None, None]
            kt = torch.from_numpy(K[:, h])[None, None]
            vt = torch.from_numpy(V[:, h])[None, None]
            out[b, hq] = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0, 0].numpy()
    return out


def test_all_positions_quantized_equals_plain_decode():
    rng = np.random.default_rng(7)
    lens = [128, 64, 192]
    kp, vp, bt, k_fp, v_fp, q = _setup(rng, 3, 2, 4, lens, 0, 0, 64)
    got = oracle.window_attention(kp, vp, q, bt, lens, k_fp, v_fp, 0, 0, 64)
    ref = oracle.decode_attention(kp, vp, q, bt, np.array(lens, np.int32))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_no_position_quantized_is_full_precision_attention():
    rng = np.random.default_rng(8)
    lens = [5, 40, 1]
    kp, vp, bt, k_fp, v_fp, q = _setup(rng, 3, 2, 2, lens, 4, 16, 32)
    got = oracle.window_attention(kp, vp, q, bt, lens, k_fp, v_fp, 4, 16, 32)
    for b, L in enumerate(lens):
        for hq in range(4):
            s = k_fp[b, :L, hq // 2].astype(np.float64) @ q[b, hq].astype(np.float64) / np.sqrt(128)
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ v_fp[b, :L, hq // 2].astype(np.float64)
            np.testing.assert_allclose(got[b, hq], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("pending", [0, 1])
@pytest.mark.parametrize("with_t", [False, True])
def test_mixed_window_matches_torch(pending, with_t):
    rng = np.random.default_rng(9 + pending + 2 * with_t)
    sink, keep, flush = 3, 20, 16
    lens = [3, 39, 40, 100, 171, 55]
    H, G = 2, 3
    t = tinv = None
    if with_t:
        t = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] * 1.3 + 0.05 * rng.standard_normal((128, 128))
                      for _ in range(H)]).astype(np.float32)
        tinv = np.stack([np.linalg.inv(x.astype(np.float64)).T for x in t]).astype(np.float32)
    kp, vp, bt, k_fp, v_fp, q = _setup(rng, len(lens), H, G, lens, sink, keep, flush, bits=(4, 2), t=t)
    got = oracle.window_attention(kp, vp, q, bt, lens, k_fp, v_fp, sink, keep, flush, pending=pending,
                                  t_inv_t=tinv, bits_k=4, bits_v=2)
    ref = _torch_reference(kp, vp, bt, k_fp, v_fp, q, lens, sink, keep, flush, pending, tinv, (4, 2))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-9)


def test_pending_reads_the_state_before_the_flush():
    rng = np.random.default_rng(11)
    sink, keep, flush = 2, 3, 4
    lens = [9, 10]              # 9 = the length whose arrival quantizes positions 2-5
    kp, vp, bt, k_fp, v_fp, q = _setup(rng, 2, 1, 2, lens, sink, keep, flush)
    a = oracle.window_attention(kp, vp, q, bt, lens, k_fp, v_fp, sink, keep, flush, pending=1)
    b = oracle.window_attention(kp, vp, q, bt, lens, k_fp, v_fp, sink, keep, flush, pending=0)
    assert np.abs(a[0] - b[0]).max() > 1e-3      # before / after the flush at length 9
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=0)   # no flush between lengths 9 and 10
