"""Pins of the oracle's decode attention (O7) against torch's fp64
scaled_dot_product_attention on the dequantized cache and closed-form special cases."""
import numpy as np
import pytest
import torch

from decode_attention_kvq_amd import synth


def _setup(orc, B=3, Hq=8, Hkv=2, bits=(2, 4), seq_lens=(130, 64, 1), seed=0, t=True):
    rng = np.random.default_rng(seed)
    pps = max(-(-n // 64) for n in seq_lens)
    num_pages = B * pps + 3
    kp = orc.new_pool(num_pages, Hkv, bits[0], rng=rng)
    vp = orc.new_pool(num_pages, Hkv, bits[1], rng=rng)
    bt = synth.shuffled_block_table(B, pps, num_pages, rng)
    seq = np.array(seq_lens, np.int32)
    slots = synth.slots_for(bt, seq)
    k = rng.standard_normal((len(slots), Hkv, 128)).astype(np.float32)
    v = rng.standard_normal((len(slots), Hkv, 128)).astype(np.float32)
    v[:, :, 5] += 3.0
    T = None
    if t:
        T = (np.eye(128) + 0.2 * rng.standard_normal((Hkv, 128, 128)) / np.sqrt(128)).astype(np.float32)
    orc.append(kp, vp, k, v, slots, t_k=T, bits_k=bits[0], bits_v=bits[1])
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32) * 2
    tinv = None if T is None else np.stack([np.linalg.inv(T[h].astype(np.float64)).T for h in range(Hkv)]).astype(np.float32)
    return kp, vp, bt, seq, slots, q, tinv


def _sdpa_reference(orc, kp, vp, bt, seq, q, tinv, bits):
    B, Hq, _ = q.shape
    Hkv = kp.shape[1]
    out = np.zeros((B, Hq, 128))
    for b in range(B):
        n = int(seq[b])
        sl = synth.slots_for(bt[b:b + 1], [n])
        kd = torch.tensor(orc.dequant(kp, 0, bits[0], sl), dtype=torch.float64)  # [n,Hkv,d]
        vd = torch.tensor(orc.dequant(vp, 1, bits[1], sl), dtype=torch.float64)
        qb = torch.tensor(q[b], dtype=torch.float64)                           # [Hq,d]
        if tinv is not None:
            qb = torch.stack([qb[h] @ torch.tensor(tinv[h // (Hq // Hkv)], dtype=torch.float64)
                              for h in range(Hq)])
        kk = kd.permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)         # [Hq,n,d]
        vv = vd.permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(qb[:, None, :], kk, vv)
        out[b] = o[:, 0, :].numpy()
    return out


@pytest.mark.parametrize("bits", [(2, 4), (3, 3), (3, 2)])
@pytest.mark.parametrize("t", [False, True])
def test_matches_torch_sdpa_fp64(orc, t, bits):
    kp, vp, bt, seq, _, q, tinv = _setup(orc, bits=bits, t=t)
    got = orc.decode_attention(kp, vp, q, bt, seq, t_inv_t=tinv, bits_k=bits[0], bits_v=bits[1])
    ref = _sdpa_reference(orc, kp, vp, bt, seq, q, tinv, bits)
    assert np.max(np.abs(got - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_single_token_and_zero_query(orc):
    bits = (4, 2)
    kp, vp, bt, seq, _, q, _ = _setup(orc, B=2, seq_lens=(1, 200), bits=bits, t=False)
    out = orc.decode_attention(kp, vp, q, bt, seq, bits_k=bits[0], bits_v=bits[1])
    v0 = orc.dequant(vp, 1, bits[1], synth.slots_for(bt[:1], [1]))[0]     # [Hkv,d]
    for hq in range(8):
        assert np.allclose(out[0, hq], v0[hq // 4], rtol=0, atol=1e-12)
    q0 = np.zeros_like(q)
    out0 = orc.decode_attention(kp, vp, q0, bt, seq, bits_k=bits[0], bits_v=bits[1])
    vall = orc.dequant(vp, 1, bits[1], synth.slots_for(bt[1:2], [200])).astype(np.float64)
    for hq in range(8):
        assert np.allclose(out0[1, hq], vall[:, hq // 4].mean(axis=0), rtol=0, atol=1e-12)


def test_split_lse_merge_equals_unsplit(orc):
    bits = (2, 2)
    kp, vp, bt, seq, _, q, tinv = _setup(orc, B=1, seq_lens=(300,), bits=bits)
    full, lse = orc.decode_attention(kp, vp, q, bt, seq, t_inv_t=tinv, bits_k=2, bits_v=2, return_lse=True)
    a = 128
    o1, l1 = orc.decode_attention(kp, vp, q, bt, np.array([a], np.int32), t_inv_t=tinv,
                                  bits_k=2, bits_v=2, return_lse=True)
    o2, l2 = orc.decode_attention(kp, vp, q, bt[:, a // 64:], np.array([300 - a], np.int32),
                                  t_inv_t=tinv, bits_k=2, bits_v=2, return_lse=True)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    merged = (w1[..., None] * o1 + w2[..., None] * o2) / (w1 + w2)[..., None]
    assert np.allclose(merged, full, rtol=0, atol=1e-12)
    assert np.allclose(m + np.log(w1 + w2), lse, rtol=0, atol=1e-12)


def test_empty_sequence_gives_zero(orc):
    kp, vp, bt, _, _, q, _ = _setup(orc, B=2, seq_lens=(64, 64), bits=(2, 2), t=False)
    out, lse = orc.decode_attention(kp, vp, q, bt, np.array([0, 64], np.int32), bits_k=2, bits_v=2,
                                    return_lse=True)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.any(out[1] != 0)


def test_values_do_not_move_probabilities(orc):
    """Values do not enter the softmax (WUSH-KV summary, App. C.5): re-encoding V changes
    the output only through the value rows, linearly."""
    bits = (2, 2)
    kp, vp, bt, seq, slots, q, _ = _setup(orc, B=1, seq_lens=(100,), bits=bits, t=False)
    out1 = orc.decode_attention(kp, vp, q, bt, seq, bits_k=2, bits_v=2)
    # a second value pool whose dequantized rows are all the unit vector e_7
    vp2 = vp.copy()
    for s in slots:
        p, o = divmod(int(s), 64)
        for h in range(vp.shape[1]):
            codes = np.zeros(128, np.uint8)
            codes[7] = 1
            orc.pack_token(vp2[p, h], 1, 2, o, codes, np.float16(1).view(np.uint16), 0)
    out2 = orc.decode_attention(kp, vp2, q, bt, seq, bits_k=2, bits_v=2)
    e7 = np.zeros(128)
    e7[7] = 1
    assert np.allclose(out2, e7, atol=1e-12)       # probabilities sum to one
    assert not np.allclose(out1, out2)


@pytest.mark.parametrize("t", [False, True])
def test_decode_step_matches_torch_sdpa_fp64(orc, t):
    """The step's attention: positions [0, L-1) from the cache, the new token from its own
    full-precision row; torch fp64 attention over the dequantized cache rows followed by the
    new row (with a key transform, the new key k_new T against q T^-T)."""
    bits = (2, 4)
    lens = (130, 64, 1, 0)
    kp, vp, bt, seq, _, q, tinv = _setup(orc, B=4, seq_lens=lens, bits=bits, t=t, seed=3)
    rng = np.random.default_rng(9)
    Hq, Hkv = q.shape[1], kp.shape[1]
    kn = rng.standard_normal((4, Hkv, 128)).astype(np.float32) * 1.5
    vn = rng.standard_normal((4, Hkv, 128)).astype(np.float32)
    got = orc.decode_step(kp, vp, q, bt, seq, kn, vn, t_inv_t=tinv, bits_k=bits[0], bits_v=bits[1])
    ref = np.zeros_like(got)
    for b, n in enumerate(lens):
        if n == 0:
            continue
        sl = synth.slots_for(bt[b:b + 1], [n - 1])
        kd = torch.tensor(orc.dequant(kp, 0, bits[0], sl), dtype=torch.float64)    # [n-1,Hkv,d]
        vd = torch.tensor(orc.dequant(vp, 1, bits[1], sl), dtype=torch.float64)
        knb = torch.tensor(kn[b], dtype=torch.float64)                             # [Hkv,d]
        qb = torch.tensor(q[b], dtype=torch.float64)
        if tinv is not None:
            tin = torch.tensor(tinv, dtype=torch.float64)
            tk = torch.linalg.inv(tin.transpose(1, 2))                             # T = (T^-T)^-T
            knb = torch.stack([knb[h] @ tk[h] for h in range(Hkv)])
            qb = torch.stack([qb[h] @ tin[h // (Hq // Hkv)] for h in range(Hq)])
        kk = torch.cat([kd, knb[None]], 0).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        vv = torch.cat([vd, torch.tensor(vn[b], dtype=torch.float64)[None]], 0).permute(1, 0, 2)
        vv = vv.repeat_interleave(Hq // Hkv, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(qb[:, None, :], kk, vv)
        ref[b] = o[:, 0, :].numpy()
    assert np.all(got[3] == 0)                                       # no tokens, no output
    assert np.allclose(got[2], np.repeat(vn[2], Hq // Hkv, axis=0), rtol=0, atol=1e-12)   # only the new token
    assert np.max(np.abs(got - ref)) < 1e-10 * max(1.0, np.max(np.abs(ref)))


def test_decode_step_equals_decode_when_the_new_row_is_the_cached_one(orc):
    """If the new token's row is exactly what the cache holds at position L-1 (no key
    transform), the step is the plain decode over [0, L)."""
    bits = (3, 2)
    kp, vp, bt, seq, _, q, _ = _setup(orc, B=3, seq_lens=(130, 64, 1), bits=bits, t=False, seed=5)
    last = np.array([synth.slots_for(bt[b:b + 1], [int(n)])[-1] for b, n in enumerate(seq)], np.int64)
    kn = orc.dequant(kp, 0, bits[0], last)
    vn = orc.dequant(vp, 1, bits[1], last)
    got = orc.decode_step(kp, vp, q, bt, seq, kn, vn, bits_k=bits[0], bits_v=bits[1])
    ref = orc.decode_attention(kp, vp, q, bt, seq, bits_k=bits[0], bits_v=bits[1])
    assert np.max(np.abs(got - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))
