"""GPU parity at the limits of the launch shapes: the largest batch a decode launch takes
(65535 sequences, the grid's z extent), many KV heads, and windows whose full-precision part
spans many tiles.  Compared with the CPU oracle on seeded samples, ≤ 2e-3 per row."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kvq_amd import api, synth
from helpers import row_rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-3


def test_max_batch_ragged_and_empty():
    rng = np.random.default_rng(65535)
    B, H, G, pps = 65535, 1, 4, 2
    seq = rng.integers(0, 2 * 64 + 1, B).astype(np.int32)
    seq[::97] = 0                                   # empty sequences
    kp = synth.random_packed_pool(rng, B * pps, H, 2)
    vp = synth.random_packed_pool(rng, B * pps, H, 2)
    bt = rng.permutation(B * pps).astype(np.int32).reshape(B, pps)
    q = synth.to_dtype(rng.standard_normal((B, H * G, 128)).astype(np.float32), "bf16")
    cache = api.KVCache(B * pps, H, 2, 2, k_pages=torch.from_numpy(kp).cuda(), v_pages=torch.from_numpy(vp).cuda())
    out = api.kvq_decode_attn(cache, torch.from_numpy(q).to(torch.bfloat16).cuda(), torch.from_numpy(bt).cuda(),
                              torch.from_numpy(seq).cuda(), 2 * 64)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[seq == 0] == 0)
    sample = np.sort(np.concatenate([rng.choice(B, 150, replace=False), [0, B - 1]]))
    ref = oracle.decode_attention(kp, vp, q[sample], bt[sample], seq[sample], bits_k=2, bits_v=2)
    nonempty = seq[sample] > 0
    assert row_rel_err(got[sample][nonempty], ref[nonempty]).max() <= TOL


def test_many_kv_heads():
    rng = np.random.default_rng(64)
    B, H, G = 3, 64, 2
    seq = np.array([300, 1, 129], np.int32)
    pps = 5
    kp = synth.random_packed_pool(rng, B * pps, H, 4)
    vp = synth.random_packed_pool(rng, B * pps, H, 2)
    bt = synth.shuffled_block_table(B, pps, B * pps, rng)
    q = synth.to_dtype(rng.standard_normal((B, H * G, 128)).astype(np.float32), "f16")
    cache = api.KVCache(B * pps, H, 4, 2, k_pages=torch.from_numpy(kp).cuda(), v_pages=torch.from_numpy(vp).cuda())
    out = api.kvq_decode_attn(cache, torch.from_numpy(q).to(torch.float16).cuda(), torch.from_numpy(bt).cuda(),
                              torch.from_numpy(seq).cuda(), 300)
    torch.cuda.synchronize()
    ref = oracle.decode_attention(kp, vp, q, bt, seq, bits_k=4, bits_v=2)
    assert row_rel_err(out.cpu().numpy(), ref).max() <= TOL


def test_window_spanning_many_tiles():
    """S_sink 700 + S_keep 1000 + S_flush 400: up to 2099 full-precision positions (17 tiles
    of the window kernel) next to the quantized middle."""
    rng = np.random.default_rng(2099)
    sink, keep, flush = 700, 1000, 400
    B, H, G = 3, 2, 4
    lens = np.array([2099, 5000, 650], np.int32)
    fp_len = int(lens.max())
    pps = -(-(fp_len - sink) // 64)
    num_pages = B * pps + 1
    kp = synth.random_packed_pool(rng, num_pages, H, 2)
    vp = synth.random_packed_pool(rng, num_pages, H, 2)
    bt = synth.shuffled_block_table(B, pps, num_pages, rng)
    W = sink + keep + flush
    kw = synth.to_dtype(rng.standard_normal((B, W, H, 128)).astype(np.float32), "bf16")
    vw = synth.to_dtype(rng.standard_normal((B, W, H, 128)).astype(np.float32), "bf16")
    cache = api.KVCache(num_pages, H, 2, 2, k_pages=torch.from_numpy(kp).cuda(), v_pages=torch.from_numpy(vp).cuda())
    win = api.Window(cache, B, sink, keep, flush, k_win=torch.from_numpy(kw).to(torch.bfloat16).cuda(),
                     v_win=torch.from_numpy(vw).to(torch.bfloat16).cuda())
    q = synth.to_dtype(rng.standard_normal((B, H * G, 128)).astype(np.float32), "bf16")
    out = api.kvq_window_decode_attn(cache, win, torch.from_numpy(q).to(torch.bfloat16).cuda(),
                                     torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(), fp_len)
    torch.cuda.synchronize()
    hk = np.zeros((B, fp_len, H, 128), np.float32)
    hv = np.zeros_like(hk)
    for b, L in enumerate(lens):
        nq = oracle.window_quantized(int(L), sink, keep, flush)
        for p in list(range(min(L, sink))) + list(range(sink + nq, L)):
            slot = p if p < sink else sink + (p - sink) % (keep + flush)
            hk[b, p], hv[b, p] = kw[b, slot], vw[b, slot]
    ref = oracle.window_attention(kp, vp, q, bt, lens, hk, hv, sink, keep, flush)
    assert row_rel_err(out.cpu().numpy(), ref).max() <= TOL


def test_long_sequences_merge_over_many_chunk_blocks():
    """Two sequences of 1,000,000 and 300,000 tokens, 2 KV heads: the launch splits every
    sequence into 127 chunks, so the merge runs over a full block of 64 chunks and a partial
    one of 63, and for the shorter sequence the second block holds no tokens at all."""
    rng = np.random.default_rng(1_000_000)
    B, H, G = 2, 2, 4
    seq = np.array([1_000_000, 300_000], np.int32)
    pps = -(-int(seq.max()) // 64)
    num_pages = B * pps
    kp = synth.random_packed_pool(rng, num_pages, H, 2)
    vp = synth.random_packed_pool(rng, num_pages, H, 2)
    bt = synth.shuffled_block_table(B, pps, num_pages, rng)
    q = synth.to_dtype(rng.standard_normal((B, H * G, 128)).astype(np.float32), "bf16")
    cache = api.KVCache(num_pages, H, 2, 2, k_pages=torch.from_numpy(kp).cuda(), v_pages=torch.from_numpy(vp).cuda())
    assert api.decode_workspace_bytes(cache, B, H * G, int(seq.max())) >= B * H * G * 127 * (128 + 2) * 4
    out = api.kvq_decode_attn(cache, torch.from_numpy(q).to(torch.bfloat16).cuda(), torch.from_numpy(bt).cuda(),
                              torch.from_numpy(seq).cuda(), int(seq.max()))
    torch.cuda.synchronize()
    ref = oracle.decode_attention(kp, vp, q, bt, seq, bits_k=2, bits_v=2)
    assert row_rel_err(out.cpu().numpy(), ref).max() <= TOL
