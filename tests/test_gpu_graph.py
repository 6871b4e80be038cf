"""The hot path under HIP-graph capture: one step (append of each sequence's new token,
then decode over the whole cache) captured once and replayed several times, with the
program's own eager work and synchronizations between replays.  Every replay must give
the eager result bit for bit (same kernels, same inputs), and the eager result must
match the CPU oracle.  A sequence long enough to be split over several workgroups makes
the merge kernel part of the graph too.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kvq_amd import api, calib, synth
from helpers import row_rel_err

pytestmark = pytest.mark.gpu


def _setup(seq_lens):
    rng = np.random.default_rng(31)
    B, H, G = len(seq_lens), 2, 4
    seq = np.array(seq_lens, np.int32)
    pps = int(-(-seq.max() // 64))
    num_pages = B * pps + 2
    bt = synth.shuffled_block_table(B, pps, num_pages, rng)
    w = synth.Workload("g", 1, H * G, H, B, int(seq.max()), 2, 2, "percentile", "bf16", True)
    ts, tis = zip(*[calib.calibrate_key_transform(*synth.calibration_set(1, h, G)) for h in range(H)])
    t_k, t_inv = np.stack(ts), np.stack(tis)
    # the cache holds every token but each sequence's last one, which the step appends
    prior = seq - 1
    slots_prior = synth.slots_for(bt, prior)
    k, v = synth.kv_tokens(w, int(seq.sum()))
    offs = np.concatenate([[0], np.cumsum(seq)])
    last = offs[1:] - 1
    keep = np.setdiff1d(np.arange(int(seq.sum())), last)
    kp = oracle.new_pool(num_pages, H, 2, rng=rng)
    vp = oracle.new_pool(num_pages, H, 2, rng=rng)
    oracle.append(kp, vp, k[keep], v[keep], slots_prior, t_k=t_k.astype(np.float32), bits_k=2, bits_v=2)
    new_slots = np.array([bt[b, (seq[b] - 1) // 64] * 64 + (seq[b] - 1) % 64 for b in range(B)], np.int64)
    q = synth.decode_queries(w)
    return dict(kp=kp, vp=vp, bt=bt, seq=seq, k_new=k[last], v_new=v[last], new_slots=new_slots,
                q=q, t_k=t_k, t_inv=t_inv, H=H, w=w)


def test_graph_replays_match_eager_and_oracle():
    d = _setup([200, 2900, 64, 1])
    dev = torch.device("cuda")
    H = d["H"]
    cache = api.KVCache(d["kp"].shape[0], H, 2, 2, k_pages=torch.from_numpy(d["kp"]).to(dev),
                        v_pages=torch.from_numpy(d["vp"]).to(dev))
    kp0, vp0 = cache.k_pages.clone(), cache.v_pages.clone()
    t_k = torch.from_numpy(d["t_k"]).to(torch.bfloat16).to(dev)
    t_inv = torch.from_numpy(d["t_inv"]).to(dev)
    knew = torch.from_numpy(d["k_new"]).to(torch.bfloat16).to(dev)
    vnew = torch.from_numpy(d["v_new"]).to(torch.bfloat16).to(dev)
    slots = torch.from_numpy(d["new_slots"]).to(dev)
    bt = torch.from_numpy(d["bt"]).to(dev)
    seq = torch.from_numpy(d["seq"]).to(dev)
    q = torch.from_numpy(d["q"]).to(torch.bfloat16).to(dev)
    msl = int(d["seq"].max())
    B, Hq = q.shape[0], q.shape[1]
    ws_bytes = api.decode_workspace_bytes(cache, B, Hq, msl)
    assert ws_bytes > 0, "the long sequence should be split (merge kernel in the graph)"
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)

    def step():
        api.kvq_quantize_append(cache, knew, vnew, slots, t_k=t_k)
        api.kvq_decode_attn(cache, q, bt, seq, msl, t_k_inv_t=t_inv, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager_out = out.clone()
    eager_k, eager_v = cache.k_pages.clone(), cache.v_pages.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        # reset the cache to its pre-step bytes and scribble over the output and workspace
        # with eager work, so each replay has to recompute everything it reports
        cache.k_pages.copy_(kp0)
        cache.v_pages.copy_(vp0)
        out.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cache.k_pages, eager_k), f"replay {r}: K pool differs from eager"
        assert torch.equal(cache.v_pages, eager_v), f"replay {r}: V pool differs from eager"
        assert torch.equal(out, eager_out), f"replay {r}: output differs from eager"

    # and the eager step itself agrees with the oracle's write + read of the same step
    kp, vp = d["kp"].copy(), d["vp"].copy()
    oracle.append(kp, vp, d["k_new"], d["v_new"], d["new_slots"], t_k=d["t_k"].astype(np.float32),
                  bits_k=2, bits_v=2)
    ref = oracle.decode_attention(kp, vp, d["q"], d["bt"], d["seq"], t_inv_t=d["t_inv"], bits_k=2, bits_v=2)
    err = row_rel_err(eager_out.cpu().numpy(), ref)
    assert err.max() <= 2e-3, err.max()


def test_graph_replays_of_the_split_step():
    """kvq_decode_step on a split decode: the decode launch (with the append blocks) writes
    the chunks' partials into the workspace, and the merge launch reads them.  Captured once and replayed with the workspace scribbled over in
    between, every replay equals the eager step bit for bit, and the eager step matches the
    oracle's step."""
    d = _setup([200, 2900, 64, 1])
    dev = torch.device("cuda")
    H = d["H"]
    cache = api.KVCache(d["kp"].shape[0], H, 2, 2, k_pages=torch.from_numpy(d["kp"]).to(dev),
                        v_pages=torch.from_numpy(d["vp"]).to(dev))
    kp0, vp0 = cache.k_pages.clone(), cache.v_pages.clone()
    t_k = torch.from_numpy(d["t_k"]).to(torch.bfloat16).to(dev)
    t_inv = torch.from_numpy(d["t_inv"]).to(dev)
    knew = torch.from_numpy(d["k_new"]).to(torch.bfloat16).to(dev)
    vnew = torch.from_numpy(d["v_new"]).to(torch.bfloat16).to(dev)
    slots = torch.from_numpy(d["new_slots"]).to(dev)
    bt = torch.from_numpy(d["bt"]).to(dev)
    seq = torch.from_numpy(d["seq"]).to(dev)
    q = torch.from_numpy(d["q"]).to(torch.bfloat16).to(dev)
    msl = int(d["seq"].max())
    B, Hq = q.shape[0], q.shape[1]
    need = api.decode_step_workspace_bytes(cache, B, Hq, msl)
    assert need == api.decode_workspace_bytes(cache, B, Hq, msl) > 0, "split decode"
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)

    def step():
        api.kvq_decode_step(cache, q, knew, vnew, slots, bt, seq, msl, t_k=t_k, t_k_inv_t=t_inv, out=out,
                            workspace=ws)

    step()
    torch.cuda.synchronize()
    eager_out = out.clone()
    eager_k, eager_v = cache.k_pages.clone(), cache.v_pages.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        cache.k_pages.copy_(kp0)
        cache.v_pages.copy_(vp0)
        out.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cache.k_pages, eager_k), f"replay {r}: K pool differs from eager"
        assert torch.equal(cache.v_pages, eager_v), f"replay {r}: V pool differs from eager"
        assert torch.equal(out, eager_out), f"replay {r}: output differs from eager"

    kp, vp = d["kp"].copy(), d["vp"].copy()
    oracle.append(kp, vp, d["k_new"], d["v_new"], d["new_slots"], t_k=d["t_k"].astype(np.float32),
                  bits_k=2, bits_v=2)
    ref = oracle.decode_step(kp, vp, d["q"], d["bt"], d["seq"], d["k_new"], d["v_new"], t_inv_t=d["t_inv"],
                             bits_k=2, bits_v=2)
    err = row_rel_err(eager_out.cpu().numpy(), ref)
    assert err.max() <= 2e-3, err.max()
