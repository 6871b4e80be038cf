"""End-to-end parity at the full sizes of the batch-64 x 16K and batch-16 x 128K workloads.

The GPU write path fills the whole cache (every sequence, all KV heads, with the dense key
transform) and the GPU decode runs in the launch configuration the benchmark times.  For
a seeded sample of sequences the oracle repeats the write from the same inputs and the
decode, and:
  * value pages are bit-identical; key codes differ on <= 1e-4 of elements (fp32 vs fp64
    accumulation of k . T); scale/zero differ by at most one fp16 ulp on <= 2e-4 of groups
    (measured 4.6e-5 to 1.07e-4 per sequence);
  * the GPU output matches the oracle's decode of the GPU-written pages, and the oracle's
    write + decode, within 2e-3 per (sequence, query head) row.
Then one decode step (kvq_decode_step) in the benchmark's configuration: a new token
rewrites every sequence's last position and takes part at full precision (the
long-context workload splits its sequences; the append blocks ride in the split launch).  The sampled sequences' value pages equal the oracle's
append of the same token into its pages bit for bit, and the output is within 2e-3 of the
oracle's step over the GPU's pages and over its own pages.
Write path: "WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms" §4.2, §4.3
(QuEST, alpha = 2.83, on the long-context workload) and §5.3 (percentile 1%/99%); read
path: §4.1, §4.2; long contexts as in its App. D.3.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kvq_amd import api, calib, synth
from helpers import (f16_ulp_distance, oracle_append_sequence, oracle_decode_sequence, oracle_step_sequence,
                     pool_codes, pool_scales_zeros, row_rel_err, SCALE_ZERO_RATE)

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _transforms(config, H, G):
    ts, tis = [], []
    for h in range(H):
        kc, qc = synth.calibration_set(config, h, G)
        t, ti = calib.calibrate_key_transform(kc, qc, store_bf16=True)
        ts.append(t)
        tis.append(ti)
    return np.stack(ts), np.stack(tis)


@pytest.mark.parametrize("name,samples", [("qwen3-8b-b64-16k", 2), ("long-b16-128k-quest", 1)])
def test_full_size_end_to_end(name, samples):
    w = synth.WORKLOADS[name]
    H, G, B, n, pps = w.heads_kv, w.group, w.batch, w.seq_len, w.pages_per_seq
    dev = torch.device("cuda")
    rng = np.random.default_rng(31 + w.config)
    picks = sorted(rng.choice(B, samples, replace=False).tolist())
    print(f"{name}: sampled sequences {picks}", flush=True)
    t, tinv = _transforms(w.config, H, G)
    qcode = oracle.RMS if w.quantizer == "rms" else oracle.PERCENTILE
    cache = api.KVCache(B * pps, H, w.bits_k, w.bits_v, w.quantizer, w.quantizer, w.p_lo, w.p_hi,
                        w.alpha, w.alpha, device=dev)
    bt = synth.contiguous_block_table(B, pps)
    t_dev = torch.from_numpy(t).to(torch.bfloat16).to(dev)
    kept = {}
    for b in range(B):                                  # one prompt-sized append per sequence
        k, v = synth.kv_tokens_torch(w, n, dev, seq=b)
        slots = torch.from_numpy(synth.slots_for(bt[b:b + 1], [n])).to(dev)
        api.kvq_quantize_append(cache, k, v, slots, t_k=t_dev)
        if b in picks:
            kept[b] = (k.float().cpu().numpy(), v.float().cpu().numpy())
    q = synth.decode_queries(w)
    seq = np.full(B, n, np.int32)
    q_dev, bt_dev, seq_dev = (torch.from_numpy(q).to(torch.bfloat16).to(dev), torch.from_numpy(bt).to(dev),
                              torch.from_numpy(seq).to(dev))
    tinv_dev = torch.from_numpy(tinv).to(dev)
    out = api.kvq_decode_attn(cache, q_dev, bt_dev, seq_dev, n, t_k_inv_t=tinv_dev)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    oracle_pools = {}
    for b in picks:
        pages = bt[b]
        gk = cache.k_pages[torch.from_numpy(pages).long().to(dev)].cpu().numpy()
        gv = cache.v_pages[torch.from_numpy(pages).long().to(dev)].cpu().numpy()
        kp, vp = oracle.new_pool(pps, H, w.bits_k), oracle.new_pool(pps, H, w.bits_v)
        local = synth.slots_for(np.arange(pps, dtype=np.int32)[None], [n])
        k, v = kept[b]
        oracle_append_sequence(kp, vp, k, v, local, t_k=t, bits_k=w.bits_k, bits_v=w.bits_v, quant_k=qcode,
                               quant_v=qcode, p_lo=w.p_lo, p_hi=w.p_hi, alpha_k=w.alpha, alpha_v=w.alpha)
        assert np.array_equal(gv, vp), b
        sample = local[::5]
        gc, _, _ = pool_codes(gk, 0, w.bits_k, sample)
        oc, _, _ = pool_codes(kp, 0, w.bits_k, sample)
        flips = np.mean(gc != oc)
        gs, gz = pool_scales_zeros(gk, w.bits_k, local)      # every group of the sequence
        os_, oz = pool_scales_zeros(kp, w.bits_k, local)
        mism = np.mean((gs != os_) | (gz != oz))
        print(f"  sequence {b}: key flips {flips:.2e}, scale/zero mismatches {mism:.2e}", flush=True)
        assert flips <= 1e-4 and mism <= SCALE_ZERO_RATE, (b, flips, mism)
        assert np.all(f16_ulp_distance(gs, os_) <= 1) and np.all(f16_ulp_distance(gz, oz) <= 1)
        all_pages = np.arange(pps)
        ref_g = oracle_decode_sequence(gk, gv, q[b], all_pages, n, t_inv_t=tinv, bits_k=w.bits_k, bits_v=w.bits_v)
        ref = oracle_decode_sequence(kp, vp, q[b], all_pages, n, t_inv_t=tinv, bits_k=w.bits_k, bits_v=w.bits_v)
        e_g = row_rel_err(got[b], ref_g).max()
        e = row_rel_err(got[b], ref).max()
        print(f"  sequence {b}: row-relative error vs oracle on GPU pages {e_g:.2e}, end to end {e:.2e}", flush=True)
        assert e_g <= TOL and e <= TOL, (b, e_g, e)
        oracle_pools[b] = (kp, vp)

    # the step: each sequence's new token rewrites its last position
    knew, vnew = synth.kv_tokens_torch(w, B, dev, seq=10_000)
    new_slots = np.array([bt[b, (n - 1) // 64] * 64 + (n - 1) % 64 for b in range(B)], np.int64)
    need = api.decode_step_workspace_bytes(cache, B, w.heads_q, n)
    assert need == api.decode_workspace_bytes(cache, B, w.heads_q, n)
    assert (need > 0) == (name == "long-b16-128k-quest")             # the long workload splits
    ws = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
    out = api.kvq_decode_step(cache, q_dev, knew, vnew, torch.from_numpy(new_slots).to(dev), bt_dev, seq_dev, n,
                              t_k=t_dev, t_k_inv_t=tinv_dev, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    kn, vn = knew.float().cpu().numpy(), vnew.float().cpu().numpy()
    for b in picks:
        pages = bt[b]
        gk = cache.k_pages[torch.from_numpy(pages).long().to(dev)].cpu().numpy()
        gv = cache.v_pages[torch.from_numpy(pages).long().to(dev)].cpu().numpy()
        kp, vp = oracle_pools[b]
        oracle.append(kp, vp, kn[b:b + 1], vn[b:b + 1], np.array([n - 1], np.int64), t_k=t, bits_k=w.bits_k,
                      bits_v=w.bits_v, quant_k=qcode, quant_v=qcode, p_lo=w.p_lo, p_hi=w.p_hi, alpha_k=w.alpha,
                      alpha_v=w.alpha)
        assert np.array_equal(gv, vp), b
        all_pages = np.arange(pps)
        ref_g = oracle_step_sequence(gk, gv, q[b], all_pages, n, kn[b], vn[b], t_inv_t=tinv, bits_k=w.bits_k,
                                     bits_v=w.bits_v)
        ref = oracle_step_sequence(kp, vp, q[b], all_pages, n, kn[b], vn[b], t_inv_t=tinv, bits_k=w.bits_k,
                                   bits_v=w.bits_v)
        e_g = row_rel_err(got[b], ref_g).max()
        e = row_rel_err(got[b], ref).max()
        print(f"  step, sequence {b}: row-relative error vs oracle on GPU pages {e_g:.2e}, end to end {e:.2e}",
              flush=True)
        assert e_g <= TOL and e <= TOL, (b, e_g, e)
