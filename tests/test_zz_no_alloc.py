"""The allocation-free decode (kvq_decode_attn_noalloc) against kvq_decode_attn, through the
C ABI.  Two calls in a row on the library's scratch, the second with a smaller input; each
output must equal the workspace entry point's (same kernels, same split) and lie within 2e-3
of the oracle's attention (per (sequence, query head) row)."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kvq_amd import api, calib, synth
from helpers import row_rel_err

pytestmark = pytest.mark.gpu


def _case(rng, seq, H, G, bits):
    B = len(seq)
    pps = int(-(-max(seq) // 64))
    num_pages = B * pps + 2
    kp = oracle.new_pool(num_pages, H, bits[0], rng=rng)
    vp = oracle.new_pool(num_pages, H, bits[1], rng=rng)
    bt = synth.shuffled_block_table(B, pps, num_pages, rng)
    slots = synth.slots_for(bt, seq)
    w = synth.Workload("n", 1, H * G, H, B, len(slots), bits[0], bits[1], "percentile", "bf16", True)
    k, v = synth.kv_tokens(w, len(slots))
    ts, tis = zip(*[calib.calibrate_key_transform(*synth.calibration_set(1, h, G)) for h in range(H)])
    t, tinv = np.stack(ts), np.stack(tis)
    oracle.append(kp, vp, k, v, slots, t_k=t, bits_k=bits[0], bits_v=bits[1])
    q = synth.decode_queries(w)
    return kp, vp, bt, q, tinv


def test_noalloc_matches_workspace_entry_point():
    rng = np.random.default_rng(4242)
    calls = [(np.array([5000, 3333, 700], np.int32), 2, 4, (2, 2)),     # larger first
             (np.array([2000], np.int32), 2, 8, (4, 2))]                # then smaller
    for seq, H, G, bits in calls:
        kp, vp, bt, q, tinv = _case(rng, seq, H, G, bits)
        cache = api.KVCache(kp.shape[0], H, bits[0], bits[1], k_pages=torch.from_numpy(kp).cuda(),
                            v_pages=torch.from_numpy(vp).cuda())
        msl = int(seq.max())
        assert api.decode_workspace_bytes(cache, len(seq), H * G, msl) > 0    # the scratch is used
        qt = torch.from_numpy(q).to(torch.bfloat16).cuda()
        btt, st, ti = torch.from_numpy(bt).cuda(), torch.from_numpy(seq).cuda(), torch.from_numpy(tinv).cuda()
        out = torch.full((len(seq), H * G, 128), float("nan"), dtype=torch.float32, device="cuda")
        api.kvq_decode_attn_noalloc(cache, qt, btt, st, msl, out, t_k_inv_t=ti)
        ref_ws = api.kvq_decode_attn(cache, qt, btt, st, msl, t_k_inv_t=ti)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, ref_ws.cpu().numpy()), (seq, np.nanmax(np.abs(got - ref_ws.cpu().numpy())))
        ref = oracle.decode_attention(kp, vp, q, bt, seq, t_inv_t=tinv, bits_k=bits[0], bits_v=bits[1])
        assert row_rel_err(got, ref).max() <= 2e-3
