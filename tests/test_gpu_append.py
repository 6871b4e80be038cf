"""GPU parity of the write path (kvq_quantize_append) and of kvq_dequant against the
CPU oracle, through the C ABI.

Stage A: fp32 inputs, no transform -> packed pools bit-identical to the oracle's,
         including every byte the call must not touch.
Stage B: bf16/f16 inputs with a dense transform on the matrix cores -> value codes
         bit-identical, key codes differ on <= 1e-4 of elements (fp32 vs fp64
         accumulation), scale/zero off by at most one fp16 ulp on few groups;
         the identity transform is bit-identical to no transform.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from decode_attention_kvq_amd import api, calib, synth
from helpers import describe_mismatch, f16_ulp_distance, pool_codes, rms_order_rows, rare_event_bound

pytestmark = pytest.mark.gpu

QMAP = {"percentile": oracle.PERCENTILE, "rms": oracle.RMS}


def _tie_row(levels):
    """A group whose 1%/99% clip bounds are exactly 0 and L (three of each), so the scale is
    1 and every other value k + 1/2 lands exactly halfway between two codes: the rounding
    must go to the even code."""
    mids = [k + 0.5 for k in range(levels)]
    row = [0.0] * 3 + [float(levels)] * 3 + [mids[i % levels] for i in range(122)]
    return np.array(row, dtype=np.float32)


def _special_rows(x, rng):
    """Overwrite some token rows with edge cases: constant, zeros, +-0, integers, heavy
    tails, tiny and huge magnitudes, exact rounding ties at 2, 3 and 4 bits, and groups
    whose RMS bound depends on the order of the sum of squares."""
    n = x.shape[0]
    if n > 8:
        x[1] = 0.37
        x[2] = 0.0
        x[3, :, ::2] = -0.0
        x[4] = np.round(x[4])
        x[5] = rng.standard_t(1.5, size=x[5].shape)
        x[6] *= 1e-6
        x[7] *= 300.0
    if n > 11:
        x[8] = _tie_row(3)
        x[9] = _tie_row(7)
        x[10] = _tie_row(15)
    if n > 13:
        rows, _ = rms_order_rows()       # sums of squares that depend on the tree's order
        x[11] = rows[0]
        x[12] = rows[1]
    return x


def _inputs(n, H, rng, dtype="f32", config=0):
    w = synth.Workload("t", config, H, H, 1, n, 2, 2, "percentile", dtype, False)
    k, v = synth.kv_tokens(w, n)
    k = _special_rows(k.astype(np.float32), rng)
    v = _special_rows(v.astype(np.float32), rng)
    return synth.to_dtype(k, dtype), synth.to_dtype(v, dtype)


def _run_both(k, v, slots, num_pages, H, bits, quant, rng, t=None, t_oracle="same",
              p=(0.01, 0.99), torch_dtype=torch.float32):
    kp = oracle.new_pool(num_pages, H, bits[0], rng=rng)
    vp = oracle.new_pool(num_pages, H, bits[1], rng=rng)
    cache = api.KVCache(num_pages, H, bits[0], bits[1], quant[0], quant[1], p[0], p[1],
                        k_pages=torch.from_numpy(kp.copy()).cuda(),
                        v_pages=torch.from_numpy(vp.copy()).cuda())
    kt = torch.from_numpy(k).to(torch_dtype).cuda()
    vt = torch.from_numpy(v).to(torch_dtype).cuda()
    tt = None if t is None else torch.from_numpy(t).to(torch_dtype).cuda()
    api.kvq_quantize_append(cache, kt, vt, torch.from_numpy(slots).cuda(), t_k=tt)
    torch.cuda.synchronize()
    t_or = t if t_oracle == "same" else t_oracle
    oracle.append(kp, vp, k, v, slots, t_k=t_or, bits_k=bits[0], bits_v=bits[1],
                  quant_k=QMAP[quant[0]], quant_v=QMAP[quant[1]], p_lo=p[0], p_hi=p[1])
    return cache.k_pages.cpu().numpy(), cache.v_pages.cpu().numpy(), kp, vp


# Batches of up to 512 tokens take the one-token-per-workgroup path, larger ones the
# 128-token-tile path: each test runs a size on both sides of that boundary.
@pytest.mark.parametrize("n", [300, 700])
@pytest.mark.parametrize("bits", [(2, 2), (4, 4), (2, 4), (3, 3), (3, 2), (4, 3)])
@pytest.mark.parametrize("quant", [("percentile", "percentile"), ("rms", "rms"), ("percentile", "rms")])
@pytest.mark.parametrize("layout", ["aligned", "scattered"])
def test_stage_a_bit_exact(bits, quant, layout, n):
    rng = np.random.default_rng(zlib.crc32(repr((bits, quant, layout, n)).encode()))
    H = 2                              # n = 700: 6 tile workgroups, ragged last wave
    num_pages = n // 64 + 4
    k, v = _inputs(n, H, rng)
    if layout == "aligned":
        slots = np.arange(n, dtype=np.int64) + 64      # page 1 onwards, 32-token aligned
    else:
        slots = rng.permutation(num_pages * 64)[:n].astype(np.int64)
        slots[::17] = -1                                 # skipped tokens
    gk, gv, ok, ov = _run_both(k, v, slots, num_pages, H, bits, quant, rng)
    assert np.array_equal(gk, ok), describe_mismatch(gk, ok)
    assert np.array_equal(gv, ov), describe_mismatch(gv, ov)


@pytest.mark.parametrize("n", [100, 600])
@pytest.mark.parametrize("p", [(0.05, 0.9), (0.25, 0.75), (0.0, 1.0), (1.0, 1.0)])
def test_stage_a_other_percentiles(p, n):
    """Selection networks of width 8 and the bitonic-sort paths."""
    rng = np.random.default_rng(11)
    H = 1
    k, v = _inputs(n, H, rng)
    slots = np.arange(n, dtype=np.int64)
    gk, gv, ok, ov = _run_both(k, v, slots, n // 64 + 1, H, (4, 2), ("percentile", "percentile"), rng, p=p)
    assert np.array_equal(gk, ok), describe_mismatch(gk, ok)
    assert np.array_equal(gv, ov), describe_mismatch(gv, ov)


def test_append_one_token_at_a_time_preserves_neighbours():
    """Decode-style appends: one token per sequence per call into partly filled pages."""
    rng = np.random.default_rng(12)
    H, B, steps = 2, 5, 40
    k, v = _inputs(B * steps, H, rng)
    kp = oracle.new_pool(B * 2, H, 2, rng=rng)
    vp = oracle.new_pool(B * 2, H, 2, rng=rng)
    cache = api.KVCache(B * 2, H, 2, 2, k_pages=torch.from_numpy(kp.copy()).cuda(),
                        v_pages=torch.from_numpy(vp.copy()).cuda())
    for s in range(steps):
        idx = np.arange(B) * steps + s
        slots = (np.arange(B) * 2 * 64 + 30 + s).astype(np.int64)   # crosses a page boundary
        api.kvq_quantize_append(cache, torch.from_numpy(k[idx]).cuda(), torch.from_numpy(v[idx]).cuda(),
                                torch.from_numpy(slots).cuda())
        oracle.append(kp, vp, k[idx], v[idx], slots, bits_k=2, bits_v=2)
    torch.cuda.synchronize()
    assert np.array_equal(cache.k_pages.cpu().numpy(), kp)
    assert np.array_equal(cache.v_pages.cpu().numpy(), vp)


@pytest.mark.parametrize("n", [512, 1024])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("bits", [(2, 2), (4, 4), (3, 3)])
def test_stage_b_transform_on_matrix_cores(dtype, bits, n):
    """n = 512: fp32 transform, one token per workgroup; n = 1024: matrix-core transform."""
    rng = np.random.default_rng(13)
    H, G = 2, 4
    k, v = _inputs(n, H, rng, dtype=dtype, config=1)
    ts = []
    for h in range(H):
        kc, qc = synth.calibration_set(1, h, G)
        ts.append(calib.calibrate_key_transform(kc, qc)[0])
    t = np.stack(ts)
    if dtype == "f16":
        t = t.astype(np.float16).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    slots = np.arange(n, dtype=np.int64)
    gk, gv, ok, ov = _run_both(k, v, slots, n // 64, H, bits, ("percentile", "percentile"), rng,
                               t=t, torch_dtype=tdt)
    assert np.array_equal(gv, ov), describe_mismatch(gv, ov)
    gc, gs, gz = pool_codes(gk, 0, bits[0], slots)
    oc, os_, oz = pool_codes(ok, 0, bits[0], slots)
    flips = np.mean(gc != oc)
    assert flips <= 1e-4 or np.sum(gc != oc) <= 2, flips
    bad = (gs != os_) | (gz != oz)
    assert np.sum(bad) <= rare_event_bound(bad.size), np.sum(bad)
    assert np.all(f16_ulp_distance(gs, os_) <= 1) and np.all(f16_ulp_distance(gz, oz) <= 1)


@pytest.mark.parametrize("n", [200, 600])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_identity_transform_is_bit_exact(dtype, n):
    rng = np.random.default_rng(14)
    H = 2
    k, v = _inputs(n, H, rng, dtype=dtype)
    eye = np.broadcast_to(np.eye(128, dtype=np.float32), (H, 128, 128)).copy()
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    gk, gv, ok, ov = _run_both(k, v, np.arange(n, dtype=np.int64), n // 64 + 1, H, (2, 2),
                               ("percentile", "rms"), rng, t=eye, t_oracle=None, torch_dtype=tdt)
    assert np.array_equal(gk, ok), describe_mismatch(gk, ok)
    assert np.array_equal(gv, ov), describe_mismatch(gv, ov)


def test_f32_transform_tiny_config():
    """The tiny workload: fp32 keys with an fp32 transform (fp32 arithmetic on the GPU)."""
    w = synth.WORKLOADS["tiny"]
    rng = np.random.default_rng(15)
    k, v = synth.kv_tokens(w, w.seq_len)
    kc, qc = synth.calibration_set(0, 0, 1)
    t = calib.calibrate_key_transform(kc, qc, store_bf16=False)[0][None]
    slots = np.arange(w.seq_len, dtype=np.int64)
    gk, gv, ok, ov = _run_both(k, v, slots, 4, 1, (4, 4), ("percentile", "percentile"), rng, t=t)
    assert np.array_equal(gv, ov)
    gc, _, _ = pool_codes(gk, 0, 4, slots)
    oc, _, _ = pool_codes(ok, 0, 4, slots)
    assert np.sum(gc != oc) <= 4, np.sum(gc != oc)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("which", [0, 1])
def test_dequant_bit_exact(bits, which):
    rng = np.random.default_rng(16 + bits + which)
    H, P = 3, 5
    pool = synth.random_packed_pool(rng, P, H, bits)
    slots = np.concatenate([rng.permutation(P * 64)[:150], [-1]]).astype(np.int64)
    kp = pool if which == 0 else oracle.new_pool(P, H, bits)
    vp = pool if which == 1 else oracle.new_pool(P, H, bits)
    cache = api.KVCache(P, H, bits, bits, k_pages=torch.from_numpy(kp).cuda(),
                        v_pages=torch.from_numpy(vp).cuda())
    got = api.kvq_dequant(cache, which, torch.from_numpy(slots).cuda()).cpu().numpy()
    ref = oracle.dequant(pool, which, bits, slots)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("bits", [4, 2, 3])
def test_bulk_prefill_full_size_sampled(bits):
    """Bulk prefill: 8 KV heads x 32768 tokens, bf16, dense transform on the matrix cores
    (3-bit: the two-plane kernel).  The oracle re-encodes a seeded sample of 1024 tokens
    (all heads)."""
    w = synth.WORKLOADS["prefill-8x32k-%dbit" % bits]
    n, H = w.seq_len, w.heads_kv
    dev = torch.device("cuda")
    k, v = synth.kv_tokens_torch(w, n, dev)
    ts = []
    for h in range(H):
        kc, qc = synth.calibration_set(w.config, h, 4)
        ts.append(calib.calibrate_key_transform(kc, qc)[0])
    t = np.stack(ts)
    cache = api.KVCache(n // 64, H, bits, bits)
    slots = torch.arange(n, dtype=torch.int64, device=dev)
    api.kvq_quantize_append(cache, k, v, slots, t_k=torch.from_numpy(t).to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(17)
    sample = np.sort(rng.choice(n, 1024, replace=False))
    ks = k[torch.from_numpy(sample).cuda()].float().cpu().numpy()
    vs = v[torch.from_numpy(sample).cuda()].float().cpu().numpy()
    kt = oracle.transform_keys(ks, t)
    pages = torch.from_numpy(sample // 64).cuda()
    gk = cache.k_pages[pages].cpu().numpy()
    gv = cache.v_pages[pages].cpu().numpy()
    local = (sample % 64).astype(np.int64) + 64 * np.arange(len(sample))
    gkc, gks, gkz = pool_codes(gk, 0, bits, local)
    gvc, gvs, gvz = pool_codes(gv, 1, bits, local)
    for h in range(H):
        oc, os_, oz, _, _ = oracle.quantize_rows(vs[:, h], bits)
        assert np.array_equal(gvc[:, h], oc) and np.array_equal(gvs[:, h], os_) and np.array_equal(gvz[:, h], oz)
        oc, os_, oz, _, _ = oracle.quantize_rows(kt[:, h], bits)
        assert np.mean(gkc[:, h] != oc) <= 1e-4 or np.sum(gkc[:, h] != oc) <= 2
        assert np.all(f16_ulp_distance(gks[:, h], os_) <= 1) and np.all(f16_ulp_distance(gkz[:, h], oz) <= 1)
