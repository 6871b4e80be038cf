"""GPU parity of the full-precision cache windows ("WUSH-KV" §4.4) against the CPU oracle,
through the C ABI: prefill (window store + quantize-append of the middle positions), the
windowed read, and decode steps (attention with the new position in full precision, then
the flush of the batch it made eligible).  Outputs within 2e-3 max relative error per
(sequence, query head) row; cache bytes equal to the oracle's where no transform rounding
differs (identity transform), window contents equal to the inputs."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_kvq_amd import api, calib, synth
from helpers import f16_ulp_distance, pool_codes, row_rel_err, rare_event_bound

pytestmark = pytest.mark.gpu

TOL = 2e-3
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _transforms(H, G, dtype):
    ts, tis = [], []
    for h in range(H):
        kc, qc = synth.calibration_set(1, h, G)
        t, ti = calib.calibrate_key_transform(kc, qc, store_bf16=(dtype == "bf16"), store_f16=(dtype == "f16"))
        ts.append(synth.to_dtype(t, dtype))
        tis.append(np.ascontiguousarray(np.linalg.inv(synth.to_dtype(t, dtype).astype(np.float64)).T, np.float32))
    return np.stack(ts), np.stack(tis)


def _history(B, H, n, dtype, seed):
    """Full-precision keys and values of every position: [B, n, H, 128] (dtype-rounded)."""
    w = synth.Workload("t", 1, H, H, 1, max(n, 1), 2, 2, "percentile", dtype, True)
    ks, vs = [], []
    for b in range(B):
        k, v = synth.kv_tokens(w, max(n, 1), seq=seed * 31 + b)
        ks.append(k[:n])
        vs.append(v[:n])
    return np.stack(ks), np.stack(vs)


def _queries(rng, B, Hq, dtype):
    return synth.to_dtype(rng.standard_normal((B, Hq, 128)).astype(np.float32) * 2.0, dtype)


class Case:
    def __init__(self, sink, keep, flush, lens, bits, dtype, with_t, G, H=2, rows_perm=False):
        self.sink, self.keep, self.flush, self.lens = sink, keep, flush, list(lens)
        self.bits, self.dtype, self.with_t, self.G, self.H, self.rows_perm = bits, dtype, with_t, G, H, rows_perm


def _quantized(L, c):
    return oracle.window_quantized(L, c.sink, c.keep, c.flush)


def _slots(bt, b, j):
    j = np.asarray(j)
    return bt[b, j // 64].astype(np.int64) * 64 + j % 64


class State:
    """The GPU cache and windows, with the oracle's mirror of the same state."""

    def __init__(self, c, max_len, seed):
        self.c = c
        B, H = len(c.lens), c.H
        rng = np.random.default_rng(seed)
        self.rng = rng
        self.pps = max(1, -(-max(max_len - c.sink, 1) // 64))
        num_pages = B * self.pps + 3
        self.bt = synth.shuffled_block_table(B, self.pps, num_pages, rng)
        self.t = self.tinv = None
        if c.with_t:
            self.t, self.tinv = _transforms(H, c.G, c.dtype)
        self.hk, self.hv = _history(B, H, max_len, c.dtype, seed)
        self.kp = oracle.new_pool(num_pages, H, c.bits[0])
        self.vp = oracle.new_pool(num_pages, H, c.bits[1])
        self.cache = api.KVCache(num_pages, H, c.bits[0], c.bits[1])
        rows = B + 1 if c.rows_perm else B
        self.win_rows = np.arange(B, dtype=np.int32)[::-1].copy() if c.rows_perm else None
        self.win = api.Window(self.cache, rows, c.sink, c.keep, c.flush, dtype=TORCH_DT[c.dtype])
        self.dt = TORCH_DT[c.dtype]
        self.bt_d = torch.from_numpy(self.bt).cuda()
        self.rows_d = None if self.win_rows is None else torch.from_numpy(self.win_rows).cuda()
        self.t_d = None if self.t is None else torch.from_numpy(self.t).to(self.dt).cuda()
        self.tinv_d = None if self.tinv is None else torch.from_numpy(self.tinv).cuda()
        self.lens = np.array(c.lens, np.int32)
        self.max_len = max_len

    def oracle_append(self, b, j0, j1):
        if j1 <= j0:
            return
        s = self.c.sink
        oracle.append(self.kp, self.vp, self.hk[b, s + j0:s + j1], self.hv[b, s + j0:s + j1],
                      _slots(self.bt, b, np.arange(j0, j1)), t_k=self.t, bits_k=self.c.bits[0],
                      bits_v=self.c.bits[1])

    def prefill(self):
        c = self.c
        k = np.concatenate([self.hk[b, :L] for b, L in enumerate(c.lens)])
        v = np.concatenate([self.hv[b, :L] for b, L in enumerate(c.lens)])
        cu = np.concatenate([[0], np.cumsum(c.lens)]).astype(np.int32)
        api.kvq_window_prefill(self.cache, self.win, torch.from_numpy(k).to(self.dt).cuda(),
                               torch.from_numpy(v).to(self.dt).cuda(), torch.from_numpy(cu).cuda(), self.bt_d,
                               win_rows=self.rows_d, t_k=self.t_d)
        for b, L in enumerate(c.lens):
            self.oracle_append(b, 0, _quantized(L, c))

    def reference(self, q, pending):
        c = self.c
        return oracle.window_attention(self.kp, self.vp, q, self.bt, self.lens, self.hk, self.hv, c.sink, c.keep,
                                       c.flush, pending=pending, t_inv_t=self.tinv, bits_k=c.bits[0],
                                       bits_v=c.bits[1])

    def read(self, q):
        out = api.kvq_window_decode_attn(self.cache, self.win, torch.from_numpy(q).to(self.dt).cuda(), self.bt_d,
                                         torch.from_numpy(self.lens).cuda(), self.max_len, win_rows=self.rows_d,
                                         t_k_inv_t=self.tinv_d)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def step(self, q):
        """Every sequence gains one position (its history row); returns the GPU output."""
        c = self.c
        B = len(c.lens)
        pos = self.lens.copy()
        self.lens = self.lens + 1
        kn = np.stack([self.hk[b, pos[b]] for b in range(B)])
        vn = np.stack([self.hv[b, pos[b]] for b in range(B)])
        out = api.kvq_window_decode_step(self.cache, self.win, torch.from_numpy(q).to(self.dt).cuda(),
                                         torch.from_numpy(kn).to(self.dt).cuda(),
                                         torch.from_numpy(vn).to(self.dt).cuda(), self.bt_d,
                                         torch.from_numpy(self.lens).cuda(), self.max_len, win_rows=self.rows_d,
                                         t_k=self.t_d, t_k_inv_t=self.tinv_d)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle_flush(self):
        for b, L in enumerate(self.lens):
            self.oracle_append(b, _quantized(L - 1, self.c), _quantized(L, self.c))

    def check_windows(self):
        """Every full-precision position of every sequence sits in its window slot."""
        c = self.c
        kw = self.win.k_win.float().cpu().numpy()
        vw = self.win.v_win.float().cpu().numpy()
        for b, L in enumerate(self.lens):
            row = b if self.win_rows is None else self.win_rows[b]
            nq = _quantized(int(L), c)
            for p in list(range(min(L, c.sink))) + list(range(c.sink + nq, L)):
                slot = p if p < c.sink else c.sink + (p - c.sink) % (c.keep + c.flush)
                assert np.array_equal(kw[row, slot], self.hk[b, p]), (b, p)
                assert np.array_equal(vw[row, slot], self.hv[b, p]), (b, p)

    def check_cache_bytes(self):
        """Pages filled with quantized positions: GPU bytes equal to the oracle's (no transform)."""
        gk = self.cache.k_pages.cpu().numpy()
        gv = self.cache.v_pages.cpu().numpy()
        for b, L in enumerate(self.lens):
            for pg in self.bt[b, :_quantized(int(L), self.c) // 64]:
                assert np.array_equal(gk[pg], self.kp[pg]) and np.array_equal(gv[pg], self.vp[pg]), (b, pg)


PREFILL_CASES = [
    Case(4, 16, 16, [1, 4, 20, 36, 37, 300, 517, 68], (2, 2), "bf16", False, 4),
    Case(0, 0, 64, [64, 128, 200], (2, 2), "bf16", True, 4),
    Case(32, 64, 64, [2000, 160, 31, 1000], (4, 4), "f16", True, 8, H=1),
    Case(1, 3, 5, [7, 8, 9, 100, 0], (2, 4), "f32", True, 2, rows_perm=True),
    Case(5, 0, 1, [3, 6, 77], (4, 2), "bf16", False, 16, H=1),
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_prefill_then_read(case):
    c = PREFILL_CASES[case]
    print(f"window prefill case {case}: sink={c.sink} keep={c.keep} flush={c.flush} lens={c.lens}", flush=True)
    s = State(c, max(max(c.lens), 1), seed=100 + case)
    s.prefill()
    q = _queries(s.rng, len(c.lens), c.H * c.G, c.dtype)
    got = s.read(q)
    ref = s.reference(q, pending=0)
    err = row_rel_err(got, ref)
    assert err.max() <= TOL, err.max()
    s.check_windows()
    if not c.with_t:
        s.check_cache_bytes()


STEP_CASES = [
    Case(3, 10, 8, [0, 5, 20, 40], (2, 2), "bf16", False, 4),
    Case(2, 5, 16, [1, 30, 63], (4, 2), "bf16", True, 4, rows_perm=True),
    Case(0, 1, 4, [9, 2], (2, 4), "f32", True, 8, H=1),
    Case(6, 0, 2, [6, 7, 50], (2, 2), "f16", False, 2),
    # batch x flush > 512 candidate positions: the flush runs on the 128-token tile kernel
    Case(4, 8, 64, [50, 60, 70, 100, 120, 130, 140, 75, 200], (2, 2), "bf16", False, 4),
    Case(4, 8, 64, [50, 60, 70, 100, 120, 130, 140, 75, 200], (4, 4), "f16", True, 4, rows_perm=True),
    Case(3, 10, 8, [0, 5, 20, 40], (3, 3), "bf16", False, 4),
    Case(4, 8, 64, [50, 60, 70, 100, 120, 130, 140, 75, 200], (3, 2), "bf16", True, 8),
]


@pytest.mark.parametrize("case", range(len(STEP_CASES)))
def test_decode_steps(case):
    c = STEP_CASES[case]
    steps = 36
    print(f"window step case {case}: sink={c.sink} keep={c.keep} flush={c.flush} lens={c.lens}", flush=True)
    s = State(c, max(c.lens) + steps, seed=200 + case)
    s.prefill()
    for i in range(steps):
        q = _queries(s.rng, len(c.lens), c.H * c.G, c.dtype)
        got = s.step(q)
        ref = s.reference(q, pending=1)
        err = row_rel_err(got, ref)
        assert err.max() <= TOL, (i, err.max())
        s.oracle_flush()
    s.check_windows()
    if not c.with_t:
        s.check_cache_bytes()
    q = _queries(s.rng, len(c.lens), c.H * c.G, c.dtype)
    assert row_rel_err(s.read(q), s.reference(q, pending=0)).max() <= TOL


def test_step_in_a_graph_matches_eager():
    """The step captured in a HIP graph (no host synchronisation inside) and replayed
    several times gives the eager results, with eager work between replays."""
    c = Case(3, 8, 8, [10, 40, 17], (2, 2), "bf16", True, 4)
    steps = 12
    a = State(c, max(c.lens) + steps, seed=300)
    b = State(c, max(c.lens) + steps, seed=300)
    a.prefill()
    b.prefill()
    B, Hq = len(c.lens), c.H * c.G
    qs = [_queries(a.rng, B, Hq, c.dtype) for _ in range(steps)]
    eager = [a.step(q) for q in qs]
    # graph: one captured step whose inputs are refilled before each replay
    q_d = torch.zeros((B, Hq, 128), dtype=b.dt, device="cuda")
    kn_d = torch.zeros((B, c.H, 128), dtype=b.dt, device="cuda")
    vn_d = torch.zeros_like(kn_d)
    lens_d = torch.from_numpy(b.lens).cuda()
    out_d = torch.zeros((B, Hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros(api.window_workspace_bytes(b.cache, b.win, B, Hq, b.max_len), dtype=torch.uint8,
                     device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.kvq_window_decode_step(b.cache, b.win, q_d, kn_d, vn_d, b.bt_d, lens_d, b.max_len, t_k=b.t_d,
                                   t_k_inv_t=b.tinv_d, out=out_d, workspace=ws)
    torch.cuda.synchronize()
    for i in range(steps):
        pos = b.lens.copy()
        b.lens = b.lens + 1
        q_d.copy_(torch.from_numpy(qs[i]).to(b.dt))
        kn_d.copy_(torch.from_numpy(np.stack([b.hk[j, pos[j]] for j in range(B)])).to(b.dt))
        vn_d.copy_(torch.from_numpy(np.stack([b.hv[j, pos[j]] for j in range(B)])).to(b.dt))
        lens_d.copy_(torch.from_numpy(b.lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_d.cpu().numpy(), eager[i]), i
    assert torch.equal(a.cache.k_pages, b.cache.k_pages) and torch.equal(a.cache.v_pages, b.cache.v_pages)
    assert torch.equal(a.win.k_win, b.win.k_win) and torch.equal(a.win.v_win, b.win.v_win)


def test_full_size_window_step_sampled():
    """Qwen3-8B-shaped layer, batch 64, about 16K positions per sequence, 2-bit, windows of
    32 sink + 64 keep + 64 flush positions, in the launch configuration the benchmark
    times: random cache codes and window contents; the oracle recomputes a seeded sample
    of sequences, and the sequence whose new position completes a batch has its flushed
    positions compared with the oracle's encoding."""
    w = synth.WORKLOADS["qwen3-8b-b64-16k"]
    H, B, G = w.heads_kv, w.batch, w.group
    sink, keep, flush = 32, 64, 64
    W = sink + keep + flush
    rng = np.random.default_rng(12)
    lens = (w.seq_len - np.arange(B)).astype(np.int32)          # b = 32 completes a batch
    pps = -(-(w.seq_len - sink) // 64)
    kp = synth.random_packed_pool(rng, B * pps, H, w.bits_k)
    vp = synth.random_packed_pool(rng, B * pps, H, w.bits_v)
    bt = synth.contiguous_block_table(B, pps)
    cache = api.KVCache(B * pps, H, w.bits_k, w.bits_v, k_pages=torch.from_numpy(kp).cuda(),
                        v_pages=torch.from_numpy(vp).cuda())
    kw = synth.to_dtype(rng.standard_normal((B, W, H, 128)).astype(np.float32), "bf16")
    vw = synth.to_dtype(rng.standard_normal((B, W, H, 128)).astype(np.float32), "bf16")
    win = api.Window(cache, B, sink, keep, flush, k_win=torch.from_numpy(kw).to(torch.bfloat16).cuda(),
                     v_win=torch.from_numpy(vw).to(torch.bfloat16).cuda())
    q = synth.decode_queries(w)
    kn = synth.to_dtype(rng.standard_normal((B, H, 128)).astype(np.float32), "bf16")
    vn = synth.to_dtype(rng.standard_normal((B, H, 128)).astype(np.float32), "bf16")
    t, tinv = _transforms(H, G, "bf16")
    out = api.kvq_window_decode_step(cache, win, torch.from_numpy(q).to(torch.bfloat16).cuda(),
                                     torch.from_numpy(kn).to(torch.bfloat16).cuda(),
                                     torch.from_numpy(vn).to(torch.bfloat16).cuda(), torch.from_numpy(bt).cuda(),
                                     torch.from_numpy(lens).cuda(), w.seq_len,
                                     t_k=torch.from_numpy(t).to(torch.bfloat16).cuda(),
                                     t_k_inv_t=torch.from_numpy(tinv).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy()

    def history(b):
        """Full-precision positions of sequence b as the attention saw them."""
        L = int(lens[b])
        hk = np.zeros((1, L, H, 128), np.float32)
        hv = np.zeros_like(hk)
        nq = oracle.window_quantized(L - 1, sink, keep, flush)
        for p in list(range(min(L, sink))) + list(range(sink + nq, L)):
            slot = p if p < sink else sink + (p - sink) % (keep + flush)
            hk[0, p], hv[0, p] = (kn[b], vn[b]) if p == L - 1 else (kw[b, slot], vw[b, slot])
        return hk, hv

    for b in sorted(set(rng.choice(B, 2, replace=False).tolist()) | {32}):
        hk, hv = history(b)
        ref = oracle.window_attention(kp, vp, q[b:b + 1], bt[b:b + 1], lens[b:b + 1], hk, hv, sink, keep, flush,
                                      pending=1, t_inv_t=tinv, bits_k=w.bits_k, bits_v=w.bits_v)
        assert row_rel_err(got[b:b + 1], ref).max() <= TOL, b
    # the flush of sequence 32: positions sink + q0 .. sink + q0 + 63 from its window row
    L = int(lens[32])
    q0, q1 = oracle.window_quantized(L - 1, sink, keep, flush), oracle.window_quantized(L, sink, keep, flush)
    assert q1 - q0 == flush
    hk, hv = history(32)
    kp2, vp2 = kp.copy(), vp.copy()
    oracle.append(kp2, vp2, hk[0, sink + q0:sink + q1], hv[0, sink + q0:sink + q1],
                  _slots(bt, 32, np.arange(q0, q1)), t_k=t, bits_k=w.bits_k, bits_v=w.bits_v)
    pg = bt[32, q0 // 64]
    gv = cache.v_pages[pg].cpu().numpy()
    assert np.array_equal(gv, vp2[pg])
    page_slots = pg * 64 + np.arange(64)
    gc, gs, gz = pool_codes(cache.k_pages.cpu().numpy(), 0, w.bits_k, page_slots)
    oc, os_, oz = pool_codes(kp2, 0, w.bits_k, page_slots)
    assert np.mean(gc != oc) <= 1e-4                          # fp32 vs fp64 transform sums
    assert np.sum((gs != os_) | (gz != oz)) <= rare_event_bound(gs.size)
    assert np.all(f16_ulp_distance(gs, os_) <= 1) and np.all(f16_ulp_distance(gz, oz) <= 1)
    untouched = [x for x in range(B * pps) if x != pg]
    assert torch.equal(cache.v_pages[untouched].cpu(), torch.from_numpy(vp[untouched]))
