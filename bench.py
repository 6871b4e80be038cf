"""Benchmark of one decode step of the quantized-KV-cache hot path on one MI355X.

A step is the whole hot path over one batch: every sequence is decoded over its cache, with
its new token at full precision, and the batch's new tokens (one per sequence) are
transformed, clipped, quantized to 2-bit percentile codes and packed into the cache for
later steps: one kvq_decode_step call.  Default workload: the Qwen3-8B-shaped layer (32 query heads, 8 KV heads, head_dim
128) at batch 64 x 16384 cached tokens, 2-bit K and V, synthetic Sigma-model data, caches
resident in HBM.

Each timed region is one replay of a HIP graph of K consecutive steps captured from the
library calls (the calls launch on torch's current stream, which the capture records), so
host-side call cost does not pace the GPU.  Prints one JSON line.  `value` is cached
tokens read per second (batch x context per step time).  `roofline` is for the step's
dominant kernel, the decode: algorithmic bytes per launch over its average launch time
(HIP events on the launch stream around the timed replay of a decode-only graph) against
8 TB/s.  `cpu_baseline` is the CPU oracle's decode timed on a bounded sample of sequences
of the same shape, on one thread and on all available cores.  `step_ms_p10_p50_p90` spreads nine more replays of the timed graph;
`reference_bandwidth` is what plain torch kernels reach on the same GPU (a 1 GiB copy and a
sum over the KV-cache pools), for context; it runs right before the step's warm-up replay, so
that the timed replay follows load rather than idle (after idle the clocks take a few
milliseconds of load to settle) and finds the cache's address translations warm.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 400 warm-up steps (~50 ms of back-to-back work): after idle the GPU runs the first
    # milliseconds of a step stream ~15% slower until its clocks settle
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="qwen3-8b-b64-16k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reference-ms", type=float, default=60.0,
                    help="how long the reference-bandwidth probe runs (directly before the timed replays)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--extra", action="store_true", help="also time the other workloads")
    ap.add_argument("--prefill-only", metavar="WORKLOAD", default=None,
                    help="only time the bulk quantize-append of a prefill workload (for profiling)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (the reference kernel "
                         "whose FETCH_SIZE/WRITE_SIZE readings scale the decode kernel's counters)")
    return ap.parse_args()


def decode_algorithmic_bytes(w, B, seq_len) -> int:
    """Bytes the decode step must move: packed K and V of every cached token (codes +
    fp16 scale and zero), the queries (bf16), the output (fp32), the block table (int32
    per page) and the inverse-transpose transform (fp32, 64 KiB per KV head)."""
    per_token = w.heads_kv * ((128 * w.bits_k // 8 + 4) + (128 * w.bits_v // 8 + 4))
    pages = -(-seq_len // 64)
    return (B * seq_len * per_token + B * w.heads_q * 128 * 2 + B * w.heads_q * 128 * 4
            + B * pages * 4 + w.heads_kv * 128 * 128 * 4)


def append_algorithmic_bytes(w, n) -> int:
    """k and v in (bf16), T (bf16), slots (int64), codes and metadata out."""
    per = w.heads_kv * 128 * 2 * 2 + 8
    out = w.heads_kv * ((128 * w.bits_k // 8 + 4) + (128 * w.bits_v // 8 + 4))
    return n * (per + out) + w.heads_kv * 128 * 128 * 2


def setup_decode(w, torch, api, calib, synth, dev):
    B, H, pps = w.batch, w.heads_kv, w.pages_per_seq
    cache = api.KVCache(B * pps, H, w.bits_k, w.bits_v, w.quantizer, w.quantizer, w.p_lo, w.p_hi,
                        w.alpha, w.alpha, device=dev)
    ts, tis = [], []
    for h in range(H):
        kc, qc = synth.calibration_set(w.config, h, w.group)
        t, ti = calib.calibrate_key_transform(kc, qc)
        ts.append(t)
        tis.append(ti)
    t_k = torch.from_numpy(np.stack(ts)).to(torch.bfloat16).to(dev)
    t_inv = torch.from_numpy(np.stack(tis)).to(dev)
    # fill the cache sequence by sequence with the GPU write path
    per = max(1, (1 << 21) // w.seq_len)
    for b0 in range(0, B, per):
        nb = min(per, B - b0)
        k, v = synth.kv_tokens_torch(w, nb * w.seq_len, dev, seq=b0)
        slots = torch.arange(b0 * pps * 64, b0 * pps * 64 + nb * w.seq_len, dtype=torch.int64, device=dev)
        api.kvq_quantize_append(cache, k, v, slots, t_k=t_k)
        del k, v
    torch.cuda.synchronize()
    bt = torch.from_numpy(synth.contiguous_block_table(B, pps)).to(dev)
    seq = torch.full((B,), w.seq_len, dtype=torch.int32, device=dev)
    q = torch.from_numpy(synth.decode_queries(w)).to(torch.bfloat16).to(dev)
    # the step's new token of each sequence is appended at its last position
    knew, vnew = synth.kv_tokens_torch(w, B, dev, seq=10_000)
    new_slots = torch.tensor([b * pps * 64 + w.seq_len - 1 for b in range(B)], dtype=torch.int64, device=dev)
    # the step's workspace: the decode's partial outputs and the query-operand image that the
    # step's append launch builds (the plain decode uses the first part only)
    ws = torch.empty(max(1, api.decode_step_workspace_bytes(cache, B, w.heads_q, w.seq_len)), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, w.heads_q, 128), dtype=torch.float32, device=dev)
    return dict(cache=cache, t_k=t_k, t_inv=t_inv, bt=bt, seq=seq, q=q, knew=knew, vnew=vnew,
                new_slots=new_slots, ws=ws, out=out)


def time_steps(w, s, torch, api, steps, warmup, before=None):
    """Times the step, kvq_decode_step (every sequence decoded with its new token at full
    precision, the new tokens appended in the same launch), as one HIP-graph replay of `steps` consecutive steps (captured from the
    library calls, which launch on torch's current stream), after one replay of a graph of
    `warmup` steps, so the host's per-call and per-replay cost does not pace the GPU.  HIP
    events on the launch stream bracket the timed replay.  The append and the decode kernel
    alone are timed the same way.  `before` runs directly before the step's warm-up replay.
    Returns ms per step of each."""

    def append():
        api.kvq_quantize_append(s["cache"], s["knew"], s["vnew"], s["new_slots"], t_k=s["t_k"])

    def decode():
        api.kvq_decode_attn(s["cache"], s["q"], s["bt"], s["seq"], w.seq_len, t_k_inv_t=s["t_inv"],
                            out=s["out"], workspace=s["ws"])

    def step():
        api.kvq_decode_step(s["cache"], s["q"], s["knew"], s["vnew"], s["new_slots"], s["bt"], s["seq"],
                            w.seq_len, t_k=s["t_k"], t_k_inv_t=s["t_inv"], out=s["out"], workspace=s["ws"])

    step()                                   # first call (library load) outside the graphs
    torch.cuda.synchronize()
    ms_step, wall_step, more = graph_time(torch, step, steps, warmup, extra_replays=9, before=before)
    ms_app, _ = graph_time(torch, append, steps, warmup)
    ms_dec, _ = graph_time(torch, decode, steps, warmup)
    return dict(step=ms_step, wall=wall_step, append=ms_app, decode=ms_dec, step_replays=[ms_step] + more)


def time_decode_from_hbm(w, s, torch, api, steps, warmup):
    """The decode alone over copies of the cache that together exceed the MALL twice over,
    one copy per call in turn (each with its own block table), so that every call reads its
    pages from HBM.  For caches that fit the MALL (batch 1).  Returns ms per call."""
    copies = max(2, -(-2 * MALL_BYTES // max(1, s["cache"].k_pages.numel() + s["cache"].v_pages.numel())) + 1)
    src = s["cache"]
    big = api.KVCache(src.num_pages * copies, src.num_kv_heads, src.bits_k, src.bits_v, src.quant_k,
                      src.quant_v, src.p_lo, src.p_hi, src.alpha_k, src.alpha_v, device=src.k_pages.device)
    for c in range(copies):
        big.k_pages[c * src.num_pages:(c + 1) * src.num_pages].copy_(src.k_pages)
        big.v_pages[c * src.num_pages:(c + 1) * src.num_pages].copy_(src.v_pages)
    bts = [s["bt"] + c * src.num_pages for c in range(copies)]
    state = {"i": 0}

    def decode():
        bt = bts[state["i"] % copies]
        state["i"] += 1
        api.kvq_decode_attn(big, s["q"], bt, s["seq"], w.seq_len, t_k_inv_t=s["t_inv"], out=s["out"],
                            workspace=s["ws"])

    ms, _ = graph_time(torch, decode, max(steps, copies), max(warmup, copies))
    del big, bts
    return ms, copies


def reference_bandwidth(torch, dev, read_tensors, nbytes=1 << 30, run_ms=60.0):
    """What plain torch kernels reach on this GPU, as an achievable-bandwidth reference: a
    1 GiB device copy (read + write), then a sum over `read_tensors` (the KV-cache pools, the
    very bytes the decode reads, viewed as fp32), in GB/s, each repeated back to back for
    about run_ms / 2.  It runs directly before the timed replays of the step: after idle the
    GPU needs some tens of milliseconds of load before its clocks settle, and reading the
    cache last leaves its address translations warm (the copy's buffers stay in torch's
    cache, so no free sits between the probe and the replays)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    views = [t.view(torch.float32).view(-1) for t in read_tensors]
    read_bytes = sum(v.numel() * 4 for v in views)

    def read_sum():
        for v in views:
            v.sum()

    out = {}
    for name, fn, moved in (("copy", lambda: dst.copy_(src), 2 * nbytes), ("cache_read_sum", read_sum, read_bytes)):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        reps = max(10, int(run_ms / 2 / max((time.perf_counter() - t0) * 1e3, 1e-3)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_GB_s"] = moved / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
        out[name + "_reps"] = reps
    out["cache_read_bytes"] = read_bytes
    del src, dst
    return out


def graph_time(torch, fn, steps, warmup, extra_replays=0, before=None):
    """ms per call of fn: one replay of a HIP graph of `steps` calls (captured from the
    library calls on torch's current stream) after one replay of a graph of `warmup`
    calls, bracketed by HIP events on the launch stream; also the host wall time.  With
    extra_replays, the timed graph is replayed that many more times and the per-call times
    of those replays are returned too.  `before`, if given, runs once the graphs are
    captured, directly before the warm-up replay."""

    def capture(count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(count):
                fn()
        return g

    gw, gt = capture(max(warmup, 1)), capture(steps)
    torch.cuda.synchronize()
    if before is not None:
        before()
    gw.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    gt.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    wall = (time.perf_counter() - t0) * 1e3 / steps
    more = []
    for _ in range(extra_replays):
        e0.record()
        gt.replay()
        e1.record()
        torch.cuda.synchronize()
        more.append(e0.elapsed_time(e1) / steps)
    del gw, gt
    return (ms, wall, more) if extra_replays else (ms, wall)


WINDOW = (32, 64, 64)          # S_sink, S_keep, S_flush: at most 159 full-precision positions


def time_window(w, s, torch, api, steps, warmup):
    """The decode step over a windowed cache (kvq_window_decode_step) on the workload's
    cache: full-precision windows of S_sink = 32, S_keep = 64, S_flush = 64 positions (under
    1% of the 16K context) in bf16.  Timed at a length whose step quantizes nothing (63 of
    every 64 steps) and at one whose step quantizes a batch of 64 positions in every
    sequence; the amortised step is (63 x plain + flush) / 64."""
    sink, keep, flush = WINDOW
    B, H = w.batch, w.heads_kv
    dev = s["q"].device
    win = api.Window(s["cache"], B, sink, keep, flush, dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    win.k_win.copy_(torch.randn(win.k_win.shape, generator=g, device=dev))
    win.v_win.copy_(torch.randn(win.v_win.shape, generator=g, device=dev))
    ws = torch.empty(api.window_workspace_bytes(s["cache"], win, B, w.heads_q, w.seq_len), dtype=torch.uint8,
                     device=dev)
    plain_len = w.seq_len                                   # (16384 - 96) % 64 != 0: no batch completes
    flush_len = sink + keep + flush * ((w.seq_len - sink - keep) // flush)   # a batch completes
    res = {}
    for name, L in (("step", plain_len), ("flush_step", flush_len)):
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)

        def step():
            api.kvq_window_decode_step(s["cache"], win, s["q"], s["knew"], s["vnew"], s["bt"], lens, w.seq_len,
                                       t_k=s["t_k"], t_k_inv_t=s["t_inv"], out=s["out"], workspace=ws)
        step()
        torch.cuda.synchronize()
        res[name] = graph_time(torch, step, steps, warmup)[0]
    lens = torch.full((B,), plain_len, dtype=torch.int32, device=dev)

    def read():
        api.kvq_window_decode_attn(s["cache"], win, s["q"], s["bt"], lens, w.seq_len, t_k_inv_t=s["t_inv"],
                                   out=s["out"], workspace=ws)
    res["read"] = graph_time(torch, read, steps, warmup)[0]
    amort = (63 * res["step"] + res["flush_step"]) / 64
    return {"window": {"sink": sink, "keep": keep, "flush": flush, "dtype": "bf16"},
            "step_us": res["step"] * 1e3, "flush_step_us": res["flush_step"] * 1e3,
            "amortised_step_us": amort * 1e3, "read_us": res["read"] * 1e3,
            "tokens_per_s": B * w.seq_len / (amort * 1e-3)}


MALL_BYTES = 256 << 20


def time_prefill(w, torch, api, calib, synth, dev, reps=200, warmup=1000):
    """Steady-state time of one bulk append: HIP events around `reps` back-to-back launches
    after `warmup` untimed ones (~40 ms, like the decode's warm-up, so that the clocks have
    settled).  One launch reads 134 MB and writes 36 MB, less than the 256 MB MALL, so the
    launches cycle over enough separate input sets and caches (more than twice the MALL)
    that every launch reads its rows from HBM: `us` and `frac` are that rate.  `us_warm`
    repeats one set, whose rows the MALL then partly serves (context, not an HBM figure)."""
    n, H = w.seq_len, w.heads_kv
    by = append_algorithmic_bytes(w, n)
    nsets = max(2, -(-2 * MALL_BYTES // by) + 1)
    ts = [calib.calibrate_key_transform(*synth.calibration_set(w.config, h, 4))[0] for h in range(H)]
    t_k = torch.from_numpy(np.stack(ts)).to(torch.bfloat16).to(dev)
    slots = torch.arange(n, dtype=torch.int64, device=dev)
    sets = []
    for _ in range(nsets):
        k, v = synth.kv_tokens_torch(w, n, dev)
        sets.append((api.KVCache(n // 64, H, w.bits_k, w.bits_v, device=dev), k, v))

    def run(count, rotate):
        for i in range(count):
            cache, k, v = sets[i % nsets if rotate else 0]
            api.kvq_quantize_append(cache, k, v, slots, t_k=t_k)

    def timed(rotate):
        run(warmup, rotate)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        run(reps, rotate)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    ms = timed(True)
    ms_warm = timed(False)
    del sets
    return {"workload": w.name, "us": ms * 1e3, "GB_s": by / (ms * 1e-3) / 1e9,
            "frac": by / (ms * 1e-3) / HBM_PEAK, "algorithmic_bytes": by, "input_sets": nsets,
            "us_warm": ms_warm * 1e3, "frac_warm": by / (ms_warm * 1e-3) / HBM_PEAK}


def step_traffic_bytes():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE scaled by a plain copy's reading), or None when that summary
    is missing or was taken on other kernel sources than the ones built here."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode_qwen3-8b-b64-16k_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(("sources_sha256:", "traffic_bytes:")))
    h = hashlib.sha256()
    for f in ("kvq_decode.hip", "kvq_device.h", "kvq_internal.h"):
        h.update(open(os.path.join(ROOT, "decode_attention_kvq_amd", "csrc", f), "rb").read())
    if fields.get("sources_sha256", "").strip() != h.hexdigest():
        return None
    return float(fields["traffic_bytes"])


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seconds):
    """The oracle's decode attention on whole sequences of the workload's shape (random
    packed codes: the oracle's cost does not depend on the values), unmodified: first on one
    thread, then on one thread per available core (up to 16), each calling the oracle on its
    own sequences (the C oracle runs outside Python's lock).  `value` is the all-core rate."""
    import concurrent.futures as cf
    import oracle
    from decode_attention_kvq_amd import synth
    rng = np.random.default_rng(0)
    H, pps = w.heads_kv, w.pages_per_seq
    kp = synth.random_packed_pool(rng, pps, H, w.bits_k)
    vp = synth.random_packed_pool(rng, pps, H, w.bits_v)
    bt = np.arange(pps, dtype=np.int32)[None]
    seq = np.array([w.seq_len], np.int32)
    q = synth.decode_queries(w, batch=1)
    tinv = np.broadcast_to(np.eye(128, dtype=np.float32), (H, 128, 128)).copy()
    oracle.lib()

    def run(deadline):
        n = 0
        while time.perf_counter() < deadline:
            oracle.decode_attention(kp, vp, q, bt, seq, t_inv_t=tinv, bits_k=w.bits_k, bits_v=w.bits_v)
            n += 1
        return n

    t0 = time.perf_counter()
    n1 = run(t0 + seconds / 3)
    el1 = time.perf_counter() - t0
    avail = len(os.sched_getaffinity(0))
    cores = max(1, min(16, avail))           # one GPU's share of a shared host: 16 threads
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        counts = list(ex.map(run, [t0 + seconds * 2 / 3] * cores))
    el = time.perf_counter() - t0
    done = sum(counts)
    return {"value": done * w.seq_len / el, "unit": "cached tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": avail,
            "thread_cap": "16 threads at most (the host share of one GPU)",
            "single_thread_value": n1 * w.seq_len / el1,
            "sample": f"whole sequences of {w.seq_len} tokens x {w.heads_q} query heads (one decode step "
                      f"each): {done} on {cores} threads in {el:.1f} s; {n1} on one thread in {el1:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path would shard by KV head with no exchange)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}), flush=True)
        return
    from decode_attention_kvq_amd import api, calib, synth
    from decode_attention_kvq_amd import build as kbuild
    if not os.path.exists(os.path.join(ROOT, "decode_attention_kvq_amd", "libkvq.so")):
        kbuild.build()
    dev = torch.device("cuda:0")
    if args.prefill_only:
        print(json.dumps(time_prefill(synth.WORKLOADS[args.prefill_only], torch, api, calib, synth, dev)), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    s = setup_decode(w, torch, api, calib, synth, dev)
    ref = {}
    t = time_steps(w, s, torch, api, args.steps, args.warmup,
                   before=lambda: ref.update(reference_bandwidth(torch, dev, (s["cache"].k_pages, s["cache"].v_pages),
                                                                 run_ms=args.reference_ms)))
    cached = w.batch * w.seq_len
    dbytes = decode_algorithmic_bytes(w, w.batch, w.seq_len)
    achieved = dbytes / (t["decode"] * 1e-3)
    rec = {
        "metric": "decode-attn cached tokens/s + HBM GB/s (% of peak), 2-bit, batch x 16K ctx",
        "value": cached / (t["step"] * 1e-3),
        "unit": "cached tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t["step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u2 codes; fp4 x fp6 (scores) and f16 (P.V) matrix-core products, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len, "heads_q": w.heads_q,
                   "heads_kv": w.heads_kv, "head_dim": 128, "bits_k": w.bits_k, "bits_v": w.bits_v,
                   "quantizer": w.quantizer, "page_tokens": 64, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "traffic": step_traffic_bytes(),
                     "kernel": "decode_kernel (kvq_decode_attn)", "algorithmic_bytes": dbytes,
                     "avg_us": t["decode"] * 1e3},
        "wall_ms_per_step": t["wall"],
        "step_ms_p10_p50_p90": [float(np.percentile(t["step_replays"], q)) for q in (10, 50, 90)],
        "append_us": t["append"] * 1e3,
        "decode_us": t["decode"] * 1e3,
        "decode_tokens_per_s": cached / (t["decode"] * 1e-3),
    }
    if args.extra:
        extra = {w.name + "-window": time_window(w, s, torch, api, args.steps, args.warmup)}
    del s
    torch.cuda.empty_cache()
    rec["reference_bandwidth"] = ref
    if args.extra:
        for name in ("qwen3-8b-b1-16k", "long-b16-128k-quest", "qwen3-8b-b64-16k-3bit"):
            w2 = synth.WORKLOADS[name]
            s2 = setup_decode(w2, torch, api, calib, synth, dev)
            t2 = time_steps(w2, s2, torch, api, 20, args.warmup)
            dby = decode_algorithmic_bytes(w2, w2.batch, w2.seq_len)
            extra[name] = {"step_us": t2["step"] * 1e3, "tokens_per_s": w2.batch * w2.seq_len / (t2["step"] * 1e-3),
                           "append_us": t2["append"] * 1e3, "decode_us": t2["decode"] * 1e3,
                           "decode_GB_s": dby / (t2["decode"] * 1e-3) / 1e9,
                           "decode_frac": dby / (t2["decode"] * 1e-3) / HBM_PEAK}
            if dby < MALL_BYTES:
                # the cache fits the MALL: also the decode with every call reading from HBM
                ms_h, copies = time_decode_from_hbm(w2, s2, torch, api, 20, args.warmup)
                extra[name].update({"decode_us_from_hbm": ms_h * 1e3, "cache_copies": copies})
            del s2
            torch.cuda.empty_cache()
        for name in ("prefill-8x32k-4bit", "prefill-8x32k-2bit", "prefill-8x32k-3bit"):
            extra[name] = time_prefill(synth.WORKLOADS[name], torch, api, calib, synth, dev)
        rec["other_workloads"] = extra
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
