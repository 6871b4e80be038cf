"""The benchmark's byte accounting against the figures the workload table states for each
configuration (algorithmic bytes: what the method itself must move)."""
import bench
from decode_attention_kvq_amd import synth


def test_decode_algorithmic_bytes_match_the_configurations():
    w = synth.WORKLOADS["qwen3-8b-b64-16k"]
    assert bench.decode_algorithmic_bytes(w, w.batch, w.seq_len) == 606_142_464       # 606.1 MB
    w1 = synth.WORKLOADS["qwen3-8b-b1-16k"]
    assert round(bench.decode_algorithmic_bytes(w1, 1, w1.seq_len) / 1e6, 2) == 9.99
    w4 = synth.WORKLOADS["long-b16-128k-quest"]
    assert round(bench.decode_algorithmic_bytes(w4, w4.batch, w4.seq_len) / 1e6, 1) == 1209.4


def test_cache_bytes_per_token_follow_the_block_layout():
    # (32 + 4) * 2 = 72 B per token per KV head at 2-bit, 136 at 4-bit, 104 at 3-bit
    for bits, per in ((2, 72), (3, 104), (4, 136)):
        w = synth.Workload("x", 2, 8, 1, 1, 64, bits, bits, "percentile", "bf16", True)
        fixed = bench.decode_algorithmic_bytes(w, 1, 0)
        assert bench.decode_algorithmic_bytes(w, 1, 64) - fixed == 64 * per + 4


def test_append_algorithmic_bytes_match_the_prefill_configurations():
    assert round(bench.append_algorithmic_bytes(synth.WORKLOADS["prefill-8x32k-4bit"], 32768) / 1e6, 1) == 170.4
    assert round(bench.append_algorithmic_bytes(synth.WORKLOADS["prefill-8x32k-2bit"], 32768) / 1e6, 1) == 153.6
