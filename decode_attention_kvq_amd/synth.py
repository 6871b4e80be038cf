"""Seeded synthetic inputs for tests and benchmarks.

This module only draws numbers; it holds none of the quantization or attention
arithmetic, so both the HIP path and the CPU oracle can be fed from it.

Distribution (a stand-in for post-RoPE Qwen3-8B keys/values and queries, whose weights
and calibration data are not available here):
  * keys and values of KV head h: x = z diag(sqrt(lam)) U^T with z ~ N(0, I), lam_i = 0.95^i
    (i = 0..127), U Haar-orthogonal; then 4 seeded channels are multiplied by 10;
  * queries of query head g: the same spectrum on a separately seeded basis, no outliers;
  * calibration: 1024 keys per KV head and 1024 queries per query head, independent draws.
Seeds: 1_000_000 * config + 1000 * role + head, with the roles below.
Values are drawn in fp64, rounded to fp32, and (where a workload says bf16) rounded to
bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses

import numpy as np

HEAD_DIM = 128
DECAY = 0.95
N_OUTLIERS = 4
OUTLIER_STD = 10.0

ROLE_K_BASIS = 1
ROLE_K_DRAW = 2
ROLE_V_BASIS = 3
ROLE_V_DRAW = 4
ROLE_Q_BASIS = 5
ROLE_Q_DRAW = 6
ROLE_CAL_K = 7
ROLE_CAL_Q = 8
ROLE_OUTLIER = 9
ROLE_LAYOUT = 10      # page shuffles, ragged lengths, slot permutations (tests only)


def seed_for(config: int, role: int, head: int) -> int:
    return 1_000_000 * config + 1000 * role + head


def rng_for(config: int, role: int, head: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_for(config, role, head)))


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload."""
    name: str
    config: int
    heads_q: int
    heads_kv: int
    batch: int
    seq_len: int
    bits_k: int
    bits_v: int
    quantizer: str          # "percentile" or "rms"
    dtype: str              # "f32" or "bf16" for K/V/Q inputs
    use_transform: bool
    p_lo: float = 0.01
    p_hi: float = 0.99
    alpha: float = 2.83

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def pages_per_seq(self) -> int:
        return -(-self.seq_len // 64)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 1, 1, 256, 4, 4, "percentile", "f32", True),
    "qwen3-8b-b1-16k": Workload("qwen3-8b-b1-16k", 1, 32, 8, 1, 16384, 2, 2, "percentile",
                                "bf16", True),
    "qwen3-8b-b64-16k": Workload("qwen3-8b-b64-16k", 2, 32, 8, 64, 16384, 2, 2, "percentile",
                                 "bf16", True),
    "prefill-8x32k-4bit": Workload("prefill-8x32k-4bit", 3, 8, 8, 1, 32768, 4, 4,
                                   "percentile", "bf16", True),
    "prefill-8x32k-2bit": Workload("prefill-8x32k-2bit", 3, 8, 8, 1, 32768, 2, 2,
                                   "percentile", "bf16", True),
    "long-b16-128k-quest": Workload("long-b16-128k-quest", 4, 64, 8, 16, 131072, 2, 2, "rms",
                                    "bf16", True),
    # 3-bit codes (two bit planes) on the batch-64 and prefill shapes
    "qwen3-8b-b64-16k-3bit": Workload("qwen3-8b-b64-16k-3bit", 2, 32, 8, 64, 16384, 3, 3, "percentile",
                                      "bf16", True),
    "prefill-8x32k-3bit": Workload("prefill-8x32k-3bit", 3, 8, 8, 1, 32768, 3, 3,
                                   "percentile", "bf16", True),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values.  Finite inputs."""
    f = np.ascontiguousarray(x, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the workload's input type ("f32", "bf16" or "f16"), as fp32."""
    x = np.asarray(x, np.float32)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    return x


def haar_orthogonal(d: int, rng: np.random.Generator) -> np.ndarray:
    z = rng.standard_normal((d, d))
    q, r = np.linalg.qr(z)
    return q * np.sign(np.diag(r))


def spectrum(d: int = HEAD_DIM) -> np.ndarray:
    return DECAY ** np.arange(d, dtype=np.float64)


def basis(config: int, role: int, head: int) -> np.ndarray:
    return haar_orthogonal(HEAD_DIM, rng_for(config, role, head))


def outlier_channels(config: int, head: int) -> np.ndarray:
    return np.sort(rng_for(config, ROLE_OUTLIER, head).choice(HEAD_DIM, N_OUTLIERS, replace=False))


def sigma_draw(n: int, u: np.ndarray, rng: np.random.Generator, outliers=None) -> np.ndarray:
    """n draws of N(0, U diag(lam) U^T), optional outlier channels scaled by 10, fp32."""
    z = rng.standard_normal((n, HEAD_DIM))
    x = (z * np.sqrt(spectrum())) @ u.T
    if outliers is not None:
        x[:, outliers] *= OUTLIER_STD
    return x.astype(np.float32)


def keys(config: int, head: int, n: int, offset_seed: int = 0) -> np.ndarray:
    u = basis(config, ROLE_K_BASIS, head)
    return sigma_draw(n, u, rng_for(config, ROLE_K_DRAW, head + offset_seed),
                      outlier_channels(config, head))


def values(config: int, head: int, n: int, offset_seed: int = 0) -> np.ndarray:
    u = basis(config, ROLE_V_BASIS, head)
    return sigma_draw(n, u, rng_for(config, ROLE_V_DRAW, head + offset_seed),
                      outlier_channels(config, 100 + head))


def queries(config: int, head_q: int, n: int, offset_seed: int = 0) -> np.ndarray:
    u = basis(config, ROLE_Q_BASIS, head_q)
    return sigma_draw(n, u, rng_for(config, ROLE_Q_DRAW, head_q + offset_seed))


def calibration_set(config: int, head_kv: int, group: int, n: int = 1024):
    """(K_cal [n,128], Q_cal [group,n,128]) for one KV head, independent of the cache draws."""
    k = sigma_draw(n, basis(config, ROLE_K_BASIS, head_kv), rng_for(config, ROLE_CAL_K, head_kv),
                   outlier_channels(config, head_kv))
    q = np.stack([sigma_draw(n, basis(config, ROLE_Q_BASIS, head_kv * group + g),
                             rng_for(config, ROLE_CAL_Q, head_kv * group + g))
                  for g in range(group)])
    return k, q


def kv_tokens(w: Workload, n: int, seq: int = 0):
    """K and V for n tokens of all KV heads: [n, Hkv, 128] each, in the workload's dtype.
    `seq` selects an independent draw (a different sequence of the batch)."""
    k = np.stack([keys(w.config, h, n, offset_seed=97 * seq) for h in range(w.heads_kv)], axis=1)
    v = np.stack([values(w.config, h, n, offset_seed=97 * seq) for h in range(w.heads_kv)], axis=1)
    return to_dtype(k, w.dtype), to_dtype(v, w.dtype)


def decode_queries(w: Workload, batch: int | None = None) -> np.ndarray:
    """One query per (sequence, query head): [B, Hq, 128] in the workload's dtype."""
    b = w.batch if batch is None else batch
    q = np.stack([queries(w.config, g, b, offset_seed=5000) for g in range(w.heads_q)], axis=1)
    return to_dtype(q, w.dtype)


def contiguous_block_table(batch: int, pages_per_seq: int) -> np.ndarray:
    """Sequence b owns pages b*P .. b*P+P-1 in order (benchmark layout)."""
    return np.arange(batch * pages_per_seq, dtype=np.int32).reshape(batch, pages_per_seq)


def shuffled_block_table(batch: int, pages_per_seq: int, num_pages: int,
                         rng: np.random.Generator) -> np.ndarray:
    """Distinct pages drawn at random from a pool of num_pages (test layout)."""
    perm = rng.permutation(num_pages)[: batch * pages_per_seq]
    return perm.astype(np.int32).reshape(batch, pages_per_seq)


def slots_for(block_table: np.ndarray, seq_lens, page_tokens: int = 64) -> np.ndarray:
    """Slot of every cached token, sequence-major: [sum(seq_lens)] int64."""
    out = []
    for b, n in enumerate(seq_lens):
        t = np.arange(int(n))
        out.append(block_table[b, t // page_tokens].astype(np.int64) * page_tokens + t % page_tokens)
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def random_packed_pool(rng: np.random.Generator, num_pages: int, kv_heads: int, bits: int,
                       scale_range=(2.0 ** -6, 2.0 ** -2), zero_range=(-2.0, 0.0)) -> np.ndarray:
    """A page pool of uniformly random codes with random but finite fp16 scales/zeros.
    Used to test the read path on caches of any size without running the write path."""
    code_bytes = 64 * HEAD_DIM * bits // 8
    block = code_bytes + 256
    pool = rng.integers(0, 256, size=(num_pages, kv_heads, block), dtype=np.uint8)
    s = rng.uniform(*scale_range, size=(num_pages, kv_heads, 64)).astype(np.float16)
    z = rng.uniform(*zero_range, size=(num_pages, kv_heads, 64)).astype(np.float16)
    pool[:, :, code_bytes:code_bytes + 128] = s.view(np.uint8).reshape(num_pages, kv_heads, 128)
    pool[:, :, code_bytes + 128:] = z.view(np.uint8).reshape(num_pages, kv_heads, 128)
    return pool


def kv_tokens_torch(w: Workload, n: int, device, seq: int = 0):
    """Large-scale variant of kv_tokens drawn with torch's generator on `device`
    (same distribution, different stream of numbers).  Returns bf16/fp32 tensors."""
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ks, vs = [], []
    lam = torch.tensor(np.sqrt(spectrum()), dtype=torch.float32, device=device)
    for h in range(w.heads_kv):
        for role_b, role_d, lst, oh in ((ROLE_K_BASIS, ROLE_K_DRAW, ks, h),
                                        (ROLE_V_BASIS, ROLE_V_DRAW, vs, 100 + h)):
            u = torch.tensor(basis(w.config, role_b, h), dtype=torch.float32, device=device)
            g = torch.Generator(device=device)
            g.manual_seed(seed_for(w.config, role_d, h) + 7919 * seq)
            z = torch.randn((n, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
            x = (z * lam) @ u.T
            x[:, torch.as_tensor(outlier_channels(w.config, oh), device=device)] *= OUTLIER_STD
            lst.append(x.to(dt))
    return torch.stack(ks, dim=1), torch.stack(vs, dim=1)
