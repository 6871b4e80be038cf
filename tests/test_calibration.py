"""WUSH key-transform calibration: pins of the fp64 reference (oracle/wush.py) against
the properties the pages state, and parity of the package's calibration with it.

Agreement with the paper's own (unprinted) Eq. (1) is parity unpinned; what is pinned
is every property the pages give for it."""
import numpy as np
import pytest

from decode_attention_kvq_amd import calib, synth
from oracle import wush


def _stats(seed=0, d=128, n=1024, g=4):
    k_cal, q_cal = synth.calibration_set(seed, 0, g, n)
    return k_cal, q_cal


def _trace_product(t, m, h):
    ti = np.linalg.inv(t)
    return np.trace(t.T @ m @ t) * np.trace(ti @ h @ ti.T)


def test_hadamard_reference():
    hd = wush.hadamard(128)
    assert np.allclose(hd @ hd.T, np.eye(128), atol=1e-14)
    assert np.allclose(np.abs(hd), 1 / np.sqrt(128))
    assert np.allclose(calib.sylvester_hadamard(128), hd)


def test_trace_product_attains_nuclear_bound():
    """App. B.2: undamped, WUSH attains min over invertible T of tr(T^T M T) tr(T^-1 H T^-T),
    which is (sum_i sigma_i)^2 with sigma_i^2 the eigenvalues of M H."""
    k_cal, q_cal = _stats(1)
    m, h = wush.statistics(k_cal, q_cal)
    t = wush.wush_from_stats(m, h, gamma=0.0)
    bound = np.sum(np.sqrt(np.clip(np.linalg.eigvals(m @ h).real, 0, None))) ** 2
    assert abs(_trace_product(t, m, h) - bound) < 1e-9 * bound
    rng = np.random.default_rng(0)
    for _ in range(300):
        r = rng.standard_normal((128, 128))
        if rng.random() < 0.5:
            r = t @ (np.eye(128) + 0.05 * r / np.sqrt(128))      # perturbations of the optimum
        assert _trace_product(r, m, h) >= bound * (1 - 1e-9)
    # orthogonal transforms leave both traces alone: tr(M) tr(H), which is larger here
    assert _trace_product(np.eye(128), m, h) > 1.05 * bound


def test_orthogonal_only_when_proportional():
    """App. B.2: an orthogonal T is optimal only if M is proportional to H; then WUSH itself
    is orthogonal up to the scalar."""
    k_cal, _ = _stats(2)
    m = k_cal.T.astype(np.float64) @ k_cal / len(k_cal)
    t = wush.wush_from_stats(m, 3.7 * m, gamma=0.0)
    tt = t.T @ t
    assert np.allclose(tt, tt[0, 0] * np.eye(128), atol=1e-9 * tt[0, 0])
    k_cal, q_cal = _stats(3)
    m, h = wush.statistics(k_cal, q_cal)
    t = wush.wush_from_stats(m, h, gamma=0.0)
    tt = t.T @ t
    assert not np.allclose(tt, tt[0, 0] * np.eye(128), atol=1e-2 * tt[0, 0])


@pytest.mark.parametrize("gamma", [0.0, 0.01])
def test_rescaling_invariance(gamma):
    """§3: WUSH does not change when M and H are rescaled independently."""
    k_cal, q_cal = _stats(4)
    t = wush.wush_transform(k_cal, q_cal, gamma=gamma)
    t2 = wush.wush_transform(k_cal.astype(np.float64) * 3.0, q_cal * 0.25, gamma=gamma)
    assert np.allclose(t, t2, rtol=0, atol=1e-8 * np.abs(t).max())


def test_norm_preserved_exactly_when_undamped():
    """§3: the scalar preserves the transformed tensor's Frobenius norm when gamma = 0."""
    k_cal, q_cal = _stats(5)
    k = k_cal.astype(np.float64)
    t = wush.wush_transform(k_cal, q_cal, gamma=0.0)
    assert abs(np.linalg.norm(k @ t) / np.linalg.norm(k) - 1) < 1e-12
    t = wush.wush_transform(k_cal, q_cal, gamma=0.01)
    assert abs(np.linalg.norm(k @ t) / np.linalg.norm(k) - 1) < 0.05


def test_balanced_and_equal_channel_variance():
    """The transformed key Gram and the transformed query Hessian are proportional, and the
    Hadamard factor gives every transformed key channel the same variance."""
    k_cal, q_cal = _stats(6)
    m, h = wush.statistics(k_cal, q_cal)
    t = wush.wush_from_stats(m, h, gamma=0.0)
    ti = np.linalg.inv(t)
    a, b = t.T @ m @ t, ti @ h @ ti.T
    assert np.allclose(a / np.trace(a), b / np.trace(b), atol=1e-10)
    dg = np.diag(a)
    assert np.allclose(dg, dg.mean(), rtol=1e-9)


def test_bf16_rounding_reference():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(100000) * np.exp2(rng.integers(-20, 20, 100000))
    r = wush.bf16_round(x).astype(np.float64)
    # brute force: nearest of the two bf16 neighbours, ties to the even mantissa
    m, e = np.frexp(x)
    lo = np.floor(m * 256) / 256 * np.exp2(e)
    hi = np.ceil(m * 256) / 256 * np.exp2(e)
    dlo, dhi = np.abs(x - lo), np.abs(hi - x)
    even_lo = (np.floor(np.abs(m) * 256) % 2 == 0)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(even_lo ^ (x < 0), lo, hi)))
    assert np.array_equal(r, pick)
    assert np.array_equal(calib.round_bf16(x).astype(np.float64), r)


@pytest.mark.parametrize("gamma", [0.0, 0.01])
def test_package_calibration_matches_reference(gamma):
    for head in range(3):
        k_cal, q_cal = synth.calibration_set(1, head, 4)
        t_ref = wush.wush_transform(k_cal, q_cal, gamma=gamma)
        t_pkg = calib.wush(*calib.key_statistics(k_cal, q_cal), gamma=gamma)
        assert np.allclose(t_pkg, t_ref, rtol=0, atol=1e-9 * np.abs(t_ref).max())
        ts, tinv = calib.calibrate_key_transform(k_cal, q_cal, gamma=gamma)
        tb = wush.bf16_round(t_ref)
        assert np.mean(ts != tb) < 1e-3           # a rounding tie may fall either way
        assert np.allclose(tinv, wush.inverse_transpose(ts), rtol=1e-6, atol=1e-7)


def test_fp16_stored_transform():
    """For fp16 inputs the transform is stored as fp16 values (what the write path receives),
    and T_inv_T is the inverse transpose of exactly that stored matrix."""
    k_cal, q_cal = synth.calibration_set(1, 0, 4)
    t_ref = wush.wush_transform(k_cal, q_cal)
    ts, tinv = calib.calibrate_key_transform(k_cal, q_cal, store_f16=True)
    assert np.array_equal(ts.astype(np.float16).astype(np.float32), ts)       # fp16 values
    assert np.max(np.abs(ts - t_ref)) <= np.abs(t_ref).max() * 2.0 ** -11      # rounded, not rescaled
    assert np.allclose(tinv, wush.inverse_transpose(ts), rtol=1e-6, atol=1e-7)
