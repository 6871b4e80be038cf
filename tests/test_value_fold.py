"""Value-transform calibration and fold ("WUSH-KV" §4.2: T_V is folded into W_V and W_O).

Pins, on the CPU:
  * the fold leaves the layer's attention output unchanged (o' W_O' = o W_O, closed form);
  * the package's T_V equals the fp64 reference construction (oracle/wush.py, eigen
    route) built from the same value Gram matrix and output-projection Hessian, up to
    the sign of each column;
  * with an output projection of uneven singular values, quantizing the folded values
    (2-bit, the encoder's percentile clip) gives a smaller error after W_O than quantizing
    the raw values, on the Sigma-model values (the direction the method claims);
  * end to end through the encoder: the output in the transformed basis, multiplied by
    the folded W_O, approximates the unquantized layer output.
"""
import numpy as np

import oracle
from decode_attention_kvq_amd import calib, synth
from oracle import wush as ref

D, DM, G = 128, 512, 4


def _w_o(rng, spread=20.0):
    """[G, d, d_model] output-projection blocks with singular values spread over `spread`."""
    blocks = []
    for _ in range(G):
        u = synth.haar_orthogonal(D, rng)
        v = np.linalg.qr(rng.standard_normal((DM, D)))[0].T
        s = np.geomspace(spread, 1.0, D)
        blocks.append((u * s) @ v / np.sqrt(D))
    return np.stack(blocks)


def _dequant(x, bits):
    c, s, z, _, _ = oracle.quantize_rows(x, bits)
    sf = oracle.f16_bits_to_f32(s)[:, None].astype(np.float64)
    zf = oracle.f16_bits_to_f32(z)[:, None].astype(np.float64)
    return c * sf + zf


def test_fold_preserves_layer_output():
    rng = np.random.default_rng(1)
    w_v = rng.standard_normal((DM, D)) / np.sqrt(DM)
    w_o = _w_o(rng)
    t = calib.calibrate_value_transform(rng.standard_normal((1024, D)), w_o)
    w_v2, w_o2 = calib.fold_value_transform(w_v, w_o, t)
    x = rng.standard_normal((40, DM))
    p = rng.dirichlet(np.ones(40), size=G)                 # one attention row per head
    for g in range(G):
        o = p[g] @ (x @ w_v)
        o2 = p[g] @ (x @ w_v2)                             # the cache holds x W_V T_V
        np.testing.assert_allclose(o2 @ w_o2[g], o @ w_o[g], rtol=0, atol=1e-10 * np.abs(o @ w_o[g]).max())


def test_value_transform_matches_reference():
    rng = np.random.default_rng(2)
    v = synth.values(1, 0, 2048)
    w_o = _w_o(rng)
    t = calib.calibrate_value_transform(v, w_o)
    m = v.astype(np.float64).T @ v.astype(np.float64) / v.shape[0]
    h = sum(w @ w.T for w in w_o.astype(np.float64))
    t_ref = ref.wush_from_stats(m, h)
    # columns agree up to sign (the Hadamard factor mixes them, so compare before it)
    hd = ref.hadamard(D)
    a, b = t @ hd.T, t_ref @ hd.T
    sign = np.sign(np.sum(a * b, axis=0))
    np.testing.assert_allclose(a * sign, b, rtol=0, atol=1e-8 * np.abs(b).max())


def test_folded_values_quantize_better_after_w_o():
    rng = np.random.default_rng(3)
    w_o = _w_o(rng)
    v_cal = synth.values(1, 0, 2048)
    v = synth.values(1, 0, 4096, offset_seed=7)
    t = calib.calibrate_value_transform(v_cal, w_o)
    err = {}
    for name, tv in (("identity", np.eye(D)), ("wush", t)):
        vt = (v.astype(np.float64) @ tv).astype(np.float32)
        e = (_dequant(vt, 2) - vt) @ np.linalg.inv(tv)          # the error seen in the raw basis
        err[name] = sum(np.sum((e @ w) ** 2) for w in w_o) / sum(np.sum((v @ w) ** 2) for w in w_o)
    assert err["wush"] < 0.5 * err["identity"], err


def test_transformed_basis_output_reaches_layer_output():
    """Attention over 4-bit codes of the folded values, then W_O' = T_V^-1 W_O: within 10%
    of the unquantized layer output, and at most a quarter of the error of 4-bit codes of
    the raw values (which the Sigma model's outlier channels dominate)."""
    rng = np.random.default_rng(4)
    w_o = _w_o(rng, spread=4.0)
    t = calib.calibrate_value_transform(synth.values(1, 0, 2048), w_o)
    v = synth.values(1, 0, 256, offset_seed=3)
    vt = (v.astype(np.float64) @ t).astype(np.float32)
    p = rng.dirichlet(np.ones(256) * 0.5, size=G)
    vq, vraw = _dequant(vt, 4), _dequant(v, 4)
    for g in range(G):
        exact = p[g] @ v.astype(np.float64) @ w_o[g]
        folded = (p[g] @ vq) @ np.linalg.solve(t, w_o[g])
        raw = (p[g] @ vraw) @ w_o[g]
        e_f = np.linalg.norm(folded - exact) / np.linalg.norm(exact)
        e_r = np.linalg.norm(raw - exact) / np.linalg.norm(exact)
        assert e_f <= 0.10 and e_f <= 0.25 * e_r, (g, e_f, e_r)
