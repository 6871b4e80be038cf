"""Host-side (offline) calibration of the per-KV-head key and value transforms.

Follows "WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms":
  §3    the transform is built from two covariance-type matrices, one per operand of
        the product: the Gram matrix M of the quantized tensor (the cached keys) and
        the Hessian H of its partner; damping makes both positive definite; a scalar keeps
        the Frobenius norm (exactly when undamped); rescaling M or H changes nothing.
  §4.2  one key transform per KV head, with a local surrogate Hessian.  For keys the
        partner is the query: a key error e moves the logit of query q by q.e, so
        H = sum over the query heads that read the KV head of E[q^T q].
  App. B.2  undamped, the transform minimises tr(T^T M T) tr(T^-1 H T^-T).
  §4.2  the value transform comes from the values' Gram matrix and the Hessian of the
        output projection, and is folded into W_V and W_O (no read-time cost).

The formula itself is not printed on the pages; this module uses the closed form that
has every stated property (balanced: T^T M T and T^-1 H T^-T are both diagonal-equal):

    M + g tr(M)/d I = B B^T,  H + g tr(H)/d I = A A^T     (Cholesky)
    B^T A = U S V^T                                      (SVD)
    T = c * B^-T U S^1/2 * Hd,  c^2 = tr(M)/tr(S)

with each column of B^-T U S^1/2 signed so that its largest-magnitude entry is
positive, and Hd the normalised Sylvester-Hadamard matrix, an orthogonal factor the
unclipped loss does not see that equalises the transformed channels' variances for the
per-token group clip.  Everything is fp64; the stored transform is rounded to bf16 and
the query side uses the exact inverse-transpose of the rounded matrix.
"""
from __future__ import annotations

import numpy as np

DEFAULT_GAMMA = 0.01


def sylvester_hadamard(d: int) -> np.ndarray:
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    return h / np.sqrt(d)


def key_statistics(k_cal: np.ndarray, q_cal: np.ndarray):
    """Gram matrix of the keys and the summed query second moment of one KV head.

    k_cal: [N, d] post-RoPE keys; q_cal: [G, N_q, d] post-RoPE queries of the G query
    heads that read this KV head."""
    k = np.asarray(k_cal, dtype=np.float64)
    q = np.asarray(q_cal, dtype=np.float64)
    if q.ndim == 2:
        q = q[None]
    gram = np.einsum("nc,nd->cd", k, k) / k.shape[0]
    hess = np.einsum("gnc,gnd->cd", q, q) / q.shape[1]
    return gram, hess


def wush(gram: np.ndarray, hess: np.ndarray, gamma: float = DEFAULT_GAMMA,
         hadamard: bool = True) -> np.ndarray:
    d = gram.shape[0]
    eye = np.eye(d)
    b = np.linalg.cholesky(gram + gamma * np.trace(gram) / d * eye)
    a = np.linalg.cholesky(hess + gamma * np.trace(hess) / d * eye)
    u, s, _ = np.linalg.svd(b.T @ a)
    t0 = np.linalg.solve(b.T, u) * np.sqrt(s)
    lead = np.abs(t0).argmax(axis=0)
    t0 *= np.sign(t0[lead, np.arange(d)])
    t = np.sqrt(np.trace(gram) / s.sum()) * t0
    return t @ sylvester_hadamard(d) if hadamard else t


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 (round to nearest even, directly from fp64), as fp32 values."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m 2^e, |m| in [0.5, 1)
    return (np.round(m * 256.0) / 256.0 * np.exp2(e)).astype(np.float32)


def calibrate_key_transform(k_cal: np.ndarray, q_cal: np.ndarray, gamma: float = DEFAULT_GAMMA,
                            hadamard: bool = True, store_bf16: bool = True, store_f16: bool = False):
    """Returns (T, T_inv_T) for one KV head as fp32 arrays [d, d].

    T is what the write path applies (k' = k T); when store_f16 it holds fp16 values (for
    fp16 inputs, whose T is passed as fp16), else when store_bf16 bf16 values.
    T_inv_T = (T^-1)^T of exactly that stored T, for the read path (q' = q T^-T)."""
    t = wush(*key_statistics(k_cal, q_cal), gamma=gamma, hadamard=hadamard)
    if store_f16:
        t_store = np.asarray(t, dtype=np.float64).astype(np.float16).astype(np.float32)
    else:
        t_store = round_bf16(t) if store_bf16 else t.astype(np.float32)
    t_store = np.ascontiguousarray(t_store)
    t_inv_t = np.ascontiguousarray(np.linalg.inv(t_store.astype(np.float64)).T, dtype=np.float32)
    return t_store, t_inv_t


def calibrate_all_heads(k_cal_heads, q_cal_heads, **kw):
    """Stacks calibrate_key_transform over KV heads: returns ([H,d,d], [H,d,d])."""
    pairs = [calibrate_key_transform(k, q, **kw) for k, q in zip(k_cal_heads, q_cal_heads)]
    return np.stack([p[0] for p in pairs]), np.stack([p[1] for p in pairs])


# --------------------------------------------------------------------------------------
# Value side ("WUSH-KV" §4.2: the value transform is folded into W_V and W_O, so the cache
# holds v T_V and the attention output stays in that basis until W_O absorbs T_V^-1).
# --------------------------------------------------------------------------------------

def value_statistics(v_cal: np.ndarray, w_o_blocks: np.ndarray):
    """Gram matrix of one KV head's values and the Hessian of their product partner.

    v_cal: [N, d] values (before any fold); w_o_blocks: [G, d, d_model], the rows of the
    output projection that the G query heads reading this KV head multiply.  Head g adds
    o_g W_O,g to the layer output with o_g a convex combination of value rows, so an error
    e in a value row moves the output by (p e) W_O,g: the surrogate Hessian is
    H = sum_g W_O,g W_O,g^T."""
    v = np.asarray(v_cal, dtype=np.float64)
    w = np.asarray(w_o_blocks, dtype=np.float64)
    if w.ndim == 2:
        w = w[None]
    gram = np.einsum("nc,nd->cd", v, v) / v.shape[0]
    hess = np.einsum("gcm,gdm->cd", w, w)
    return gram, hess


def calibrate_value_transform(v_cal: np.ndarray, w_o_blocks: np.ndarray, gamma: float = DEFAULT_GAMMA,
                              hadamard: bool = True) -> np.ndarray:
    """T_V [d, d] (fp64) for one KV head: the same construction as the key transform, with
    the values' Gram matrix and the output projection's Hessian."""
    return wush(*value_statistics(v_cal, w_o_blocks), gamma=gamma, hadamard=hadamard)


def fold_value_transform(w_v: np.ndarray, w_o_blocks: np.ndarray, t_v: np.ndarray):
    """Folds T_V into the projections: W_V' = W_V T_V (so the cached values are v T_V) and
    W_O,g' = T_V^-1 W_O,g (so o' W_O,g' = o W_O,g for the transformed-basis output o').

    w_v: [d_model, d]; w_o_blocks: [G, d, d_model].  Returns (W_V', W_O') in fp64."""
    t = np.asarray(t_v, dtype=np.float64)
    w_v_f = np.asarray(w_v, dtype=np.float64) @ t
    w_o_f = np.stack([np.linalg.solve(t, w) for w in np.asarray(w_o_blocks, dtype=np.float64)])
    return w_v_f, w_o_f
