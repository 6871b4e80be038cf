"""fp64 reference construction of the WUSH key transform (test infrastructure only).

Follows "WUSH-KV: KV Cache Quantization with Data-Adaptive Transforms" (summary page):
  §3    the transform is built from the Gram matrix M of the quantized tensor and the
        Hessian H of its product partner; damping gamma makes both positive definite; a
        scalar keeps the transformed tensor's Frobenius norm (exactly at gamma = 0); the
        result does not change when M and H are rescaled independently.
  §4.2  one key transform per KV head, from the cached keys' Gram matrix and a local
        surrogate Hessian (here: the summed second moment of the query heads that read
        this KV head, since a key error e moves the logit by q.e).
  App. B.2  at gamma = 0 the transform minimises tr(T^T M T) * tr(T^-1 H T^-T) over all
        invertible T; an orthogonal T reaches that minimum only when M is proportional
        to H.

The pages do not print the formula.  The reading used here is the closed form that has
all of the properties above:

    T0 = M^-1/2 U S^1/2,  with  M^1/2 H^1/2 = U S V^T  (SVD, symmetric square roots)
    T  = c T0 Hd,         c^2 = tr(M) / tr(S),  Hd = normalised Sylvester Hadamard

Each column of T0 is signed so that its largest-magnitude entry is positive.  Hd is an
orthogonal factor the unclipped loss cannot see; it gives every transformed channel the
same variance, which a per-token group clip needs ("sensitivity-balanced", App. B.3).
Agreement with the paper's own Eq. (1) is parity unpinned: only the properties are.

This module computes through eigendecompositions; the package's calibration uses a
Cholesky/SVD route.  The two are compared in tests/test_calibration.py.
"""
from __future__ import annotations

import numpy as np


def hadamard(d: int) -> np.ndarray:
    """Normalised Sylvester Hadamard matrix (d a power of two)."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == d
    return h / np.sqrt(d)


def _sym_sqrt(a: np.ndarray) -> np.ndarray:
    w, v = np.linalg.eigh(a)
    return (v * np.sqrt(w)) @ v.T


def damp(a: np.ndarray, gamma: float) -> np.ndarray:
    """a + gamma * tr(a)/d * I (damping relative to the mean eigenvalue)."""
    d = a.shape[0]
    return a + gamma * np.trace(a) / d * np.eye(d)


def statistics(k_cal: np.ndarray, q_cal: np.ndarray):
    """M = K^T K / N for the KV head's keys; H = sum over its query heads of Q^T Q / N.

    k_cal: [N, d]; q_cal: [G, N, d]."""
    k = np.asarray(k_cal, np.float64)
    q = np.asarray(q_cal, np.float64)
    m = k.T @ k / k.shape[0]
    h = sum(qg.T @ qg for qg in q) / q.shape[1]
    return m, h


def wush_from_stats(m: np.ndarray, h: np.ndarray, gamma: float = 0.01,
                    use_hadamard: bool = True) -> np.ndarray:
    d = m.shape[0]
    mg, hg = damp(m, gamma), damp(h, gamma)
    ms, hs = _sym_sqrt(mg), _sym_sqrt(hg)
    u, s, _ = np.linalg.svd(ms @ hs)
    t0 = np.linalg.inv(ms) @ u * np.sqrt(s)
    idx = np.argmax(np.abs(t0), axis=0)
    t0 = t0 * np.sign(t0[idx, np.arange(d)])
    c = np.sqrt(np.trace(m) / np.sum(s))
    t = c * t0
    return t @ hadamard(d) if use_hadamard else t


def wush_transform(k_cal, q_cal, gamma: float = 0.01, use_hadamard: bool = True) -> np.ndarray:
    m, h = statistics(k_cal, q_cal)
    return wush_from_stats(m, h, gamma, use_hadamard)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (8 significant bits, ties to even) in one step,
    returned as fp32.  Finite values inside the bf16 normal range only."""
    u = np.ascontiguousarray(x, np.float64).view(np.uint64)
    drop = np.uint64(45)                       # 52 fraction bits -> 7
    half = np.uint64((1 << 44) - 1)
    u = (u + half + ((u >> drop) & np.uint64(1))) & ~np.uint64((1 << 45) - 1)
    return u.view(np.float64).astype(np.float32)


def inverse_transpose(t_stored: np.ndarray) -> np.ndarray:
    """T^-T of the transform exactly as stored (e.g. after bf16 rounding), fp64 -> fp32."""
    return np.linalg.inv(np.asarray(t_stored, np.float64)).T.astype(np.float32)
