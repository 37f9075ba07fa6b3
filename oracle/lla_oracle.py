"""fp64 CPU reference for exact local linear attention (LLA) — TEST INFRASTRUCTURE ONLY.

Like the Parallax oracle beside it, only the tests may import this module; the
product path never calls it and it shares no code with that path.

What it computes. Exact LLA asks for one linear solve per query, done with a
conjugate-gradient solver, and that solve carries a trade-off between
regularisation and expressivity (encorp.ai (de), section "Warum das Entfernen
des konjugierten Gradienten-Solvers ..."; the Polish version, section "Dlaczego
usunięcie solvera gradientów sprzężonych ..."). Parallax replaces the solve by
a probe learned from the layer input; softmax attention is the local-constant
estimate and the correction makes it local-linear (zubnet.ai (pt) and (fr),
first paragraph).

Reading taken (the pages do not print the system): local linear attention is
the softmax-weighted local linear regression of the values on the keys around
the query, v_j ~ a + B (k_j - q), read off at the query (the intercept a). The
normal equations give

    a = vbar - C rho*,   (Sigma_kk + lam I) rho* = kbar - q,

with w the softmax weights of the query, kbar/vbar the weighted means,
Sigma_kk = sum_j w_j (k_j - kbar)(k_j - kbar)^T the weighted key covariance,
C = sum_j w_j (v_j - vbar)(k_j - kbar)^T the KV covariance, and lam >= 0 a ridge
penalty on B (lam = 0 is the unregularised fit; lam -> infinity gives rho* -> 0
and plain softmax attention). So exact LLA is the Parallax output with the
probe replaced by the solved rho*. The solve here is the plain
conjugate-gradient method (Hestenes and Stiefel, 1952) on that symmetric
positive (semi-)definite d x d system.
"""
from __future__ import annotations

import numpy as np

from .parallax_oracle import _f64, kv_covariance, softmax_weights, weighted_means

__all__ = ["key_covariance", "conjugate_gradient", "lla_probe", "lla_decode_head",
           "lla_decode"]


def key_covariance(w: np.ndarray, K: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Softmax-weighted key covariance Sigma_kk = sum_j w_j (k_j - kbar)(k_j - kbar)^T."""
    Kc = K - kbar
    return (Kc * w[:, None]).T @ Kc


def conjugate_gradient(A: np.ndarray, b: np.ndarray, tol: float = 1e-13,
                       max_iter: int | None = None):
    """Solve A x = b for symmetric positive-definite A by conjugate gradients.

    Starts from x = 0. Each step moves along a search direction that is
    A-conjugate to all previous ones, with the exact line-search step length
    along it; the next direction is the new residual made A-conjugate to the last
    direction. Stops when ||r|| <= tol * ||b||. In exact arithmetic it ends after
    at most as many steps as A has distinct eigenvalues (so at most d).
    Returns (x, steps taken, final relative residual).
    """
    n = b.shape[0]
    if max_iter is None:
        max_iter = 10 * n
    x = np.zeros(n)
    r = b.copy()                 # residual b - A x at x = 0
    bnorm = np.linalg.norm(b)
    if bnorm == 0.0:
        return x, 0, 0.0
    p = r.copy()
    rr = r @ r
    steps = 0
    while steps < max_iter and np.sqrt(rr) > tol * bnorm:
        Ap = A @ p
        alpha = rr / (p @ Ap)    # minimises the A-norm error along p
        x = x + alpha * p
        r = r - alpha * Ap
        rr_new = r @ r
        beta = rr_new / rr       # makes the next direction A-conjugate to p
        p = r + beta * p
        rr = rr_new
        steps += 1
    return x, steps, float(np.sqrt(rr) / bnorm)


def lla_probe(q, K, lam: float, tol: float = 1e-13):
    """The solved probe rho* = (Sigma_kk + lam I)^{-1} (kbar - q) of one query,
    by conjugate gradients. q: [d]; K: [n, d], n >= 1. Returns (rho*, steps,
    relative residual)."""
    q = _f64(q)
    K = _f64(K)
    d = q.shape[0]
    w = softmax_weights(q, K)
    kbar = w @ K
    A = key_covariance(w, K, kbar) + lam * np.eye(d)
    return conjugate_gradient(A, kbar - q, tol=tol)


def lla_decode_head(q, K, V, lam: float, tol: float = 1e-13) -> np.ndarray:
    """Exact LLA output of one query: vbar - C rho*, rho* from lla_probe.
    n == 0 gives zeros (the same convention as the Parallax oracle)."""
    q = _f64(q)
    K = _f64(K)
    V = _f64(V)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    rho, _, _ = lla_probe(q, K, lam, tol)
    w = softmax_weights(q, K)
    kbar, vbar = weighted_means(w, K, V)
    return vbar - kv_covariance(w, K, V, kbar, vbar) @ rho


def lla_decode(q, K_parts, V_parts, seq_lens, Hkv: int, lam: float):
    """Exact LLA for every (sequence, query head): returns (out [B, Hq, d],
    rho* [B, Hq, d]). Same inputs and head map as the Parallax oracle's decode
    (query head h reads KV head h // (Hq / Hkv))."""
    qa = _f64(q)
    B, Hq, d = qa.shape
    G = Hq // Hkv
    lens = [int(n) for n in _f64(seq_lens)]
    out = np.zeros((B, Hq, d))
    rho = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            n = lens[b]
            Kb = _f64(K_parts[b][h // G][:n])
            Vb = _f64(V_parts[b][h // G][:n])
            if n == 0:
                continue
            rho[b, h] = lla_probe(qa[b, h], Kb, lam)[0]
            out[b, h] = lla_decode_head(qa[b, h], Kb, Vb, lam)
    return out, rho
