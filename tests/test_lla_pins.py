"""Pins of the exact local-linear-attention (LLA) reference (oracle/lla_oracle.py).

Exact LLA solves one linear system per query with conjugate gradients
(encorp.ai (de), section on removing the conjugate-gradient solver). Each pin
checks the reference against something fixed outside it: a library linear
solve, the finite-termination property of conjugate gradients, an independent
least-squares formulation of the local linear (ridge) fit, exactness on linear
data, the large-penalty limit (plain softmax attention) and a hand-worked
example. ``test_planted_mistakes`` plants plausible mistakes in the reference
and checks that a pin catches each.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import lla_oracle as lla


def _rng(seed):
    return np.random.default_rng(seed)


def _softmax_w(q, K):
    s = K @ q / math.sqrt(q.shape[0])
    w = np.exp(s - s.max())
    return w / w.sum()


# ---------------------------------------------------------------- pins
def pin_cg_matches_library_solve():
    """Random SPD systems: conjugate gradients agree with LAPACK's solve."""
    r = _rng(0)
    for d in (3, 16, 64):
        M = r.standard_normal((d, d))
        A = M @ M.T + 0.5 * np.eye(d)
        b = r.standard_normal(d)
        x, steps, res = lla.conjugate_gradient(A, b)
        ref = np.linalg.solve(A, b)
        assert res <= 1e-12
        np.testing.assert_allclose(x, ref, rtol=0, atol=1e-9 * np.abs(ref).max())


def pin_cg_finite_termination():
    """A = Q diag(lambda) Q^T with three distinct eigenvalues: conjugate
    gradients end in at most three steps, at x = Q diag(1/lambda) Q^T b."""
    r = _rng(1)
    d = 12
    Q, _ = np.linalg.qr(r.standard_normal((d, d)))
    lam = np.array([1.0] * 4 + [3.0] * 5 + [10.0] * 3)
    A = (Q * lam) @ Q.T
    b = r.standard_normal(d)
    x, steps, res = lla.conjugate_gradient(A, b, tol=1e-12)
    assert steps <= 3, steps
    np.testing.assert_allclose(x, (Q / lam) @ (Q.T @ b), rtol=0, atol=1e-10)


def pin_lla_ridge_least_squares():
    """The LLA output equals the intercept a of the softmax-weighted ridge fit
    min_{a,B} sum_j w_j |v_j - a - B (k_j - q)|^2 + lam |B|_F^2, solved here as an
    augmented least-squares problem (d extra rows sqrt(lam) e_i with zero
    targets; the intercept is not penalised)."""
    r = _rng(2)
    for d, n, lam in ((2, 9, 0.0), (3, 20, 0.05), (5, 40, 0.7), (8, 6, 2.0)):
        q = r.standard_normal(d)
        K = r.standard_normal((n, d))
        V = r.standard_normal((n, d))
        w = _softmax_w(q, K)
        X = np.hstack([np.ones((n, 1)), K - q]) * np.sqrt(w)[:, None]
        Y = V * np.sqrt(w)[:, None]
        if lam > 0:
            X = np.vstack([X, np.hstack([np.zeros((d, 1)), math.sqrt(lam) * np.eye(d)])])
            Y = np.vstack([Y, np.zeros((d, d))])
        coef, *_ = np.linalg.lstsq(X, Y, rcond=None)
        np.testing.assert_allclose(lla.lla_decode_head(q, K, V, lam), coef[0], rtol=0, atol=1e-9,
                                   err_msg=f"d={d} n={n} lam={lam}")


def pin_lla_exact_on_linear_data():
    """Values that are an exact affine function of the keys, v = a0 + M k: the
    unpenalised local linear estimate at the query is a0 + M q (a local linear
    fit reproduces affine data), which softmax attention does not."""
    r = _rng(3)
    for d, n in ((4, 30), (16, 100)):
        q = r.standard_normal(d)
        K = r.standard_normal((n, d))
        M = r.standard_normal((d, d))
        a0 = r.standard_normal(d)
        V = a0 + K @ M.T
        want = a0 + M @ q
        np.testing.assert_allclose(lla.lla_decode_head(q, K, V, 0.0), want, rtol=0, atol=1e-8)
        assert np.abs(oracle.decode_head(q, np.zeros(d), K, V) - want).max() > 1e-3


def pin_lla_large_penalty_is_softmax():
    """lam -> infinity: rho* ~ (kbar - q) / lam -> 0 and the output tends to
    plain softmax attention."""
    r = _rng(4)
    d, n, lam = 6, 25, 1e9
    q = r.standard_normal(d)
    K = r.standard_normal((n, d))
    V = r.standard_normal((n, d))
    w = _softmax_w(q, K)
    rho, _, _ = lla.lla_probe(q, K, lam)
    np.testing.assert_allclose(rho, (w @ K - q) / lam, rtol=1e-6, atol=0)
    np.testing.assert_allclose(lla.lla_decode_head(q, K, V, lam), w @ V, rtol=0, atol=1e-8)


# Hand-worked example, d = 1: q = 0 makes every score 0, so two keys k = 0, 2 get
# weights 1/2 each. kbar = 1, Sigma_kk = (1 + 1)/2 = 1. With values 0 and 3:
# vbar = 3/2 and C = ((-3/2)(-1) + (3/2)(1))/2 = 3/2. Then
# rho* = (kbar - q)/(Sigma_kk + lam) = 1/(1 + lam) and
# out = vbar - C rho* = 3/2 - (3/2)/(1 + lam): 0 at lam = 0 (the line v = 3k/2
# read at k = 0), 3/4 at lam = 1, 1/2 at lam = 1/2, 6/5 at lam = 4.
HAND = [(0.0, 0.0), (1.0, 0.75), (0.5, 0.5), (4.0, 1.2)]


def pin_lla_hand_example():
    q = np.array([0.0])
    K = np.array([[0.0], [2.0]])
    V = np.array([[0.0], [3.0]])
    for lam, want in HAND:
        rho, _, _ = lla.lla_probe(q, K, lam)
        np.testing.assert_allclose(rho, [1.0 / (1.0 + lam)], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lla.lla_decode_head(q, K, V, lam), [want], rtol=0, atol=1e-14)


def pin_lla_batch_matches_heads():
    """lla_decode over a GQA batch equals lla_decode_head per (sequence, head)
    with query head h reading KV head h // G; length 0 gives zeros."""
    r = _rng(5)
    B, Hq, Hkv, d = 3, 4, 2, 5
    lens = [7, 0, 12]
    q = r.standard_normal((B, Hq, d))
    K = [r.standard_normal((Hkv, n, d)) for n in lens]
    V = [r.standard_normal((Hkv, n, d)) for n in lens]
    out, rho = lla.lla_decode(q, K, V, np.array(lens), Hkv, 0.3)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            want = lla.lla_decode_head(q[b, h], K[b][g], V[b][g], 0.3) if lens[b] else np.zeros(d)
            np.testing.assert_allclose(out[b, h], want, rtol=0, atol=0)
    assert not out[1].any() and not rho[1].any()


ALL_PINS = [pin_cg_matches_library_solve, pin_cg_finite_termination, pin_lla_ridge_least_squares,
            pin_lla_exact_on_linear_data, pin_lla_large_penalty_is_softmax, pin_lla_hand_example,
            pin_lla_batch_matches_heads]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------------- planted mistakes
def _cg_variant(beta_inverted=False, residual_plus=False):
    def cg(A, b, tol=1e-13, max_iter=None):
        n = b.shape[0]
        max_iter = 10 * n if max_iter is None else max_iter
        x, r = np.zeros(n), b.copy()
        p, rr, steps = r.copy(), r @ r, 0
        bnorm = np.linalg.norm(b)
        while steps < max_iter and np.sqrt(rr) > tol * bnorm:
            Ap = A @ p
            alpha = rr / (p @ Ap)
            x = x + alpha * p
            r = r + alpha * Ap if residual_plus else r - alpha * Ap
            rr_new = r @ r
            beta = rr / rr_new if beta_inverted else rr_new / rr
            p = r + beta * p
            rr = rr_new
            steps += 1
        return x, steps, float(np.sqrt(rr) / bnorm)
    return cg


def _probe_variant(rhs_flip=False, drop_lam=False):
    def probe(q, K, lam, tol=1e-13):
        q, K = np.asarray(q, float), np.asarray(K, float)
        w = _softmax_w(q, K)
        kbar = w @ K
        A = lla.key_covariance(w, K, kbar) + (0.0 if drop_lam else lam) * np.eye(q.shape[0])
        return lla.conjugate_gradient(A, (q - kbar) if rhs_flip else (kbar - q), tol=tol)
    return probe


def _keycov_unweighted(w, K, kbar):
    Kc = K - K.mean(0)
    return Kc.T @ Kc / K.shape[0]


def _keycov_bessel(w, K, kbar):
    Kc = K - kbar
    n = K.shape[0]
    return (Kc * w[:, None]).T @ Kc * (n / (n - 1))


MUTANTS = {
    "cg_beta_inverted": ("conjugate_gradient", _cg_variant(beta_inverted=True)),
    "cg_residual_sign": ("conjugate_gradient", _cg_variant(residual_plus=True)),
    "rhs_sign": ("lla_probe", _probe_variant(rhs_flip=True)),
    "penalty_dropped": ("lla_probe", _probe_variant(drop_lam=True)),
    "unweighted_key_covariance": ("key_covariance", _keycov_unweighted),
    "bessel_key_covariance": ("key_covariance", _keycov_bessel),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(lla, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, np.linalg.LinAlgError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
