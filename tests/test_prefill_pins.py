"""Pins of the oracle's causal many-query forward (oracle.prefill).

Each token attends to its own cache position and everything before it. The
pins check the oracle's prefill against: a library causal softmax attention
when W_R = 0 (torch SDPA in float64, with and without a cached prefix),
causality (changing keys after a token leaves its output unchanged), the
one-token case (the decode oracle, itself pinned), chunked prefill, and a
pure-Python brute force. ``test_planted_mistakes`` checks that off-by-one
masks, a dropped prefix and a probe taken from the wrong token are caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import parallax_oracle as po


def _case(seed, B=2, T=6, P=(0, 3), Hq=4, Hkv=2, d=5):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, Hq, d))
    rho = r.standard_normal((B, T, Hq, d)) * 0.3
    K = [r.standard_normal((Hkv, P[b] + T, d)) for b in range(B)]
    V = [r.standard_normal((Hkv, P[b] + T, d)) for b in range(B)]
    return q, rho, K, V, np.array(P)


def pin_wr_zero_is_causal_sdpa():
    """rho = 0: torch SDPA over the cached prefix plus a causal block, float64.
    The mask is built here as a lower-triangular band shifted by the prefix."""
    q, rho, K, V, P = _case(0)
    B, T, Hq, d = q.shape
    Hkv = K[0].shape[0]
    got = oracle.prefill(q, np.zeros_like(rho), K, V, P, Hkv)
    for b in range(B):
        n = P[b] + T
        allowed = np.tril(np.ones((T, n), dtype=bool), k=int(P[b]))
        qt = torch.from_numpy(q[b].transpose(1, 0, 2).copy())              # [Hq, T, d]
        kt = torch.from_numpy(np.repeat(K[b], Hq // Hkv, axis=0).copy())   # [Hq, n, d]
        vt = torch.from_numpy(np.repeat(V[b], Hq // Hkv, axis=0).copy())
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=torch.from_numpy(allowed)).numpy()
        np.testing.assert_allclose(got[b], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)
    # no prefix: the library's own causal mask
    q0, _, K0, V0, _ = _case(1, P=(0, 0))
    got0 = oracle.prefill(q0, np.zeros_like(q0), K0, V0, np.array([0, 0]), Hkv)
    for b in range(2):
        qt = torch.from_numpy(q0[b].transpose(1, 0, 2).copy())
        kt = torch.from_numpy(np.repeat(K0[b], Hq // Hkv, axis=0).copy())
        vt = torch.from_numpy(np.repeat(V0[b], Hq // Hkv, axis=0).copy())
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).numpy()
        np.testing.assert_allclose(got0[b], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def pin_causality():
    """Changing keys and values after position P + t0 leaves tokens 0..t0
    unchanged and changes token t0 + 1."""
    q, rho, K, V, P = _case(2)
    Hkv = K[0].shape[0]
    base = oracle.prefill(q, rho, K, V, P, Hkv)
    t0 = 2
    K2 = [k.copy() for k in K]
    V2 = [v.copy() for v in V]
    for b in range(len(K)):
        K2[b][:, P[b] + t0 + 1:] += 1.5
        V2[b][:, P[b] + t0 + 1:] -= 0.7
    pert = oracle.prefill(q, rho, K2, V2, P, Hkv)
    np.testing.assert_array_equal(pert[:, :t0 + 1], base[:, :t0 + 1])
    assert np.abs(pert[:, t0 + 1] - base[:, t0 + 1]).min() > 1e-6


def pin_last_token_is_decode():
    """Every token equals the decode oracle over its prefix (n = P + t + 1)
    with its own query and probe; the last token sees the whole cache."""
    q, rho, K, V, P = _case(3)
    B, T, Hq, d = q.shape
    Hkv = K[0].shape[0]
    got = oracle.prefill(q, rho, K, V, P, Hkv)
    for t in (0, T // 2, T - 1):
        lens = P + t + 1
        ref = oracle.decode(q[:, t], rho[:, t], K, V, lens, Hkv)
        np.testing.assert_allclose(got[:, t], ref, rtol=0, atol=0)


def pin_chunked_prefill():
    """Prefill of T tokens equals a prefill of the first T1 tokens followed by
    a prefill of the rest with the prefix grown by T1."""
    q, rho, K, V, P = _case(4)
    Hkv = K[0].shape[0]
    full = oracle.prefill(q, rho, K, V, P, Hkv)
    T1 = 4
    a = oracle.prefill(q[:, :T1], rho[:, :T1], K, V, P, Hkv)
    b = oracle.prefill(q[:, T1:], rho[:, T1:], K, V, P + T1, Hkv)
    np.testing.assert_allclose(np.concatenate([a, b], axis=1), full, rtol=0, atol=0)


def pin_bruteforce():
    """Pure-Python loops on a tiny case: explicit weights, means, covariance."""
    q, rho, K, V, P = _case(5, B=1, T=3, P=(2,), Hq=2, Hkv=1, d=2)
    got = oracle.prefill(q, rho, K, V, P, 1)
    d = 2
    for t in range(3):
        n = 2 + t + 1
        for h in range(2):
            s = [sum(q[0, t, h, i] * K[0][0, j, i] for i in range(d)) / math.sqrt(d) for j in range(n)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            w = [x / sum(e) for x in e]
            kb = [sum(w[j] * K[0][0, j, i] for j in range(n)) for i in range(d)]
            vb = [sum(w[j] * V[0][0, j, i] for j in range(n)) for i in range(d)]
            out = []
            for a in range(d):
                corr = 0.0
                for c in range(d):
                    cov = sum(w[j] * (V[0][0, j, a] - vb[a]) * (K[0][0, j, c] - kb[c]) for j in range(n))
                    corr += cov * rho[0, t, h, c]
                out.append(vb[a] - corr)
            np.testing.assert_allclose(got[0, t, h], out, rtol=0, atol=1e-12)


ALL_PINS = [pin_wr_zero_is_causal_sdpa, pin_causality, pin_last_token_is_decode,
            pin_chunked_prefill, pin_bruteforce]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_prefill_rows_match_prefill():
    q, rho, K, V, P = _case(6)
    full = oracle.prefill(q, rho, K, V, P, 2)
    rows = [(0, 0, 0), (1, 5, 3), (1, 2, 1)]
    np.testing.assert_array_equal(oracle.prefill_rows(q, rho, K, V, P, 2, rows),
                                  np.stack([full[b, t, h] for b, t, h in rows]))


# ---------------------------------------------------------------- planted mistakes
def _prefill_variant(shift=0, ignore_prefix=False, first_token_rho=False):
    def prefill(q, rho, K_parts, V_parts, prefix_lens, Hkv):
        qa, ra = po._f64(q), po._f64(rho)
        B, T, Hq, d = qa.shape
        out = np.zeros((B, T, Hq, d))
        for b in range(B):
            for t in range(T):
                n = (0 if ignore_prefix else int(prefix_lens[b])) + t + 1 + shift
                for h in range(Hq):
                    g = h // (Hq // Hkv)
                    r = ra[b, 0, h] if first_token_rho else ra[b, t, h]
                    out[b, t, h] = po.decode_head(qa[b, t, h], r, K_parts[b][g][:max(n, 0)],
                                                  V_parts[b][g][:max(n, 0)])
        return out
    return prefill


MUTANTS = {
    "mask_excludes_self": _prefill_variant(shift=-1),
    "mask_includes_next": _prefill_variant(shift=1),
    "prefix_ignored": _prefill_variant(ignore_prefix=True),
    "probe_of_first_token": _prefill_variant(first_token_rho=True),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name, monkeypatch):
    monkeypatch.setattr(po, "prefill", MUTANTS[name])
    monkeypatch.setattr(oracle, "prefill", MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
