"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each pin checks the oracle against something the pages or the mathematics fix:
hand-worked examples (tests/golden/hand_examples.json), the W_R = 0 reduction to
a library softmax attention, the local-linear least-squares identity, closed
forms, invariances and a pure-Python brute force. ``test_planted_mistakes``
plants plausible mistakes in the oracle (on the CPU) and checks that at least
one pin catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import parallax_oracle as po

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- pins as functions
def pin_golden_decode():
    """Hand-derived worked examples (closed forms in the fixture)."""
    ex = json.load(open(GOLDEN))
    for case in ex["decode"]:
        q, K, V, rho = (np.array(case[k], dtype=np.float64) for k in ("q", "K", "V", "rho"))
        got = oracle.decode_head(q, rho, K, V)
        np.testing.assert_allclose(got, case["out"], rtol=0, atol=1e-12, err_msg=case["name"])
        got0 = oracle.decode_head(q, np.zeros_like(rho), K, V)
        np.testing.assert_allclose(got0, case["softmax_out"], rtol=0, atol=1e-12,
                                   err_msg=case["name"] + " (softmax)")


def pin_golden_gqa():
    """Hand-derived GQA case: consecutive query heads share a KV head."""
    g = json.load(open(GOLDEN))["gqa"]
    K = np.array(g["K"])[None]           # [1, Hkv, n, d]
    V = np.array(g["V"])[None]
    q = np.array(g["q"])[None]           # [1, Hq, d]
    rho = np.array(g["rho"])[None]
    out = oracle.decode(q, rho, K, V, [K.shape[2]], Hkv=g["Hkv"])
    np.testing.assert_allclose(out[0], g["out"], rtol=0, atol=1e-12)


def pin_golden_probe():
    p = json.load(open(GOLDEN))["probe"]
    rho = oracle.probe(np.array(p["W_R"]), np.array(p["x"]), p["Hq"], p["d"])
    np.testing.assert_allclose(rho, p["rho"], rtol=0, atol=0)


def pin_probe_bruteforce():
    """Probe against explicit scalar loops on a small shape."""
    r = _rng(11)
    B, Hq, d, dm = 3, 3, 4, 5
    W = r.standard_normal((Hq * d, dm))
    x = r.standard_normal((B, dm))
    got = oracle.probe(W, x, Hq, d)
    for b in range(B):
        for h in range(Hq):
            for i in range(d):
                acc = 0.0
                for c in range(dm):
                    acc += W[h * d + i][c] * x[b][c]
                assert abs(got[b, h, i] - acc) < 1e-12


def _sdpa(q, K, V):
    """torch's scaled_dot_product_attention in float64 for one (b, head)."""
    qt = torch.from_numpy(q)[None, None, None, :]
    kt = torch.from_numpy(K)[None, None]
    vt = torch.from_numpy(V)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0, 0].numpy()


def pin_wr_zero_is_softmax():
    """P1: W_R = 0 => rho = 0 => plain softmax attention (encorp.ai (de), section
    'Parallax behält Softmax bei'; zubnet.ai second paragraph), checked against
    torch SDPA in fp64 with KV heads repeated for GQA."""
    r = _rng(1)
    B, Hq, Hkv, d, dm = 2, 4, 2, 8, 6
    lens = [5, 9]
    x = r.standard_normal((B, dm))
    W = np.zeros((Hq * d, dm))
    rho = oracle.probe(W, x, Hq, d)
    assert np.all(rho == 0)
    q = r.standard_normal((B, Hq, d))
    K = [r.standard_normal((Hkv, n, d)) * 1.5 for n in lens]
    V = [r.standard_normal((Hkv, n, d)) for n in lens]
    out = oracle.decode(q, rho, K, V, lens, Hkv)
    G = Hq // Hkv
    for b in range(B):
        Kr = np.repeat(K[b], G, axis=0)      # repeat_interleave over heads
        Vr = np.repeat(V[b], G, axis=0)
        for h in range(Hq):
            ref = _sdpa(q[b, h], Kr[h], Vr[h])
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-13)


def pin_single_pass_identity():
    """P2: C rho = sum_j w_j p_j v_j - vbar * sum_j w_j p_j with p_j = k_j . rho
    (the streaming form both branches use on one KV pass), computed here from
    unnormalised running sums with an online max, as a kernel would."""
    r = _rng(2)
    for d, n in ((4, 7), (16, 33), (64, 200)):
        q = r.standard_normal(d)
        rho = r.standard_normal(d) * 0.3
        K = r.standard_normal((n, d)) * 2.0
        V = r.standard_normal((n, d))
        m, l, S = -math.inf, 0.0, 0.0
        A = np.zeros(d)
        P = np.zeros(d)
        for j in range(n):
            s = float(K[j] @ q) / math.sqrt(d)
            p = float(K[j] @ rho)
            m_new = max(m, s)
            a = 0.0 if m == -math.inf else math.exp(m - m_new)
            e = math.exp(s - m_new)
            l, S = l * a + e, S * a + e * p
            A, P = A * a + e * V[j], P * a + (e * p) * V[j]
            m = m_new
        vbar = A / l
        stream = vbar - (P / l - vbar * (S / l))
        np.testing.assert_allclose(oracle.decode_head(q, rho, K, V), stream,
                                   rtol=0, atol=1e-12)


def pin_local_linear_lstsq():
    """P3: with rho* = Sigma_kk^{-1} (kbar - q), out equals the intercept of the
    softmax-weighted least-squares fit v_j ~ a + B (k_j - q). This is the
    local-linear estimate at the query that exact local linear attention gets
    from a per-query linear solve (encorp.ai (de), section on the conjugate
    gradient solver; zubnet.ai, first paragraph). Weights, means and Sigma_kk are
    computed here independently of the oracle."""
    r = _rng(3)
    for d, n in ((2, 8), (3, 12), (5, 40)):
        q = r.standard_normal(d)
        K = r.standard_normal((n, d))
        V = r.standard_normal((n, d))
        s = K @ q / math.sqrt(d)
        w = np.exp(s - s.max())
        w /= w.sum()
        kbar = w @ K
        Skk = ((K - kbar) * w[:, None]).T @ (K - kbar)
        rho_star = np.linalg.solve(Skk, kbar - q)
        X = np.hstack([np.ones((n, 1)), K - q])
        sw = np.sqrt(w)[:, None]
        coef, *_ = np.linalg.lstsq(X * sw, V * sw, rcond=None)
        intercept = coef[0]
        np.testing.assert_allclose(oracle.decode_head(q, rho_star, K, V), intercept,
                                   rtol=0, atol=1e-10)


def pin_closed_forms():
    """P4/P5: n = 1 => v_0; identical keys => mean of values; identical values => v."""
    r = _rng(4)
    d = 6
    q, rho = r.standard_normal(d), r.standard_normal(d) * 5
    K1, V1 = r.standard_normal((1, d)), r.standard_normal((1, d))
    np.testing.assert_allclose(oracle.decode_head(q, rho, K1, V1), V1[0], atol=1e-14, rtol=0)
    k = r.standard_normal(d)
    Keq = np.tile(k, (9, 1))
    V = r.standard_normal((9, d))
    np.testing.assert_allclose(oracle.decode_head(q, rho, Keq, V), V.mean(0), atol=1e-13, rtol=0)
    K = r.standard_normal((9, d))
    v = r.standard_normal(d)
    np.testing.assert_allclose(oracle.decode_head(q, rho, K, np.tile(v, (9, 1))), v,
                               atol=1e-13, rtol=0)
    np.testing.assert_array_equal(oracle.decode_head(q, rho, K[:0], V[:0]), np.zeros(d))


def pin_invariances():
    """P6/P7/P8: key shift leaves out unchanged; value shift moves it by the same
    vector; out - vbar is linear in rho; permuting keys (with their values)
    leaves out unchanged."""
    r = _rng(5)
    d, n = 8, 23
    q, rho1, rho2 = r.standard_normal(d), r.standard_normal(d), r.standard_normal(d)
    K, V = r.standard_normal((n, d)), r.standard_normal((n, d))
    base = oracle.decode_head(q, rho1, K, V)
    c = r.standard_normal(d)
    np.testing.assert_allclose(oracle.decode_head(q, rho1, K + c, V), base, atol=1e-12, rtol=0)
    np.testing.assert_allclose(oracle.decode_head(q, rho1, K, V + c), base + c, atol=1e-12, rtol=0)
    v0 = oracle.decode_head(q, np.zeros(d), K, V)
    a, b = 0.7, -2.5
    lhs = oracle.decode_head(q, a * rho1 + b * rho2, K, V) - v0
    rhs = a * (oracle.decode_head(q, rho1, K, V) - v0) + b * (oracle.decode_head(q, rho2, K, V) - v0)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12, rtol=0)
    perm = r.permutation(n)
    np.testing.assert_allclose(oracle.decode_head(q, rho1, K[perm], V[perm]), base,
                               atol=1e-12, rtol=0)


def _brute_head(q, rho, K, V):
    """Pure-Python scalar loops: weights, means, covariance entries, output."""
    n, d = len(K), len(q)
    s = [sum(q[i] * K[j][i] for i in range(d)) / math.sqrt(d) for j in range(n)]
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    tot = sum(e)
    w = [x / tot for x in e]
    kb = [sum(w[j] * K[j][i] for j in range(n)) for i in range(d)]
    vb = [sum(w[j] * V[j][i] for j in range(n)) for i in range(d)]
    out = []
    for a in range(d):
        corr = 0.0
        for c in range(d):
            cov = sum(w[j] * (V[j][a] - vb[a]) * (K[j][c] - kb[c]) for j in range(n))
            corr += cov * rho[c]
        out.append(vb[a] - corr)
    return out


def pin_bruteforce():
    """P9: the NumPy oracle equals pure-Python scalar loops on tiny shapes (with
    GQA groups G in {1, 2})."""
    r = _rng(6)
    for (Hq, Hkv, d, lens) in ((2, 2, 3, [1, 4]), (4, 2, 4, [8, 3]), (2, 1, 2, [6, 5])):
        B = len(lens)
        q = r.standard_normal((B, Hq, d))
        rho = r.standard_normal((B, Hq, d))
        K = [r.standard_normal((Hkv, n, d)) * 2 for n in lens]
        V = [r.standard_normal((Hkv, n, d)) for n in lens]
        out = oracle.decode(q, rho, K, V, lens, Hkv)
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                g = h // G
                ref = _brute_head(q[b, h].tolist(), rho[b, h].tolist(),
                                  K[b][g].tolist(), V[b][g].tolist())
                np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)


def pin_gqa_equals_mha():
    """P10: GQA equals MHA with each KV head repeated G times (repeat_interleave)."""
    r = _rng(7)
    B, Hq, Hkv, d = 2, 6, 2, 5
    lens = [7, 11]
    q = r.standard_normal((B, Hq, d))
    rho = r.standard_normal((B, Hq, d))
    K = [r.standard_normal((Hkv, n, d)) for n in lens]
    V = [r.standard_normal((Hkv, n, d)) for n in lens]
    G = Hq // Hkv
    Kr = [np.repeat(k, G, axis=0) for k in K]
    Vr = [np.repeat(v, G, axis=0) for v in V]
    np.testing.assert_allclose(oracle.decode(q, rho, K, V, lens, Hkv),
                               oracle.decode(q, rho, Kr, Vr, lens, Hq), atol=0, rtol=0)


def _ragged_gqa_case(seed, pad=np.nan):
    """A ragged GQA batch (Hq 6, Hkv 2, lengths 9, 0, 1, 13 in a 16-row cache)
    in both layouts the oracle accepts: per-sequence [Hkv, n_b, d] arrays and a
    padded [B, Hkv, 16, d] cache whose rows past each length hold `pad`."""
    r = _rng(seed)
    B, Hq, Hkv, d, cap = 4, 6, 2, 5, 16
    lens = [9, 0, 1, 13]
    q = r.standard_normal((B, Hq, d))
    rho = r.standard_normal((B, Hq, d))
    K = [r.standard_normal((Hkv, n, d)) * 2 for n in lens]
    V = [r.standard_normal((Hkv, n, d)) for n in lens]
    Kp = np.full((B, Hkv, cap, d), pad)
    Vp = np.full((B, Hkv, cap, d), pad)
    for b, n in enumerate(lens):
        Kp[b, :, :n], Vp[b, :, :n] = K[b], V[b]
    return q, rho, K, V, Kp, Vp, lens, Hkv


def pin_decode_heads_equals_decode():
    """decode_heads (the checker of sampled output rows) returns, for every
    listed (b, h) pair in any order and with repeats, exactly row (b, h) of
    decode(): on a ragged GQA batch with an empty and a one-key sequence, from
    per-sequence arrays and from a NaN-padded cache (a read past a length would
    give NaN)."""
    q, rho, K, V, Kp, Vp, lens, Hkv = _ragged_gqa_case(12)
    B, Hq = q.shape[:2]
    pairs = [(b, h) for b in range(B) for h in range(Hq)]
    order = _rng(13).permutation(len(pairs))
    pairs = [pairs[i] for i in order] + [(3, 5), (0, 1), (3, 5)]
    for Kc, Vc in ((K, V), (Kp, Vp)):
        full = oracle.decode(q, rho, Kc, Vc, lens, Hkv)
        got = oracle.decode_heads(q, rho, Kc, Vc, lens, Hkv, pairs)
        assert np.isfinite(got).all()
        np.testing.assert_array_equal(got, np.stack([full[b, h] for b, h in pairs]))
    assert oracle.decode_heads(q, rho, K, V, lens, Hkv, []).shape == (0, q.shape[2])


def pin_length_clamp():
    """A length above the cache's rows counts as all of them and a negative one
    as 0 (zero output), for decode and decode_heads alike; checked against
    decode_head on explicitly sliced rows."""
    q, rho, K, V, Kp, Vp, lens, Hkv = _ragged_gqa_case(14, pad=0.5)
    Kp[2, :, :], Vp[2, :, :] = Kp[3, :, :], Vp[3, :, :]   # sequence 2: all 16 rows valid
    lens2 = [-3, 0, 100, 13]
    Hq = q.shape[1]
    G = Hq // Hkv
    full = oracle.decode(q, rho, Kp, Vp, lens2, Hkv)
    rows = oracle.decode_heads(q, rho, Kp, Vp, lens2, Hkv, [(0, 4), (2, 5)])
    assert np.all(full[0] == 0.0) and np.all(full[1] == 0.0) and np.all(rows[0] == 0.0)
    for h in range(Hq):
        ref = oracle.decode_head(q[2, h], rho[2, h], Kp[2, h // G, :16], Vp[2, h // G, :16])
        np.testing.assert_allclose(full[2, h], ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(rows[1], full[2, 5], rtol=0, atol=0)


ALL_PINS = [pin_golden_decode, pin_golden_gqa, pin_golden_probe, pin_probe_bruteforce,
            pin_wr_zero_is_softmax, pin_single_pass_identity, pin_local_linear_lstsq,
            pin_closed_forms, pin_invariances, pin_bruteforce, pin_gqa_equals_mha,
            pin_decode_heads_equals_decode, pin_length_clamp]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_torch_tensor_inputs_match_numpy():
    """The oracle upcasts bf16 torch tensors exactly."""
    t = torch.randn(3, 4, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    a = po._f64(t)
    assert a.dtype == np.float64
    np.testing.assert_array_equal(a, t.float().numpy().astype(np.float64))


# ---------------------------------------------------------------- planted mistakes
def _mut_transposed_cov(w, K, V, kbar, vbar):
    return ((V - vbar) * w[:, None]).T.dot(K - kbar).T


def _mut_bessel(w, K, V, kbar, vbar):
    n = len(w)
    C = ((V - vbar) * w[:, None]).T @ (K - kbar)
    return C * (n / (n - 1)) if n > 1 else C


def _mut_raw_second_moment(w, K, V, kbar, vbar):
    return (V * w[:, None]).T @ K


def _mut_unweighted_means(w, K, V, kbar, vbar):
    return ((V - V.mean(0)) * w[:, None]).T @ (K - K.mean(0))


def _mut_no_scale(q, K):
    s = K @ q
    e = np.exp(s - s.max())
    return e / e.sum()


def _mut_unnormalised(q, K):
    s = (K @ q) / np.sqrt(q.shape[0])
    return np.exp(s - s.max())


def _mut_plus_sign(q, rho, K, V):
    q, rho, K, V = (po._f64(a) for a in (q, rho, K, V))
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    w = po.softmax_weights(q, K)
    kbar, vbar = po.weighted_means(w, K, V)
    return vbar + po.kv_covariance(w, K, V, kbar, vbar) @ rho


def _mut_head_map(h, Hq, Hkv):
    return h % Hkv


def _mut_probe_layout(W_R, x, Hq, d):
    W, X = po._f64(W_R), po._f64(x)
    return (X @ W.T).reshape(X.shape[0], d, Hq).transpose(0, 2, 1)


def _mut_heads_pair_length(q, rho, K_parts, V_parts, seq_lens, Hkv, pairs):
    """decode_heads taking the length of the i-th sequence for the i-th pair."""
    Hq = q.shape[1]
    res = []
    for i, (b, h) in enumerate(pairs):
        n = int(seq_lens[i % len(seq_lens)])
        Kb, Vb = po._seq_kv(K_parts, V_parts, b, po.kv_head_of(h, Hq, Hkv), n)
        res.append(po.decode_head(q[b, h], rho[b, h], Kb, Vb))
    return np.stack(res) if res else np.zeros((0, q.shape[2]))


def _mut_heads_no_kv_map(q, rho, K_parts, V_parts, seq_lens, Hkv, pairs):
    """decode_heads reading KV head h instead of kv_head_of(h)."""
    res = []
    for b, h in pairs:
        Kb, Vb = po._seq_kv(K_parts, V_parts, b, h % Hkv, int(seq_lens[b]))
        res.append(po.decode_head(q[b, h], rho[b, h], Kb, Vb))
    return np.stack(res) if res else np.zeros((0, q.shape[2]))


def _mut_unclamped_rows(K_parts, V_parts, b, g, n):
    return K_parts[b][g][:n], V_parts[b][g][:n]


MUTANTS = {
    "heads_length_of_pair_index": ("decode_heads", _mut_heads_pair_length),
    "heads_without_kv_head_map": ("decode_heads", _mut_heads_no_kv_map),
    "unclamped_length": ("_seq_kv", _mut_unclamped_rows),
    "transposed_covariance": ("kv_covariance", _mut_transposed_cov),
    "bessel_factor": ("kv_covariance", _mut_bessel),
    "raw_second_moment": ("kv_covariance", _mut_raw_second_moment),
    "unweighted_means": ("kv_covariance", _mut_unweighted_means),
    "missing_score_scale": ("softmax_weights", _mut_no_scale),
    "unnormalised_weights": ("softmax_weights", _mut_unnormalised),
    "plus_sign": ("decode_head", _mut_plus_sign),
    "interleaved_head_map": ("kv_head_of", _mut_head_map),
    "probe_layout": ("probe", _mut_probe_layout),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name, monkeypatch):
    """Each planted mistake in the oracle makes at least one pin fail."""
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(po, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, np.linalg.LinAlgError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
