"""fp64 CPU oracle for Parallax decode attention — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this module. The product path (the HIP library and its Python binding) never
calls it, and it shares no code with that path: it imports NumPy and nothing
else.

What it computes, in the order the pages state the method:

* The layer-input probe: a learned projection W_R maps the layer input x_i to a
  probe rho_i = W_R x_i that lives in key space (zubnet.ai (pt), "Parallax
  mantém softmax ...", second paragraph; the French version, "Parallax garde
  softmax ...", second paragraph; encorp.ai (de), section "Warum das Entfernen
  des konjugierten Gradienten-Solvers ...": W_R acts on the layer input).
* The output is softmax attention minus a projected covariance term: the KV
  covariance multiplied by the probe (same two paragraphs). Softmax attention is
  the local-constant estimate and the correction makes it local-linear (same
  pages, first paragraph), so the covariance is the one under the softmax
  weights of that query: weights normalised to sum to one, centred on the
  softmax-weighted means, no n/(n-1) factor.
* W_R = 0 recovers plain softmax attention exactly (encorp.ai (de), section
  "Parallax behält Softmax bei ..."; zubnet.ai, second paragraph).

Readings where the pages are silent (each pinned by a test, see tests/):
scores are q.k/sqrt(d); the covariance is C = sum_j w_j (v_j - vbar)(k_j - kbar)^T
(value rows, key columns) so that C rho contracts rho with keys; rho is per
query head; query head h reads KV head floor(h / (Hq/Hkv)); a sequence of
length 0 gives an all-zero output; a length outside [0, rows in the cache] is
clamped into it (the decode library's documented treatment of a caller
error), so a negative length also gives zeros.

Everything is float64; inputs are the exact values the GPU receives (bf16 or
fp32), upcast without rounding.
"""
from __future__ import annotations

import numpy as np

__all__ = ["probe", "softmax_weights", "weighted_means", "kv_covariance",
           "decode_head", "decode", "decode_heads", "kv_head_of", "clamp_len", "prefill",
           "prefill_rows"]


def _f64(a) -> np.ndarray:
    """Upcast to a float64 ndarray (accepts NumPy arrays or CPU torch tensors)."""
    if hasattr(a, "detach"):              # torch tensor, without importing torch
        a = a.detach().to("cpu")
        if str(a.dtype) in ("torch.bfloat16", "torch.float16"):
            a = a.float()
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def probe(W_R, x, Hq: int, d: int) -> np.ndarray:
    """rho[b, h, :] = W_R[h*d:(h+1)*d, :] @ x[b]  ->  [B, Hq, d] float64.

    The probe is a plain matrix-vector product of the learned projection with
    the layer input (zubnet.ai (pt), second paragraph: rho_i = W_R x_i).
    Row h*d + i of W_R produces component i of query head h's probe.
    """
    W = _f64(W_R)
    X = _f64(x)
    if W.shape[0] != Hq * d or W.shape[1] != X.shape[1]:
        raise ValueError("W_R must be [Hq*d, d_model] and x [B, d_model]")
    rho = X @ W.T                          # [B, Hq*d]
    return rho.reshape(X.shape[0], Hq, d)


def softmax_weights(q: np.ndarray, K: np.ndarray) -> np.ndarray:
    """Normalised softmax weights w_j = exp(s_j - max s) / sum_k exp(s_k - max s),
    with scores s_j = q . k_j / sqrt(d). K is [n, d], n >= 1."""
    d = q.shape[0]
    s = (K @ q) / np.sqrt(d)
    e = np.exp(s - s.max())
    return e / e.sum()


def weighted_means(w: np.ndarray, K: np.ndarray, V: np.ndarray):
    """kbar = sum_j w_j k_j and vbar = sum_j w_j v_j (vbar is the softmax output)."""
    return w @ K, w @ V


def kv_covariance(w: np.ndarray, K: np.ndarray, V: np.ndarray,
                  kbar: np.ndarray, vbar: np.ndarray) -> np.ndarray:
    """Softmax-weighted KV covariance, explicit and two-pass:
    C = sum_j w_j (v_j - vbar)(k_j - kbar)^T, a [d_v, d_k] matrix."""
    Vc = V - vbar                           # [n, d]
    Kc = K - kbar                           # [n, d]
    return (Vc * w[:, None]).T @ Kc


def decode_head(q, rho, K, V) -> np.ndarray:
    """One query head against n cached keys/values: out = vbar - C rho.

    q, rho: [d]; K, V: [n, d]. n == 0 gives zeros (a convention: the pages do
    not define attention over an empty cache).
    """
    q = _f64(q)
    rho = _f64(rho)
    K = _f64(K)
    V = _f64(V)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    w = softmax_weights(q, K)
    kbar, vbar = weighted_means(w, K, V)
    C = kv_covariance(w, K, V, kbar, vbar)
    return vbar - C @ rho


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Query head h reads KV head floor(h / G), G = Hq / Hkv (consecutive query
    heads share a KV head)."""
    return h // (Hq // Hkv)


def clamp_len(n: int, rows: int) -> int:
    """A sequence length as the decode uses it: lengths above the rows the cache
    holds (max_ctx for a padded cache) count as all of them, and a negative
    length counts as 0, i.e. an empty cache and a zero output (the n = 0
    convention of decode_head)."""
    return max(0, min(int(n), int(rows)))


def _seq_kv(K_parts, V_parts, b, g, n):
    """K, V rows 0..n-1 of KV head g of sequence b, from either per-sequence
    [Hkv, n_b, d] lists or a padded [B, Hkv, max_ctx, d] cache; n is clamped
    to the rows present (clamp_len)."""
    Kg, Vg = K_parts[b][g], V_parts[b][g]
    n = clamp_len(n, Kg.shape[0])
    return Kg[:n], Vg[:n]


def decode(q, rho, K_parts, V_parts, seq_lens, Hkv: int) -> np.ndarray:
    """Full decode: out[b, h] = decode_head(q[b,h], rho[b,h], K[b, g(h), :n_b], V[...]).

    q, rho: [B, Hq, d]; K_parts/V_parts: per-sequence [Hkv, n_b, d] (or a padded
    cache [B, Hkv, max_ctx, d]); seq_lens: [B].
    """
    qa = _f64(q)
    ra = _f64(rho)
    B, Hq, d = qa.shape
    lens = [int(n) for n in _f64(seq_lens)]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            Kb, Vb = _seq_kv(K_parts, V_parts, b, g, lens[b])
            out[b, h] = decode_head(qa[b, h], ra[b, h], Kb, Vb)
    return out


def decode_heads(q, rho, K_parts, V_parts, seq_lens, Hkv: int, pairs) -> np.ndarray:
    """decode() restricted to the listed (b, h) pairs -> [len(pairs), d]: pair
    (b, h) reads the length of sequence b and KV head kv_head_of(h), exactly
    as decode() does for that output row."""
    Hq = q.shape[1]
    lens = [int(n) for n in _f64(seq_lens)]
    res = []
    for b, h in pairs:
        g = kv_head_of(h, Hq, Hkv)
        Kb, Vb = _seq_kv(K_parts, V_parts, b, g, lens[b])
        res.append(decode_head(q[b, h], rho[b, h], Kb, Vb))
    if not res:
        return np.zeros((0, q.shape[2]))
    return np.stack(res)


def prefill(q, rho, K_parts, V_parts, prefix_lens, Hkv: int) -> np.ndarray:
    """Causal many-query forward (prefill) -> [B, T, Hq, d].

    Token t of sequence b sits at position prefix_lens[b] + t of its cache and
    attends to cache rows 0 .. prefix_lens[b] + t (itself and everything
    before it); each (token, head) output is the Parallax output of that query
    over that prefix: decode_head with the token's own query and probe. The
    layer is pretrained as the attention of a language model at a 4096-token
    context (encorp.ai (de), section "Die Pretraining-Gewinne sind real ...");
    the causal prefix is the reading taken for that forward pass (the pages do
    not spell the mask out), and decode is its one-token case.
    q, rho: [B, T, Hq, d]; K_parts/V_parts: per-sequence [Hkv, n_b, d] arrays
    holding at least prefix_lens[b] + T rows (or a padded cache).
    """
    qa = _f64(q)
    ra = _f64(rho)
    B, T, Hq, d = qa.shape
    pre = [int(p) for p in _f64(prefix_lens)]
    out = np.zeros((B, T, Hq, d))
    for b in range(B):
        for t in range(T):
            n = pre[b] + t + 1
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                Kb, Vb = _seq_kv(K_parts, V_parts, b, g, n)
                out[b, t, h] = decode_head(qa[b, t, h], ra[b, t, h], Kb, Vb)
    return out


def prefill_rows(q, rho, K_parts, V_parts, prefix_lens, Hkv: int, rows) -> np.ndarray:
    """prefill() restricted to the listed (b, t, h) rows -> [len(rows), d]."""
    qa = _f64(q)
    ra = _f64(rho)
    Hq = qa.shape[2]
    res = []
    for b, t, h in rows:
        n = int(prefix_lens[b]) + t + 1
        Kb, Vb = _seq_kv(K_parts, V_parts, b, kv_head_of(h, Hq, Hkv), n)
        res.append(decode_head(qa[b, t, h], ra[b, t, h], Kb, Vb))
    return np.stack(res)
