"""Seeded synthetic inputs for Parallax decode attention.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the fp64 oracle (via the tests and the bench's CPU
baseline) and the HIP path take their inputs from here, so the two sides see
bit-identical values.

Recipe (one ``torch.Generator('cpu')`` per input set, seeded explicitly):

1. ``x``    [B, d_model]        ~ N(0, 1)
2. ``W_R``  [Hq*d, d_model]     ~ N(0, wr_std^2)
3. ``q``    [B, Hq, d]          ~ N(0, 1)
4. lengths (ragged workloads only): n_b = round(exp(U[ln lo, ln hi])), clamped
   to [lo, hi]; fixed-length workloads use n_b = ctx for every b.
5. for b in 0..B-1: ``K_b`` [Hkv, n_b, d] ~ k_scale * N(0, 1), then
   ``V_b`` [Hkv, n_b, d] ~ N(0, 1).

All draws are fp32 normals, scaled, then cast with round-to-nearest-even to the
workload's storage dtype (bf16 or fp32). Only the valid rows (j < n_b) of the
cache are drawn; the padded device cache is filled separately (NaN for parity
runs, so that any read past n_b shows up).

The workloads follow the pages' decode setting: a KV cache per sequence, one
query token, batch 1 to 2048 and context 128 to 32768 (zubnet.ai, "Parallax
mantém softmax ...", second paragraph). No public dataset is involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import List, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "InputSet", "make_inputs", "padded_cache", "device_cache",
           "algorithmic_bytes", "sweep_points"]


@dataclass(frozen=True)
class Workload:
    """Shape and value distribution of one decode workload."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    ctx: int                 # fixed length, or the upper bound of ragged lengths
    d_model: int
    dtype: str               # "f32" or "bf16": storage type of x, W_R, q, K, V, out
    wr_std: float            # W_R ~ N(0, wr_std^2)
    k_scale: float = 1.0     # keys ~ k_scale * N(0, 1)
    ragged_lo: int = 0       # >0: lengths log-uniform in [ragged_lo, ctx]
    max_ctx: int = 0         # cache capacity (0: equal to ctx)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def capacity(self) -> int:
        return self.max_ctx if self.max_ctx > 0 else self.ctx

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads (tiny fp32, mid-context GQA, long-context, large batch,
# ragged batch).
WORKLOADS = {
    1: Workload("tiny_fp32_B1_H2_d64_ctx128", B=1, Hq=2, Hkv=2, d=64, ctx=128,
                d_model=128, dtype="f32", wr_std=math.sqrt(1.0 / 128)),
    2: Workload("gqa_B16_Hq16_Hkv8_d128_ctx4096", B=16, Hq=16, Hkv=8, d=128,
                ctx=4096, d_model=2048, dtype="bf16", wr_std=0.02),
    3: Workload("long_B1_Hq16_Hkv8_d128_ctx32768", B=1, Hq=16, Hkv=8, d=128,
                ctx=32768, d_model=2048, dtype="bf16", wr_std=0.02),
    4: Workload("batch_B2048_Hq16_Hkv8_d128_ctx128", B=2048, Hq=16, Hkv=8, d=128,
                ctx=128, d_model=2048, dtype="bf16", wr_std=0.02),
    5: Workload("ragged_B64_Hq32_Hkv8_d128_ctx128to32768", B=64, Hq=32, Hkv=8,
                d=128, ctx=32768, d_model=2560, dtype="bf16", wr_std=0.02,
                k_scale=2.0, ragged_lo=128),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclass
class InputSet:
    """Host (CPU) tensors of one seeded input set, in storage dtype."""
    wl: Workload
    seed: int
    x: torch.Tensor            # [B, d_model]
    W_R: torch.Tensor          # [Hq*d, d_model]
    q: torch.Tensor            # [B, Hq, d]
    seq_lens: torch.Tensor     # [B] int32
    K: List[torch.Tensor]      # per sequence [Hkv, n_b, d]
    V: List[torch.Tensor]      # per sequence [Hkv, n_b, d]

    @property
    def max_ctx(self) -> int:
        return self.wl.capacity

    def total_tokens(self) -> int:
        return int(self.seq_lens.to(torch.int64).sum())


def _normal(g: torch.Generator, shape, std: float, dt: torch.dtype) -> torch.Tensor:
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dt)          # round-to-nearest-even for bf16


def draw_lengths(g: torch.Generator, B: int, lo: int, hi: int) -> torch.Tensor:
    u = torch.rand(B, generator=g, dtype=torch.float64)
    ln = math.log(lo) + u * (math.log(hi) - math.log(lo))
    n = torch.round(torch.exp(ln)).clamp_(lo, hi)
    return n.to(torch.int32)


def make_inputs(wl: Workload, seed: int = 0, *, wr_zero: bool = False,
                lengths: Optional[List[int]] = None, with_kv: bool = True) -> InputSet:
    """Draw one input set in the fixed order documented in the module header.

    ``wr_zero`` replaces W_R by zeros after drawing it (so the rest of the
    stream is unchanged). ``lengths`` overrides the per-sequence lengths (the
    lengths draw is then skipped); each must lie in [0, capacity].
    ``with_kv=False`` stops after the lengths (K and V are left empty): x, W_R,
    q and the lengths are those of the full draw, for callers that fill the
    cache themselves (the benchmark draws K/V on the device).
    """
    dt = torch_dtype(wl.dtype)
    g = torch.Generator("cpu").manual_seed(seed)
    x = _normal(g, (wl.B, wl.d_model), 1.0, dt)
    W_R = _normal(g, (wl.Hq * wl.d, wl.d_model), wl.wr_std, dt)
    if wr_zero:
        W_R = torch.zeros_like(W_R)
    q = _normal(g, (wl.B, wl.Hq, wl.d), 1.0, dt)
    if lengths is not None:
        if len(lengths) != wl.B:
            raise ValueError("lengths must have B entries")
        seq = torch.tensor(lengths, dtype=torch.int32)
        if int(seq.min()) < 0 or int(seq.max()) > wl.capacity:
            raise ValueError("lengths must lie in [0, capacity]")
    elif wl.ragged_lo > 0:
        seq = draw_lengths(g, wl.B, wl.ragged_lo, wl.ctx)
    else:
        seq = torch.full((wl.B,), wl.ctx, dtype=torch.int32)
    K, V = [], []
    for b in range(wl.B if with_kv else 0):
        n = int(seq[b])
        K.append(_normal(g, (wl.Hkv, n, wl.d), wl.k_scale, dt))
        V.append(_normal(g, (wl.Hkv, n, wl.d), 1.0, dt))
    return InputSet(wl, seed, x, W_R, q, seq, K, V)


def device_cache(wl: Workload, seed: int, device="cuda"):
    """K and V caches [B, Hkv, capacity, d] drawn directly in device memory
    (normals from a device generator, keys scaled by k_scale, rounded to the
    storage dtype): the same distribution as make_inputs, other values, every
    row filled (rows past a sequence's length are never read). For timing
    runs, where drawing gigabytes on the host would dominate."""
    dt = torch_dtype(wl.dtype)
    g = torch.Generator(device=device).manual_seed(seed)
    shape = (wl.B, wl.Hkv, wl.capacity, wl.d)
    K = torch.randn(shape, generator=g, device=device, dtype=dt)
    if wl.k_scale != 1.0:
        K.mul_(wl.k_scale)
    V = torch.randn(shape, generator=g, device=device, dtype=dt)
    return K, V


@dataclass
class PrefillSet:
    """Inputs of a causal many-query forward: T new tokens per sequence after
    prefix[b] cached ones (K/V hold prefix[b] + T rows per sequence)."""
    wl: Workload
    seed: int
    T: int
    prefix: torch.Tensor          # [B] int32
    x: torch.Tensor               # [B, T, d_model]
    W_R: torch.Tensor             # [Hq*d, d_model]
    q: torch.Tensor               # [B, T, Hq, d]
    K: List[torch.Tensor]         # per sequence [Hkv, prefix[b] + T, d]
    V: List[torch.Tensor]

    @property
    def max_ctx(self) -> int:
        return int(self.prefix.max()) + self.T


def make_prefill_inputs(wl: Workload, T: int, prefix: List[int], seed: int = 0) -> PrefillSet:
    """Draw a prefill input set: x [B, T, d_model], W_R, q [B, T, Hq, d], then
    per sequence K and V of prefix[b] + T rows, with the distributions of
    make_inputs (bf16 rounding of scaled fp32 normals)."""
    if len(prefix) != wl.B or min(prefix) < 0:
        raise ValueError("prefix must have B non-negative entries")
    dt = torch_dtype(wl.dtype)
    g = torch.Generator("cpu").manual_seed(seed)
    x = _normal(g, (wl.B, T, wl.d_model), 1.0, dt)
    W_R = _normal(g, (wl.Hq * wl.d, wl.d_model), wl.wr_std, dt)
    q = _normal(g, (wl.B, T, wl.Hq, wl.d), 1.0, dt)
    K, V = [], []
    for b in range(wl.B):
        n = prefix[b] + T
        K.append(_normal(g, (wl.Hkv, n, wl.d), wl.k_scale, dt))
        V.append(_normal(g, (wl.Hkv, n, wl.d), 1.0, dt))
    return PrefillSet(wl, seed, T, torch.tensor(prefix, dtype=torch.int32), x, W_R, q, K, V)


def padded_cache(parts: List[torch.Tensor], max_ctx: int, pad: float = float("nan"),
                 device="cpu") -> torch.Tensor:
    """Lay per-sequence [Hkv, n_b, d] tensors into a [B, Hkv, max_ctx, d] cache.

    Rows j >= n_b hold ``pad`` (NaN by default). The copy goes sequence by
    sequence so a large cache can be built directly in device memory.
    """
    B = len(parts)
    Hkv, _, d = parts[0].shape
    cache = torch.full((B, Hkv, max_ctx, d), pad, dtype=parts[0].dtype, device=device)
    for b, p in enumerate(parts):
        n = p.shape[1]
        if n:
            cache[b, :, :n, :].copy_(p, non_blocking=False)
    return cache


def algorithmic_bytes(wl: Workload, total_tokens: int) -> dict:
    """Bytes the decode step must move: valid K/V rows, q, rho (fp32), out, seq_lens."""
    es = 2 if wl.dtype == "bf16" else 4
    kv = 2 * total_tokens * wl.Hkv * wl.d * es
    q = wl.B * wl.Hq * wl.d * es
    rho = wl.B * wl.Hq * wl.d * 4
    out = wl.B * wl.Hq * wl.d * es
    lens = wl.B * 4
    return {"kv": kv, "q": q, "rho": rho, "out": out, "seq_lens": lens,
            "decode_read": kv + q + rho + lens, "total": kv + q + rho + out + lens}


def sweep_points(max_kv_bytes: int = 64 << 30):
    """Batch x context grid (powers of two, B 1..2048, ctx 128..32768) at
    Hq=16, Hkv=8, d=128, bf16; points whose K+V exceed ``max_kv_bytes`` skipped."""
    pts = []
    B = 1
    while B <= 2048:
        c = 128
        while c <= 32768:
            kv = 2 * B * c * 8 * 128 * 2
            if kv <= max_kv_bytes:
                pts.append((B, c))
            c *= 2
        B *= 2
    return pts
