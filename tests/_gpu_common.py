"""Shared helpers of the GPU parity tests: upload a seeded input set, run the
HIP path through the C ABI, run the oracle on the same values, compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
from parallax_covariance_corrected_amd import binding as pb
from parallax_covariance_corrected_amd.workloads import InputSet, padded_cache

# Tolerances of the decode output against the fp64 oracle.
BF16_REL_L2 = 2e-3        # bf16 output
F32OUT_MAX_ABS = 1e-2     # bf16 inputs, fp32 output (the kernel's value before the bf16 cast)
F32_TOL = 1e-5            # fp32 path: rel-L2 and max-abs
RHO_REL_L2 = 1e-5         # probe (fp32 result) against the fp64 oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (nb if nb > 0 else 1.0)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0


class Device:
    """Device copies of one input set (K/V padded with NaN past each length)."""

    def __init__(self, s: InputSet, pad: float = float("nan")):
        dev = "cuda"
        self.s = s
        self.x = s.x.to(dev)
        self.W_R = s.W_R.to(dev)
        self.q = s.q.to(dev)
        self.seq_lens = s.seq_lens.to(dev)
        self.K = padded_cache(s.K, s.max_ctx, pad, device=dev)
        self.V = padded_cache(s.V, s.max_ctx, pad, device=dev)

    def probe(self) -> torch.Tensor:
        wl = self.s.wl
        return pb.probe(self.W_R, self.x, wl.Hq, wl.d)

    def decode(self, rho, out_dtype=None) -> torch.Tensor:
        return pb.decode(self.q, rho, self.K, self.V, self.seq_lens, out_dtype=out_dtype)


def oracle_rho(s: InputSet) -> np.ndarray:
    return oracle.probe(s.W_R, s.x, s.wl.Hq, s.wl.d)


def oracle_out(s: InputSet, rho: np.ndarray, pairs=None) -> np.ndarray:
    """Oracle output for all (b, h) or the listed pairs (rows in pair order)."""
    q = s.q.float().numpy().astype(np.float64)
    if pairs is None:
        return oracle.decode(q, rho, s.K, s.V, s.seq_lens.tolist(), s.wl.Hkv)
    return oracle.decode_heads(q, rho, s.K, s.V, s.seq_lens.tolist(), s.wl.Hkv, pairs)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_rne(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even), returned as float64."""
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def sample_pairs(s: InputSet, k: int, seed: int = 0):
    """k (b, h) pairs, always including the longest and the shortest sequence."""
    B, Hq = s.wl.B, s.wl.Hq
    r = np.random.default_rng(seed)
    lens = s.seq_lens.numpy()
    pairs = {(int(np.argmax(lens)), 0), (int(np.argmax(lens)), Hq - 1), (int(np.argmin(lens)), 1 % Hq)}
    while len(pairs) < min(k, B * Hq):
        pairs.add((int(r.integers(B)), int(r.integers(Hq))))
    return sorted(pairs)
