"""fp64 CPU oracle for Parallax decode attention (test infrastructure only:
imported by tests, the smoke check and the bench's CPU-baseline leg, never by
the product path). ``oracle.lla_oracle`` adds the exact local-linear-attention
reference (a per-query conjugate-gradient solve) that Parallax replaces."""
from .parallax_oracle import (probe, softmax_weights, weighted_means, kv_covariance,
                              decode_head, decode, decode_heads, kv_head_of, clamp_len,
                              prefill, prefill_rows)

__all__ = ["probe", "softmax_weights", "weighted_means", "kv_covariance",
           "decode_head", "decode", "decode_heads", "kv_head_of", "clamp_len", "prefill",
           "prefill_rows"]
