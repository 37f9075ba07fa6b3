"""GPU parity of parallax_probe_decode, the whole decode step in one call (the
probe rho = W_R x, then the Parallax decode), against the fp64 oracle, with the
probe inside the decode kernel (fused) and as a separate launch.

The K/V caches are padded with NaN past every length. Tolerances as in the
decode parity tests: bf16 output rel-L2 <= 2e-3, the fp32 output of the same
plan max-abs <= 1e-2 and its RNE rounding equal to the bf16 output bit for bit;
fp32 inputs rel-L2 and max-abs <= 1e-5. Fused and separate results differ only
by the fp32 rounding of rho (accumulated in another order), so their fp32
outputs must agree to 1e-5 relative.
"""
import numpy as np
import pytest
import torch

from parallax_covariance_corrected_amd import binding as pb
from parallax_covariance_corrected_amd.workloads import WORKLOADS, make_inputs

from _gpu_common import (BF16_REL_L2, F32OUT_MAX_ABS, F32_TOL, Device, bf16_rne, max_abs,
                         oracle_out, oracle_rho, rel_l2, sample_pairs, say, to64)

pytestmark = pytest.mark.gpu


def _pd(dev: Device, out_dtype=None) -> torch.Tensor:
    return pb.probe_decode(dev.W_R, dev.x, dev.q, dev.K, dev.V, dev.seq_lens, out_dtype=out_dtype)


def _plan(s) -> bool:
    wl = s.wl
    code = pb.F32 if wl.dtype == "f32" else pb.BF16
    return pb.probe_decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.d_model, s.max_ctx, code)


def _check(s, dev, ref, tag, pairs=None):
    """Output of probe_decode under the current options against the oracle;
    returns the fp32 output (bf16 inputs) or the output (fp32 inputs)."""
    if s.wl.dtype == "f32":
        o = to64(_pd(dev))
        torch.cuda.synchronize()
        if pairs is not None:
            o = np.stack([o[b, h] for b, h in pairs])
        say(f"{tag}: rel {rel_l2(o, ref):.3e} max_abs {max_abs(o, ref):.3e}")
        assert rel_l2(o, ref) <= F32_TOL and max_abs(o, ref) <= F32_TOL, tag
        return o
    o16, o32 = to64(_pd(dev)), to64(_pd(dev, torch.float32))
    torch.cuda.synchronize()
    if pairs is not None:
        o16 = np.stack([o16[b, h] for b, h in pairs])
        o32 = np.stack([o32[b, h] for b, h in pairs])
    assert np.isfinite(o32).all(), f"{tag}: non-finite output"
    e16, m32 = rel_l2(o16, ref), max_abs(o32, ref)
    say(f"{tag}: rel_l2 bf16 {e16:.3e} max_abs fp32out {m32:.3e}")
    assert e16 <= BF16_REL_L2, (tag, e16)
    assert m32 <= F32OUT_MAX_ABS, (tag, m32)
    np.testing.assert_array_equal(o16, bf16_rne(o32), err_msg=f"{tag}: bf16 out != RNE(fp32 out)")
    return o32


def _both_paths(s, tag, expect_fusable=True, pairs=None):
    say(f"[case] {tag} B={s.wl.B} Hq={s.wl.Hq} Hkv={s.wl.Hkv} d={s.wl.d} "
        f"d_model={s.wl.d_model} {s.wl.dtype} lens={s.seq_lens.tolist()[:12]}")
    dev = Device(s)
    ref = oracle_out(s, oracle_rho(s), pairs)
    with pb.options(fuse=2):
        assert _plan(s) == expect_fusable, tag
        fused = _check(s, dev, ref, tag + " fused", pairs)
    with pb.options(fuse=1):
        assert not _plan(s)
        sep = _check(s, dev, ref, tag + " separate", pairs)
    d = rel_l2(fused, sep)
    say(f"{tag}: fused vs separate rel {d:.3e}")
    assert d <= 1e-5, (tag, d)
    return dev, fused


def test_tiny_fp32_workload_runs_fused():
    wl = WORKLOADS[1]
    for wr_zero in (False, True):
        s = make_inputs(wl, 0, wr_zero=wr_zero)
        assert _plan(s), "the tiny fp32 workload takes the fused plan"
        tag = f"tiny fp32 wr_zero={wr_zero}"
        say(f"[case] {tag}")
        dev = Device(s)
        ref = oracle_out(s, oracle_rho(s))
        _check(s, dev, ref, tag + " auto")
        _both_paths(s, tag)


EDGE_LENS = [0, 1, 15, 16, 17, 127, 128, 129, 300]

# (d, Hq, Hkv, dtype, d_model): head blocks of 1 to 8 query heads on the
# matrix-core kernel (1 to 4 on the generic one), d_model from one 16-byte
# piece per row to a ragged number of pieces.
SHAPES = [(128, 4, 2, "bf16", 256), (64, 6, 2, "bf16", 64), (128, 32, 8, "bf16", 128),
          (128, 10, 2, "bf16", 8), (64, 3, 3, "bf16", 2056), (128, 16, 2, "bf16", 136),
          (64, 14, 2, "bf16", 72), (128, 12, 2, "bf16", 24),
          (128, 4, 2, "f32", 96), (64, 2, 1, "f32", 4), (128, 6, 3, "f32", 260)]


@pytest.mark.parametrize("d,Hq,Hkv,dtype,d_model", SHAPES)
def test_fused_and_separate_match_oracle(d, Hq, Hkv, dtype, d_model):
    """Lengths 0, 1, tile and chunk boundaries and the cache size; one split
    (default plan at this cache size) and 128-key chunks (three splits and the
    merge); for bf16 also the generic kernel."""
    wl = WORKLOADS[2].scaled(B=len(EDGE_LENS), Hq=Hq, Hkv=Hkv, d=d, ctx=300, d_model=d_model,
                             dtype=dtype, wr_std=0.05)
    s = make_inputs(wl, 4, lengths=EDGE_LENS)
    tag = f"d={d} Hq={Hq} Hkv={Hkv} {dtype} d_model={d_model}"
    dev, fused = _both_paths(s, tag)
    assert np.all(fused[0] == 0.0), "length 0 gives 0"
    with pb.options(chunk=128):
        _both_paths(s, tag + " chunk=128")
    if dtype == "bf16":
        with pb.options(kernel=1):
            _both_paths(s, tag + " generic kernel")


def test_fp32_rows_not_in_whole_pieces_use_the_separate_probe():
    wl = WORKLOADS[1].scaled(B=3, d_model=130, ctx=200)
    s = make_inputs(wl, 6, lengths=[200, 77, 1])
    _both_paths(s, "fp32 d_model=130", expect_fusable=False)


def test_long_context_splits_fused():
    """One sequence over many splits (the merge combines the fused items)."""
    wl = WORKLOADS[3].scaled(ctx=9000, d_model=128)
    s = make_inputs(wl, 1)
    _both_paths(s, "long ctx d_model=128")


@pytest.mark.parametrize("idx", [2, 4, 5])
def test_full_size_separate_plan_equals_probe_then_decode(idx):
    """On the bf16 workloads the plan keeps the probe separate; the result is
    then bit for bit that of parallax_probe followed by parallax_decode (same
    kernels), and forcing the fused plan changes it only by rho's rounding."""
    s = make_inputs(WORKLOADS[idx], 0)
    assert not _plan(s)
    say(f"[case] full size {WORKLOADS[idx].name}")
    dev = Device(s)
    one = _pd(dev, torch.float32)
    two = dev.decode(dev.probe(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    torch.testing.assert_close(one, two, rtol=0, atol=0)
    pairs = sample_pairs(s, 24)
    ref = oracle_out(s, oracle_rho(s), pairs)
    o = to64(one)
    o = np.stack([o[b, h] for b, h in pairs])
    say(f"full size: max_abs fp32out {max_abs(o, ref):.3e}")
    assert max_abs(o, ref) <= F32OUT_MAX_ABS
    if idx == 2:
        with pb.options(fuse=2):
            assert _plan(s)
            f = _pd(dev, torch.float32)
            torch.cuda.synchronize()
        d = rel_l2(to64(f), to64(one))
        say(f"full size forced fused vs separate rel {d:.3e}")
        assert d <= 1e-5


def test_random_shapes_both_placements():
    """Twenty seeded random shapes: batch 1-9, G in 1..8, d in {64, 128},
    d_model a multiple of 8 up to 600, cache 1-700 keys with random lengths
    (zero allowed), forced chunk sizes; probe fused and separate against the
    oracle."""
    rng = np.random.default_rng(2026)
    for case in range(20):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 4))
        G = int(rng.integers(1, 9))
        B = int(rng.integers(1, 10))
        cap = int(rng.integers(1, 701))
        d_model = 8 * int(rng.integers(1, 76))
        lens = [int(x) for x in rng.integers(0, cap + 1, size=B)]
        chunk = int(rng.choice([0, 64, 128, 256]))
        wl = WORKLOADS[2].scaled(B=B, Hq=G * Hkv, Hkv=Hkv, d=d, ctx=cap, d_model=d_model,
                                 wr_std=0.05)
        s = make_inputs(wl, 100 + case, lengths=lens)
        with pb.options(chunk=chunk):
            _both_paths(s, f"random case {case} chunk={chunk}")
