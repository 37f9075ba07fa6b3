"""GPU parity of the causal many-query forward (parallax_prefill) against the
fp64 oracle's prefill, through the C ABI.

Inputs: seeded bf16 q, K, V and an fp32 probe rho = W_R x computed by the
oracle (the same rho goes to both sides); K/V caches padded with NaN past each
sequence's prefix + T rows, so any read past them would surface.

Tolerances: the bf16 output as for decode (rel-L2 <= 2e-3 against the fp64
oracle, and equal bit for bit to the RNE rounding of the fp32 output). The
fp32 output carries the kernel's own error: rho and the weights e and e*p enter
the bf16 matrix cores as hi + lo pairs (16 significant bits, relative error
<= 2^-17 each), so rel-L2 <= 2e-5 and max-abs <= 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
from parallax_covariance_corrected_amd import binding as pb
from parallax_covariance_corrected_amd.workloads import WORKLOADS, make_prefill_inputs, padded_cache
from _gpu_common import BF16_REL_L2, bf16_rne, max_abs, rel_l2, say, to64

pytestmark = pytest.mark.gpu

F32OUT_REL = 2e-5
F32OUT_ABS = 1e-3


def _rho(s):
    """rho [B, T, Hq, d] = W_R x per token (oracle probe), as fp32."""
    wl = s.wl
    x = s.x.reshape(wl.B * s.T, wl.d_model)
    r = oracle.probe(s.W_R, x, wl.Hq, wl.d).reshape(wl.B, s.T, wl.Hq, wl.d)
    return r.astype(np.float32)


def _run(s, rho32, out_dtype, max_ctx=None, with_prefix=True):
    wl = s.wl
    mc = max_ctx or s.max_ctx
    K = padded_cache(s.K, mc, device="cuda")
    V = padded_cache(s.V, mc, device="cuda")
    pre = s.prefix.cuda() if with_prefix else None
    out = pb.prefill(s.q.cuda(), torch.from_numpy(rho32).cuda(), K, V, pre, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to64(out)


def _oracle(s, rho32):
    return oracle.prefill(s.q, rho32.astype(np.float64), s.K, s.V, s.prefix.numpy(), s.wl.Hkv)


CASES = [  # (Hq, Hkv, d, T, prefix)
    (4, 2, 128, 1, [0, 9]),
    (4, 2, 128, 63, [0, 37]),
    (4, 2, 128, 200, [100, 5]),
    (16, 8, 128, 129, [0, 64]),
    (6, 2, 128, 70, [3, 0]),        # G = 3: rows of one token straddle waves
    (8, 1, 64, 40, [0, 130]),       # G = 8
    (2, 2, 64, 97, [0, 1]),         # G = 1
    (4, 2, 64, 150, [64, 0]),
    (32, 8, 128, 40, [0, 150]),     # G = 4 (the ragged workload's heads)
    (12, 2, 64, 45, [7, 0]),        # G = 6
]


@pytest.mark.parametrize("Hq,Hkv,d,T,prefix", CASES)
def test_prefill_matches_oracle(Hq, Hkv, d, T, prefix):
    wl = WORKLOADS[2].scaled(B=len(prefix), Hq=Hq, Hkv=Hkv, d=d, d_model=256)
    s = make_prefill_inputs(wl, T, prefix, seed=T + d)
    say(f"[case] prefill Hq={Hq} Hkv={Hkv} d={d} T={T} prefix={prefix}")
    rho = _rho(s)
    ref = _oracle(s, rho)
    o32 = _run(s, rho, torch.float32)
    obf = _run(s, rho, torch.bfloat16)
    e32, a32, ebf = rel_l2(o32, ref), max_abs(o32, ref), rel_l2(obf, ref)
    say(f"prefill Hq={Hq} Hkv={Hkv} d={d} T={T}: f32 rel {e32:.2e} abs {a32:.2e}, bf16 rel {ebf:.2e}")
    assert e32 <= F32OUT_REL and a32 <= F32OUT_ABS
    assert ebf <= BF16_REL_L2
    np.testing.assert_array_equal(obf, bf16_rne(o32))


@pytest.mark.parametrize("Hq,Hkv,d,T,prefix", [(4, 2, 128, 150, [0, 70]), (8, 2, 64, 65, [3, 0])])
def test_softmax_prefill_matches_oracle(Hq, Hkv, d, T, prefix):
    """rho = None: plain causal softmax attention (the oracle with rho = 0)."""
    wl = WORKLOADS[2].scaled(B=len(prefix), Hq=Hq, Hkv=Hkv, d=d, d_model=256)
    s = make_prefill_inputs(wl, T, prefix, seed=3 * T)
    say(f"[case] softmax prefill Hq={Hq} Hkv={Hkv} d={d} T={T} prefix={prefix}")
    K = padded_cache(s.K, s.max_ctx, device="cuda")
    V = padded_cache(s.V, s.max_ctx, device="cuda")
    o32 = to64(pb.prefill(s.q.cuda(), None, K, V, s.prefix.cuda(), out_dtype=torch.float32))
    obf = to64(pb.prefill(s.q.cuda(), None, K, V, s.prefix.cuda()))
    torch.cuda.synchronize()
    ref = oracle.prefill(s.q, np.zeros((len(prefix), T, Hq, d)), s.K, s.V, s.prefix.numpy(), Hkv)
    e = rel_l2(o32, ref)
    say(f"softmax prefill: f32 rel {e:.2e}, bf16 rel {rel_l2(obf, ref):.2e}")
    assert e <= F32OUT_REL and max_abs(o32, ref) <= F32OUT_ABS
    assert rel_l2(obf, ref) <= BF16_REL_L2
    np.testing.assert_array_equal(obf, bf16_rne(o32))


def test_prefill_without_prefix_pointer_and_larger_cache():
    """prefix_lens = null means no cached prefix; a cache larger than needed
    (NaN beyond the valid rows) changes nothing."""
    wl = WORKLOADS[2].scaled(B=2, Hq=4, Hkv=2, d=128, d_model=256)
    s = make_prefill_inputs(wl, 90, [0, 0], seed=5)
    rho = _rho(s)
    ref = _oracle(s, rho)
    a = _run(s, rho, torch.float32, with_prefix=False)
    b = _run(s, rho, torch.float32, max_ctx=s.max_ctx + 300)
    assert rel_l2(a, ref) <= F32OUT_REL
    np.testing.assert_array_equal(a, b)


def test_prefill_last_token_equals_decode():
    """The last token of a prefill is a decode over the whole sequence."""
    wl = WORKLOADS[2].scaled(B=2, Hq=4, Hkv=2, d=128, d_model=256)
    s = make_prefill_inputs(wl, 40, [300, 1000], seed=9)
    rho = _rho(s)
    o = _run(s, rho, torch.float32)
    K = padded_cache(s.K, s.max_ctx, device="cuda")
    V = padded_cache(s.V, s.max_ctx, device="cuda")
    lens = (s.prefix + s.T).to(torch.int32).cuda()
    dec = pb.decode(s.q[:, -1].contiguous().cuda(), torch.from_numpy(rho[:, -1].copy()).cuda(), K, V,
                    lens, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.decode(s.q[:, -1], rho[:, -1].astype(np.float64), s.K, s.V, lens.cpu().numpy(), wl.Hkv)
    assert rel_l2(to64(dec), ref) <= 1e-5
    assert rel_l2(o[:, -1], ref) <= F32OUT_REL


def test_prefill_full_size_sampled():
    """B = 1, T = 4096 (the pretraining context), Hq = 16, Hkv = 8, d = 128, on
    sampled (token, head) rows, always including the first and last token."""
    wl = WORKLOADS[2].scaled(B=1)
    T = 4096
    s = make_prefill_inputs(wl, T, [0], seed=1)
    say(f"[case] prefill full size T={T}")
    rho = _rho(s)
    o32 = _run(s, rho, torch.float32)
    r = np.random.default_rng(0)
    rows = [(0, 0, 0), (0, T - 1, 15), (0, 63, 3), (0, 64, 4)]
    rows += [(0, int(t), int(h)) for t, h in zip(r.integers(0, T, 20), r.integers(0, 16, 20))]
    ref = oracle.prefill_rows(s.q, rho.astype(np.float64), s.K, s.V, s.prefix.numpy(), wl.Hkv, rows)
    got = np.stack([o32[b, t, h] for b, t, h in rows])
    e, a = rel_l2(got, ref), max_abs(got, ref)
    say(f"prefill full size: rel {e:.2e} abs {a:.2e}")
    assert e <= F32OUT_REL and a <= F32OUT_ABS


@pytest.mark.parametrize("Hq,Hkv,d,T,prefix", [(2, 2, 64, 60, [0, 13]), (6, 2, 128, 33, [70, 0])])
def test_fp32_prefill_matches_oracle(Hq, Hkv, d, T, prefix):
    """fp32 inputs go through the vector-ALU kernel (one single-token
    sequence per token): rel-L2 and max-abs within 1e-5, as for fp32 decode."""
    wl = WORKLOADS[1].scaled(B=len(prefix), Hq=Hq, Hkv=Hkv, d=d, d_model=128)
    s = make_prefill_inputs(wl, T, prefix, seed=2 * T)
    say(f"[case] fp32 prefill Hq={Hq} Hkv={Hkv} d={d} T={T} prefix={prefix}")
    rho = _rho(s)
    ref = _oracle(s, rho)
    o = _run(s, rho, torch.float32)
    soft = pb.prefill(s.q.cuda(), None, padded_cache(s.K, s.max_ctx, device="cuda"),
                      padded_cache(s.V, s.max_ctx, device="cuda"), s.prefix.cuda())
    torch.cuda.synchronize()
    ref0 = oracle.prefill(s.q, np.zeros_like(rho, dtype=np.float64), s.K, s.V, s.prefix.numpy(), Hkv)
    say(f"fp32 prefill: rel {rel_l2(o, ref):.2e} abs {max_abs(o, ref):.2e}; "
        f"softmax rel {rel_l2(to64(soft), ref0):.2e}")
    assert rel_l2(o, ref) <= 1e-5 and max_abs(o, ref) <= 1e-5
    assert rel_l2(to64(soft), ref0) <= 1e-5


def test_prefill_rejects_bad_arguments():
    wl = WORKLOADS[2].scaled(B=1, Hq=4, Hkv=2, d=128, d_model=256)
    s = make_prefill_inputs(wl, 8, [0], seed=0)
    q = s.q.cuda()
    rho = torch.zeros((1, 8, 4, 128), device="cuda")
    K = padded_cache(s.K, 8, device="cuda")
    with pytest.raises(pb.ParallaxError):
        pb.prefill(q, rho, K[:, :, :4].contiguous(), K[:, :, :4].contiguous())   # T > max_ctx
    with pytest.raises(ValueError):
        pb.prefill(q, rho, K.float(), K.float())      # mixed dtypes


def test_prefill_zero_covariance_closed_forms():
    """The causal forward on degenerate caches, against closed forms: all keys
    of sequence 0 equal (token t sees prefix + t + 1 equal scores, so its output
    is the mean of those values) and all values of sequence 1 equal (every
    output is that value), with a large probe (W_R ~ N(0, 1), |p| up to a few
    hundred) so that the one-pass form must cancel P/l - vbar S/l; sequence 2
    is ordinary. The bound per output row follows the kernel's precision
    model: e p enters the matrix cores as a 16-bit hi + lo pair while S sums it
    in fp32, so the cancellation leaves at most 2^-16 sum_j w_j |p_j| |v_j|
    (w, p in fp64 from the same inputs), plus fp32 rounding."""
    wl = WORKLOADS[2].scaled(B=3, Hq=8, Hkv=2, d=128, d_model=64, wr_std=1.0)
    prefix = [40, 0, 17]
    s = make_prefill_inputs(wl, 150, prefix, seed=77)
    K0, V1 = s.K[0].clone(), s.V[1].clone()
    K0[:] = K0[:, :1, :]
    V1[:] = V1[:, :1, :]
    s.K[0], s.V[1] = K0, V1
    say("[case] prefill zero covariance")
    rho = _rho(s)
    o32 = _run(s, rho, torch.float32)
    obf = _run(s, rho, torch.bfloat16)
    G = wl.Hq // wl.Hkv
    q64 = s.q.float().numpy().astype(np.float64)
    r64 = rho.astype(np.float64)
    worst = 0.0
    for b, closed in ((0, "mean"), (1, "value")):
        for g in range(wl.Hkv):
            Kg, Vg = s.K[b][g].double().numpy(), s.V[b][g].double().numpy()
            for t in range(s.T):
                n = prefix[b] + t + 1
                want = Vg[:n].mean(0) if closed == "mean" else Vg[0]
                for h in range(g * G, (g + 1) * G):
                    w = oracle.softmax_weights(q64[b, t, h], Kg[:n])
                    p = np.abs(Kg[:n] @ r64[b, t, h])
                    bound = 2.0 ** -16 * float(w @ (p * np.abs(Vg[:n]).max(1))) + 2e-6
                    err = float(np.abs(o32[b, t, h] - want).max())
                    worst = max(worst, err / bound)
                    assert err <= bound, (b, t, h, err, bound)
    say(f"prefill zero covariance: worst error / model bound {worst:.3f}")
    np.testing.assert_array_equal(obf, bf16_rne(o32))
    rows = [(2, t, h) for t in (0, 75, 149) for h in range(wl.Hq)]
    ref = oracle.prefill_rows(s.q, r64, s.K, s.V, s.prefix.numpy(), wl.Hkv, rows)
    got = np.stack([o32[b, t, h] for b, t, h in rows])
    assert rel_l2(got, ref) <= F32OUT_REL
