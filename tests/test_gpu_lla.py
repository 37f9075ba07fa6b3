"""Exact local linear attention through the HIP decode path.

Exact LLA is the Parallax output with the probe replaced by the per-query solve
rho* = (Sigma_kk + lam I)^{-1} (kbar - q) (reference: oracle/lla_oracle.py,
conjugate gradients in fp64). Feeding rho* (rounded to fp32, the probe type of
the boundary) to parallax_decode must reproduce the exact LLA output: the
kernel's covariance branch is then the whole local-linear correction, about
90% of the output here.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import lla_oracle as lla
from parallax_covariance_corrected_amd import binding as pb
from parallax_covariance_corrected_amd.workloads import WORKLOADS, make_inputs
from _gpu_common import BF16_REL_L2, Device, bf16_rne, max_abs, oracle_out, rel_l2, say, to64

pytestmark = pytest.mark.gpu

LAM = 0.1


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("chunk", [0, 64])
def test_decode_with_solved_probe_is_exact_lla(d, chunk):
    wl = WORKLOADS[2].scaled(B=3, Hq=4, Hkv=2, d=d, ctx=1000, d_model=256)
    s = make_inputs(wl, 21, lengths=[1000, 300, 129])
    say(f"[case] lla d={d} chunk={chunk} lengths={s.seq_lens.tolist()}")
    q64 = s.q.float().numpy().astype(np.float64)
    want, rho = lla.lla_decode(q64, s.K, s.V, s.seq_lens.numpy(), wl.Hkv, LAM)
    rho32 = rho.astype(np.float32)
    dev = Device(s)
    with pb.options(chunk=chunk):
        o32 = dev.decode(torch.from_numpy(rho32).cuda(), out_dtype=torch.float32)
        obf = dev.decode(torch.from_numpy(rho32).cuda())
    torch.cuda.synchronize()
    # Precision model of the matrix-core kernel: it multiplies the keys by rho
    # carried as two bf16 terms, hi = bf16(rho) and lo = bf16(rho - hi) (16
    # significant bits). Against the oracle fed exactly hi + lo the kernel is
    # at fp32 accumulation error; against exact LLA the 16-bit probe adds
    # about 2e-5 here, where the correction is ~90% of the output and |rho*|
    # reaches 10 (a fp32-exact probe would cost ~2% more decode time).
    hi = bf16_rne(rho32.astype(np.float64))
    lo = bf16_rne(rho32.astype(np.float64) - hi)
    modeled = oracle_out(s, hi + lo)
    e_lla, e_model = rel_l2(to64(o32), want), rel_l2(to64(o32), modeled)
    say(f"lla d={d} chunk={chunk}: rel vs LLA {e_lla:.2e}, vs oracle(hi+lo rho) {e_model:.2e}, "
        f"max-abs {max_abs(to64(o32), want):.2e}, bf16 rel {rel_l2(to64(obf), want):.2e}")
    assert e_model <= 2e-6
    assert e_lla <= 5e-5
    # The bound the boundary documents for the 16-bit probe, computed here in
    # fp64 from the oracle's weights: per output component,
    # 2^-16 sum_j w_j (sum_i |k_ji rho_i|) |v_j - vbar| (plus fp32 rounding of
    # rho itself and of the kernel's sums), against the exact LLA output.
    G = wl.Hq // wl.Hkv
    got = to64(o32)
    scale = np.abs(want).max()
    for b, n in enumerate(s.seq_lens.tolist()):
        for h in range(wl.Hq):
            Kb = s.K[b][h // G].double().numpy()
            Vb = s.V[b][h // G].double().numpy()
            w = oracle.softmax_weights(q64[b, h], Kb)
            vbar = w @ Vb
            kr = np.abs(Kb) @ np.abs(rho[b, h])
            bound = (2.0 ** -16 + 2.0 ** -24) * ((w * kr) @ np.abs(Vb - vbar))
            err = np.abs(got[b, h] - want[b, h])
            assert np.all(err <= bound + 2e-6 * scale), (b, h, float((err - bound).max()))
    assert max_abs(to64(o32), want) <= 1e-3
    assert rel_l2(to64(obf), want) <= BF16_REL_L2
