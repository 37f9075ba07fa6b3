"""The allocation-free decode step (parallax_probe_decode_noalloc, through the
C ABI) against parallax_probe_decode on the same inputs: two calls in a row,
the second on a smaller input, so the second one runs over what the first
left in the shared static scratch array. Each must equal the allocating
call's output bit for bit (same plan and kernels) and match the fp64 oracle
within the bf16 output tolerance."""
import numpy as np
import pytest
import torch

from parallax_covariance_corrected_amd import binding as pb
from parallax_covariance_corrected_amd.workloads import WORKLOADS, make_inputs

from _gpu_common import BF16_REL_L2, Device, oracle_out, oracle_rho, rel_l2, say, to64

pytestmark = pytest.mark.gpu

# (input set, expected probe placement): the first is the larger one, with
# the probe in its own launch (rho in the scratch array) and six splits; the
# second is smaller, probe fused into the decode, six splits.
CALLS = [
    (dict(wl=WORKLOADS[5].scaled(B=6, ctx=6000), seed=31), False),
    (dict(wl=WORKLOADS[2].scaled(B=3, ctx=700, d_model=64), seed=32, lengths=[700, 129, 1]), True),
]


def test_noalloc_step_matches_allocating_step():
    assert pb.noalloc_scratch_bytes() == 64 << 20
    for kw, fused in CALLS:
        s = make_inputs(kw["wl"], kw["seed"], lengths=kw.get("lengths"))
        wl = s.wl
        say(f"[case] noalloc B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} ctx={wl.ctx} d_model={wl.d_model}")
        assert pb.probe_decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.d_model, wl.capacity) == fused
        _, splits, _ = pb.decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.capacity)
        assert splits > 1
        dev = Device(s)
        out_na = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        ref = pb.probe_decode(dev.W_R, dev.x, dev.q, dev.K, dev.V, dev.seq_lens)
        pb.probe_decode(dev.W_R, dev.x, dev.q, dev.K, dev.V, dev.seq_lens, out=out_na, noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(out_na.view(torch.int16), ref.view(torch.int16))
        want = oracle_out(s, oracle_rho(s))
        e = rel_l2(to64(out_na), want)
        say(f"noalloc B={wl.B}: bit-equal to probe_decode, rel_l2 vs oracle {e:.3e}")
        assert e <= BF16_REL_L2

