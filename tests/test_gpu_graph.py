"""A decode step (probe + split-K decode + merge) captured into a HIP graph.

The library launches no memset and allocates only when a stream's workspace
must grow, which it refuses during capture; after one call of the shape on the
capture stream, a step can be captured and replayed. Every replay, with eager
work and synchronisations between replays and new inputs copied into the
captured buffers, must equal the eager result bit for bit.
"""
import pytest
import torch

from parallax_covariance_corrected_amd import binding as pb
from parallax_covariance_corrected_amd.workloads import WORKLOADS, make_inputs
from _gpu_common import Device, say

pytestmark = pytest.mark.gpu


def test_decode_step_in_a_graph_replays_exactly():
    wl = WORKLOADS[2].scaled(B=4, ctx=1500, d_model=512)   # several splits: the merge runs
    assert pb.decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.capacity)[1] > 1
    sets = [make_inputs(wl, seed) for seed in (11, 12, 13)]
    devs = [Device(s, pad=0.0) for s in sets]
    say(f"[case] graph decode B={wl.B} ctx={wl.ctx}")

    def eager(dv):
        rho = pb.probe(dv.W_R, dv.x, wl.Hq, wl.d)
        out = pb.decode(dv.q, rho, dv.K, dv.V, dv.seq_lens)
        torch.cuda.synchronize()
        return out.clone()

    refs = [eager(dv) for dv in devs]

    # Static buffers the graph reads and writes.
    st = Device(sets[0], pad=0.0)
    rho = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.float32, device="cuda")
    out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):   # size this stream's workspace before capture
        pb.probe(st.W_R, st.x, wl.Hq, wl.d, out=rho)
        pb.decode(st.q, rho, st.K, st.V, st.seq_lens, out=out)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pb.probe(st.W_R, st.x, wl.Hq, wl.d, out=rho)
        pb.decode(st.q, rho, st.K, st.V, st.seq_lens, out=out)
    torch.cuda.synchronize()

    for rep in range(6):
        i = rep % 3
        for name in ("x", "W_R", "q", "K", "V", "seq_lens"):
            getattr(st, name).copy_(getattr(devs[i], name))
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, refs[i]), f"replay {rep} (input set {i}) differs from eager"
        # eager work between replays, on the default stream
        again = eager(devs[(i + 1) % 3])
        assert torch.equal(again, refs[(i + 1) % 3])
    say("graph decode: 6 replays equal to eager")


@pytest.mark.parametrize("fuse", [1, 2])
def test_one_call_step_in_a_graph_replays_exactly(fuse):
    """parallax_probe_decode captured into a graph, with the probe in a launch
    of its own (rho in the library's workspace) and fused into the decode."""
    wl = WORKLOADS[2].scaled(B=4, ctx=1500, d_model=64)
    sets = [make_inputs(wl, seed) for seed in (21, 22, 23)]
    devs = [Device(s, pad=0.0) for s in sets]
    say(f"[case] graph probe_decode fuse={fuse} B={wl.B} ctx={wl.ctx}")
    with pb.options(fuse=fuse):
        assert pb.probe_decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.d_model, wl.capacity) == (fuse == 2)

        def eager(dv):
            out = pb.probe_decode(dv.W_R, dv.x, dv.q, dv.K, dv.V, dv.seq_lens)
            torch.cuda.synchronize()
            return out.clone()

        refs = [eager(dv) for dv in devs]
        st = Device(sets[0], pad=0.0)
        out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.bfloat16, device="cuda")
        s = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):   # size this stream's workspace before capture
            pb.probe_decode(st.W_R, st.x, st.q, st.K, st.V, st.seq_lens, out=out)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            pb.probe_decode(st.W_R, st.x, st.q, st.K, st.V, st.seq_lens, out=out)
        torch.cuda.synchronize()
        for rep in range(6):
            i = rep % 3
            for name in ("x", "W_R", "q", "K", "V", "seq_lens"):
                getattr(st, name).copy_(getattr(devs[i], name))
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, refs[i]), f"replay {rep} (input set {i}) differs from eager"
            again = eager(devs[(i + 1) % 3])
            assert torch.equal(again, refs[(i + 1) % 3])
    say(f"graph probe_decode fuse={fuse}: 6 replays equal to eager")
