"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every K/V cache is padded with NaN past each sequence length, so any read past
seq_lens shows up as a NaN output. Tolerances: bf16 output rel-L2 <= 2e-3; the
same kernel with an fp32 output max-abs <= 1e-2 (and bf16 output == RNE of
that fp32 output, bitwise); fp32 path rel-L2 and max-abs <= 1e-5; probe rel-L2
<= 1e-5.
"""
import numpy as np
import pytest
import torch

from parallax_covariance_corrected_amd import binding as pb
from parallax_covariance_corrected_amd.workloads import WORKLOADS, make_inputs

from _gpu_common import (BF16_REL_L2, F32OUT_MAX_ABS, F32_TOL, RHO_REL_L2, Device, bf16_rne,
                         max_abs, oracle_out, oracle_rho, rel_l2, sample_pairs, say, to64)

pytestmark = pytest.mark.gpu


def _check_bf16(s, dev, rho_dev, ref, pairs=None, tag=""):
    """bf16 and fp32-output runs of the same plan against the oracle."""
    out16 = dev.decode(rho_dev)
    out32 = dev.decode(rho_dev, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o16, o32 = to64(out16), to64(out32)
    if pairs is not None:
        o16 = np.stack([o16[b, h] for b, h in pairs])
        o32 = np.stack([o32[b, h] for b, h in pairs])
    assert np.isfinite(o32).all(), f"{tag}: non-finite output"
    e16, e32, m32 = rel_l2(o16, ref), rel_l2(o32, ref), max_abs(o32, ref)
    say(f"{tag}: rel_l2 bf16 {e16:.3e} fp32out {e32:.3e} max_abs fp32out {m32:.3e}")
    assert e16 <= BF16_REL_L2, (tag, e16)
    assert m32 <= F32OUT_MAX_ABS, (tag, m32)
    np.testing.assert_array_equal(o16, bf16_rne(o32), err_msg=f"{tag}: bf16 out != RNE(fp32 out)")
    return o32


def _run_full_check(s, tag, pairs=None, wr_zero_too=True):
    say(f"[case] {tag} B={s.wl.B} Hq={s.wl.Hq} Hkv={s.wl.Hkv} d={s.wl.d} "
        f"lens[min,max]=[{int(s.seq_lens.min())},{int(s.seq_lens.max())}] seed={s.seed}")
    dev = Device(s)
    rho = dev.probe()
    torch.cuda.synchronize()
    rho_o = oracle_rho(s)
    er = rel_l2(to64(rho), rho_o)
    say(f"{tag}: rho rel_l2 {er:.3e}")
    assert er <= RHO_REL_L2
    ref = oracle_out(s, rho_o, pairs)
    _check_bf16(s, dev, rho, ref, pairs, tag)
    if wr_zero_too:
        zero = torch.zeros_like(rho)
        ref0 = oracle_out(s, np.zeros_like(rho_o), pairs)
        _check_bf16(s, dev, zero, ref0, pairs, tag + " W_R=0")


# ------------------------------------------------------------------ tiny fp32 workload
def test_tiny_fp32_workload():
    wl = WORKLOADS[1]
    for wr_zero in (False, True):
        s = make_inputs(wl, 0, wr_zero=wr_zero)
        say(f"[case] tiny fp32 wr_zero={wr_zero}")
        dev = Device(s)
        rho = dev.probe()
        out = dev.decode(rho)
        torch.cuda.synchronize()
        rho_o = oracle_rho(s)
        ref = oracle_out(s, rho_o)
        o = to64(out)
        say(f"tiny fp32: rho rel {rel_l2(to64(rho), rho_o):.3e} out rel {rel_l2(o, ref):.3e} "
            f"max_abs {max_abs(o, ref):.3e}")
        assert rel_l2(to64(rho), rho_o) <= F32_TOL
        assert rel_l2(o, ref) <= F32_TOL and max_abs(o, ref) <= F32_TOL
        if wr_zero:
            # W_R = 0 is plain softmax attention: compare with torch SDPA too
            qt = s.q.double()[:, :, None, :]
            kt = torch.stack([k for k in s.K]).double()
            vt = torch.stack([v for v in s.V]).double()
            sdpa = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, :, 0]
            assert max_abs(o, sdpa.numpy()) <= F32_TOL


# ------------------------------------------------------------------ bf16 workloads, reduced size
SMALL = {
    "gqa_mid_ctx": (WORKLOADS[2].scaled(B=3), [4096, 1000, 37]),
    "long_ctx_full": (WORKLOADS[3], None),
    "large_batch": (WORKLOADS[4].scaled(B=40), None),
    "ragged_G4": (WORKLOADS[5].scaled(B=6, ctx=6000), None),
}


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("name", list(SMALL))
def test_bf16_workloads_reduced(name, seed):
    wl, lengths = SMALL[name]
    s = make_inputs(wl, seed, lengths=lengths)
    _run_full_check(s, f"{name} seed{seed}")


# ------------------------------------------------------------------ full sizes
def heads_of_every_sequence(s, per_seq: int = 4, seed: int = 0):
    """per_seq distinct query heads of every sequence (seeded), plus the first
    and last head of the longest one."""
    r = np.random.default_rng(seed)
    B, Hq = s.wl.B, s.wl.Hq
    pairs = {(b, int(h)) for b in range(B) for h in r.choice(Hq, min(per_seq, Hq), replace=False)}
    longest = int(np.argmax(s.seq_lens.numpy()))
    pairs |= {(longest, 0), (longest, Hq - 1)}
    return sorted(pairs)


# workload -> None (every (sequence, head) pair) or heads per sequence
FULL = {"gqa_mid_ctx": (2, None), "large_batch": (4, None), "ragged_G4": (5, 4)}


@pytest.mark.parametrize("name", list(FULL))
def test_bf16_workloads_full_size(name):
    """The bf16 workloads at full size in the default launch plan: every output
    row of the mid-context (256 rows) and large-batch (32768 rows) workloads,
    and 4 query heads of each of the 64 ragged sequences (258 rows)."""
    idx, per_seq = FULL[name]
    s = make_inputs(WORKLOADS[idx], 0)
    pairs = None if per_seq is None else heads_of_every_sequence(s, per_seq)
    if pairs is not None:
        assert {b for b, _ in pairs} == set(range(s.wl.B)) and len(pairs) >= 256
    _run_full_check(s, f"{name} full", pairs=pairs, wr_zero_too=False)


# ------------------------------------------------------------------ edge cases
EDGE_LENS = [0, 1, 15, 16, 17, 127, 128, 129, 300]


@pytest.mark.parametrize("d,Hq,Hkv,dtype", [(128, 4, 2, "bf16"), (64, 6, 2, "bf16"),
                                            (128, 16, 2, "bf16"), (64, 3, 3, "bf16"),
                                            (128, 32, 2, "bf16"), (64, 20, 4, "bf16"),
                                            (128, 12, 2, "bf16"), (128, 14, 2, "bf16"),
                                            (64, 8, 1, "bf16"), (128, 24, 3, "bf16"),
                                            (128, 4, 2, "f32"), (64, 2, 1, "f32")])
def test_edge_lengths(d, Hq, Hkv, dtype):
    """Lengths 0, 1, tile and chunk boundaries, max; G in {1, 2, 3, 5, 6, 7, 8,
    16} (head blocks of 1 to 8 query heads: the whole group up to 8, two blocks
    of 8 at G = 16). bf16 runs on the default plan (one split at this cache
    size) and with 128-key chunks (three splits + merge)."""
    wl = WORKLOADS[2].scaled(B=len(EDGE_LENS), Hq=Hq, Hkv=Hkv, d=d, ctx=300, d_model=256,
                             dtype=dtype, wr_std=0.05)
    s = make_inputs(wl, 3, lengths=EDGE_LENS)
    tag = f"edge d={d} Hq={Hq} Hkv={Hkv} {dtype}"
    if dtype == "bf16":
        _run_full_check(s, tag)
        with pb.options(chunk=128):
            _run_full_check(s, tag + " chunk=128", wr_zero_too=False)
        # First tiles requested before the lengths arrive (rows past a length
        # fetched from the NaN padding and zeroed) or after: equal bit for bit.
        dev = Device(s)
        rho = dev.probe()
        outs = []
        for chunk in (0, 128):
            for pf in (1, 2):
                with pb.options(chunk=chunk, prefetch=pf):
                    outs.append(to64(dev.decode(rho, out_dtype=torch.float32)))
        torch.cuda.synchronize()
        for k in (0, 2):
            assert np.isfinite(outs[k + 1]).all()
            np.testing.assert_array_equal(outs[k], outs[k + 1])
        return
    say(f"[case] {tag}")
    dev = Device(s)
    rho = dev.probe()
    out = dev.decode(rho)
    torch.cuda.synchronize()
    ref = oracle_out(s, oracle_rho(s))
    o = to64(out)
    say(f"{tag}: rel {rel_l2(o, ref):.3e} max_abs {max_abs(o, ref):.3e}")
    assert rel_l2(o, ref) <= F32_TOL and max_abs(o, ref) <= F32_TOL
    assert np.all(o[0] == 0.0)


@pytest.mark.parametrize("chunk", [0, 64])
def test_zero_length_gives_zero_and_clamps_long_lengths(chunk):
    """Length 0 and a negative length give a zero output; a length above
    max_ctx counts as max_ctx (one split, and four splits with the merge)."""
    wl = WORKLOADS[2].scaled(B=4, ctx=200, d_model=64, Hq=4, Hkv=2)
    s = make_inputs(wl, 5, lengths=[0, 200, 200, 200])
    say(f"[case] zero length / clamp chunk={chunk}")
    dev = Device(s)
    # sequence 2 is a copy of sequence 1 whose length 1000 exceeds max_ctx = 200
    for t in (dev.K, dev.V, dev.q, dev.x):
        t[2].copy_(t[1])
    dev.seq_lens = torch.tensor([0, 200, 1000, -7], dtype=torch.int32, device="cuda")
    rho = dev.probe()
    with pb.options(chunk=chunk):
        out = to64(dev.decode(rho, out_dtype=torch.float32))
    torch.cuda.synchronize()
    assert np.all(out[0] == 0.0) and np.all(out[3] == 0.0)
    np.testing.assert_array_equal(out[1], out[2])   # same data, length clamped to 200


@pytest.mark.parametrize("chunk", [64, 128, 256, 1024, 2048])
@pytest.mark.parametrize("kernel,items", [(1, 0), (2, 1), (2, 2)])
def test_split_and_kernel_invariance(chunk, kernel, items):
    wl = WORKLOADS[5].scaled(B=4, ctx=5000, d_model=256)
    s = make_inputs(wl, 2, lengths=[5000, 4097, 129, 2048])
    say(f"[case] chunk={chunk} kernel={kernel} items={items}")
    dev = Device(s)
    rho = dev.probe()
    ref = oracle_out(s, oracle_rho(s))
    with pb.options(chunk=chunk, kernel=kernel, items=items):
        o32 = to64(dev.decode(rho, out_dtype=torch.float32))
    torch.cuda.synchronize()
    say(f"chunk={chunk} kernel={kernel}: rel {rel_l2(o32, ref):.3e} max_abs {max_abs(o32, ref):.3e}")
    assert rel_l2(o32, ref) <= 1e-5 and max_abs(o32, ref) <= 1e-4


@pytest.mark.parametrize("B,Hq", [(70, 8), (130, 8), (256, 8), (257, 8), (130, 16)])
def test_compacted_item_order_matches_split_major(B, Hq):
    """Numbering only the non-empty work items (a ragged batch in a cache of
    many chunks; sequences in two to four groups of 64) computes the same
    items as the split-major numbering of every item: equal bit for bit, and
    right against the oracle when the workspace still holds another input's
    partial states (an item left out would leave one of those behind). At
    B = 257 the compacted numbering does not apply and the option falls back
    to split-major. Hq = 16 over 2 KV heads runs head blocks of 8 (eight-wave
    workgroup items)."""
    wl = WORKLOADS[5].scaled(B=B, Hq=Hq, Hkv=2, ctx=2000, d_model=256)
    r = np.random.default_rng(B)
    lens = [0, 1, 255, 256, 257, 2000] + [int(x) for x in r.integers(0, 2001, B - 6)]
    s = make_inputs(wl, 21, lengths=lens)
    other = make_inputs(wl, 22, lengths=[2000] * B)
    say(f"[case] compacted order B={B} Hq={Hq} chunk=256")
    dev, dev2 = Device(s), Device(other)
    rho, rho2 = dev.probe(), dev2.probe()
    with pb.options(chunk=256, order=1, items=1, prefetch=1):
        plain = to64(dev.decode(rho, out_dtype=torch.float32))
    with pb.options(chunk=256, order=1, items=1, prefetch=2):
        # empty splits among the items, each with its first tiles in flight
        plain_pf = to64(dev.decode(rho, out_dtype=torch.float32))
    with pb.options(chunk=256, order=2, items=1):
        dev2.decode(rho2, out_dtype=torch.float32)
        comp = to64(dev.decode(rho, out_dtype=torch.float32))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(plain_pf, plain)
    np.testing.assert_array_equal(comp, plain)
    pairs = sample_pairs(s, 24) + [(0, 0), (1, 3), (5, 7), (B - 1, 7)]
    ref = oracle_out(s, oracle_rho(s), pairs)
    got = np.stack([comp[b, h] for b, h in pairs])
    say(f"compacted B={B}: rel {rel_l2(got, ref):.3e} max_abs {max_abs(got, ref):.3e}")
    assert rel_l2(got, ref) <= 1e-5 and max_abs(got, ref) <= 1e-4


def test_gqa_equals_replicated_mha():
    wl = WORKLOADS[2].scaled(B=2, ctx=700, d_model=128)
    s = make_inputs(wl, 4, lengths=[700, 333])
    say("[case] GQA vs replicated MHA")
    dev = Device(s)
    rho = dev.probe()
    gqa = to64(dev.decode(rho, out_dtype=torch.float32))
    G = wl.Hq // wl.Hkv
    Kr = dev.K.repeat_interleave(G, dim=1).contiguous()
    Vr = dev.V.repeat_interleave(G, dim=1).contiguous()
    mha = to64(pb.decode(dev.q, rho, Kr, Vr, dev.seq_lens, out_dtype=torch.float32))
    torch.cuda.synchronize()
    assert rel_l2(gqa, mha) <= 1e-6 and max_abs(gqa, mha) <= 1e-5


def test_bitwise_repeatable_and_output_guards():
    wl = WORKLOADS[2].scaled(B=4, ctx=3000, d_model=512)
    s = make_inputs(wl, 6, lengths=[3000, 2999, 1, 640])
    say("[case] repeatability / guards")
    dev = Device(s)
    rho = dev.probe()
    n = wl.B * wl.Hq * wl.d
    guard = 64
    buf = torch.full((n + 2 * guard,), 12345.0, dtype=torch.bfloat16, device="cuda")
    out = buf[guard:guard + n].view(wl.B, wl.Hq, wl.d)
    pb.decode(dev.q, rho, dev.K, dev.V, dev.seq_lens, out=out)
    first = out.clone()
    pb.decode(dev.q, rho, dev.K, dev.V, dev.seq_lens, out=out)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), out.view(torch.int16))
    assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[guard + n:] == 12345.0)


@pytest.mark.parametrize("Hq,Hkv,dtype,kernel,items", [(16, 8, "bf16", 0, 0), (32, 8, "bf16", 0, 0),
                                                      (16, 8, "bf16", 0, 2), (32, 8, "bf16", 2, 1),
                                                      (12, 4, "bf16", 0, 0), (64, 8, "bf16", 0, 0),
                                                      (64, 8, "bf16", 2, 2), (14, 2, "bf16", 0, 0),
                                                      (4, 2, "f32", 0, 0)])
def test_softmax_only_variant(Hq, Hkv, dtype, kernel, items):
    """parallax_softmax_decode: plain softmax attention over the same cache (the
    W_R = 0 reduction) against the oracle with rho = 0 and torch SDPA (fp64)."""
    wl = WORKLOADS[2].scaled(B=4, Hq=Hq, Hkv=Hkv, ctx=3000, d_model=64, dtype=dtype)
    s = make_inputs(wl, 8, lengths=[3000, 1, 0, 1777])
    say(f"[case] softmax-only Hq={Hq} Hkv={Hkv} {dtype} kernel={kernel} items={items}")
    dev = Device(s)
    with pb.options(kernel=kernel, items=items):
        o = to64(pb.softmax_decode(dev.q, dev.K, dev.V, dev.seq_lens, out_dtype=torch.float32))
    torch.cuda.synchronize()
    ref = oracle_out(s, np.zeros((wl.B, wl.Hq, wl.d)))
    G = Hq // Hkv
    for b, n in enumerate(s.seq_lens.tolist()):
        if n == 0:
            continue
        qt = s.q[b].double()[:, None, :]
        kt = s.K[b].double().repeat_interleave(G, dim=0)
        vt = s.V[b].double().repeat_interleave(G, dim=0)
        sdpa = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0].numpy()
        np.testing.assert_allclose(ref[b], sdpa, rtol=0, atol=1e-12)
    tol = 1e-5 if dtype == "f32" else 2e-6
    say(f"softmax-only: rel {rel_l2(o, ref):.3e} max_abs {max_abs(o, ref):.3e}")
    assert rel_l2(o, ref) <= tol and max_abs(o, ref) <= 1e-4
    assert np.all(o[2] == 0.0)


def test_workspace_grows_across_shapes_and_streams():
    """The per-stream split-K workspace grows when a larger shape arrives and
    stays right for every shape after that (smaller shapes after larger ones,
    a second stream with its own workspace, repeated calls)."""
    cases = [(2, 900, [900, 700]), (5, 4000, [4000, 3999, 2500, 1, 130]), (3, 1500, [1500, 20, 1499])]
    side = torch.cuda.Stream()
    for rep in range(2):
        for B, ctx, lens in cases:
            wl = WORKLOADS[2].scaled(B=B, ctx=ctx, d_model=64)
            s = make_inputs(wl, 10 + B, lengths=lens)
            say(f"[case] workspace B={B} ctx={ctx} rep={rep}")
            dev = Device(s)
            rho = dev.probe()
            torch.cuda.synchronize()   # inputs ready before the side stream reads them
            ref = oracle_out(s, oracle_rho(s))
            for st in (torch.cuda.current_stream(), side):
                with torch.cuda.stream(st):
                    o = dev.decode(rho, out_dtype=torch.float32)
                st.synchronize()
                assert rel_l2(to64(o), ref) <= 1e-5


@pytest.mark.parametrize("B,d_model,dtype,Hq,d", [
    (1, 2048, "bf16", 16, 128), (17, 2560, "bf16", 16, 128), (64, 2048, "bf16", 16, 128),
    (65, 512, "bf16", 16, 128), (130, 72, "bf16", 16, 128), (3, 100, "f32", 16, 128),
    (2048, 2048, "bf16", 16, 128), (300, 520, "bf16", 3, 64), (129, 4096, "bf16", 5, 128),
    (40, 2048, "bf16", 16, 128), (48, 1024, "bf16", 32, 128), (33, 264, "bf16", 5, 64),
    (128, 2560, "bf16", 32, 128), (97, 264, "bf16", 6, 64), (64, 2048, "bf16", 64, 128),
    (120, 520, "bf16", 66, 64), (70, 3072, "bf16", 4, 128), (200, 1024, "bf16", 3, 64),
    (257, 2560, "bf16", 7, 128)])
def test_probe_shapes(B, d_model, dtype, Hq, d):
    """Automatic kernel choice, then (bf16) each of the two probe kernels forced:
    the small-batch kernel in row blocks and the tiled GEMM, at every batch."""
    wl = WORKLOADS[2].scaled(B=B, d_model=d_model, ctx=16, dtype=dtype, Hq=Hq, Hkv=1, d=d)
    s = make_inputs(wl, 7)
    W, x = s.W_R.cuda(), s.x.cuda()
    want = oracle_rho(s)
    for path in ((0, 1, 2) if dtype == "bf16" else (0,)):
        say(f"[case] probe B={B} d_model={d_model} Hq={Hq} d={d} {dtype} path={path}")
        with pb.options(probe=path):
            rho = pb.probe(W, x, wl.Hq, wl.d)
        torch.cuda.synchronize()
        e = rel_l2(to64(rho), want)
        say(f"probe B={B} d_model={d_model} path={path}: rel {e:.3e}")
        assert e <= RHO_REL_L2


def test_cache_past_4gib():
    """K and V of 5.2 GB each, so the streams of the later sequences start past
    byte 2^32: the ragged workload's shapes over a 40000-key cache (lengths
    log-uniform in [128, 40000], the last sequence full, K/V drawn on the
    device), through the automatic plan (split-K with the compacted item
    order) and the one-call step. Checked against the oracle on one query
    head of KV head 7 (the highest stream of its sequence) for every sequence
    from 40 on and two early ones, plus the first and last head of the
    longest sequence."""
    from parallax_covariance_corrected_amd.workloads import device_cache
    import oracle
    wl = WORKLOADS[5].scaled(ctx=40000)
    s = make_inputs(wl, 31, with_kv=False)
    lens = s.seq_lens.clone()
    lens[-1] = wl.ctx
    K, V = device_cache(wl, 32)
    per_seq = wl.Hkv * wl.ctx * wl.d * 2
    assert K.numel() * 2 > 2 ** 32 and (wl.B - 1) * per_seq > 2 ** 32
    say(f"[case] cache past 4 GiB: K, V {K.numel() * 2 / 2 ** 30:.2f} GiB each, "
        f"lengths {lens.min().item()}..{lens.max().item()}, plan {pb.decode_plan(wl.B, wl.Hq, wl.Hkv, wl.d, wl.ctx)}")
    G = wl.Hq // wl.Hkv
    longest = int(torch.argmax(lens))
    pairs = sorted({(b, 7 * G + b % G) for b in [0, 1] + list(range(40, wl.B))}
                   | {(longest, 0), (longest, wl.Hq - 1)})
    W, x, q, dl = s.W_R.cuda(), s.x.cuda(), s.q.cuda(), lens.cuda()
    rho = pb.probe(W, x, wl.Hq, wl.d)
    o32 = pb.decode(q, rho, K, V, dl, out_dtype=torch.float32)
    o16 = pb.decode(q, rho, K, V, dl)
    step = pb.probe_decode(W, x, q, K, V, dl)
    torch.cuda.synchronize()
    assert torch.equal(step.view(torch.int16), o16.view(torch.int16))
    # host copies of the K/V rows the sampled pairs read
    need = {}
    for b, h in pairs:
        need.setdefault(b, set()).add(h // G)
    Kp, Vp = {}, {}
    for b, gs in need.items():
        n = int(lens[b])
        Kp[b] = {g: K[b, g, :n].cpu() for g in gs}
        Vp[b] = {g: V[b, g, :n].cpu() for g in gs}
    q64 = s.q.float().numpy().astype(np.float64)
    ref = oracle.decode_heads(q64, oracle_rho(s), Kp, Vp, lens.tolist(), wl.Hkv, pairs)
    got32 = np.stack([to64(o32[b, h]) for b, h in pairs])
    got16 = np.stack([to64(o16[b, h]) for b, h in pairs])
    say(f"past 4 GiB: {len(pairs)} pairs, rel bf16 {rel_l2(got16, ref):.3e}, "
        f"max-abs fp32 out {max_abs(got32, ref):.3e}")
    assert np.isfinite(got32).all()
    assert rel_l2(got16, ref) <= BF16_REL_L2 and max_abs(got32, ref) <= F32OUT_MAX_ABS
    np.testing.assert_array_equal(got16, bf16_rne(got32))


@pytest.mark.parametrize("opts", [{}, {"chunk": 128}, {"kernel": 1}])
def test_zero_covariance_closed_forms(opts):
    """Degenerate covariance against closed forms, not the oracle: all keys of a
    sequence equal (equal scores, uniform weights, C = 0) gives the mean of its
    values; all values equal gives that value, whatever rho. The probe is made
    large (W_R ~ N(0, 1)), so the one-pass form's P/l - vbar S/l must cancel to
    within fp32 rounding of |p| |vbar|."""
    wl = WORKLOADS[2].scaled(B=3, Hq=8, Hkv=2, ctx=700, d_model=64, wr_std=1.0)
    s = make_inputs(wl, 41, lengths=[700, 513, 300])
    K0, V1 = s.K[0].clone(), s.V[1].clone()
    K0[:] = K0[:, :1, :]                # sequence 0: every key equal to its first
    V1[:] = V1[:, :1, :]                # sequence 1: every value equal to its first
    s.K[0], s.V[1] = K0, V1
    say(f"[case] zero covariance {opts}")
    dev = Device(s)
    rho = dev.probe()
    with pb.options(**opts):
        o32 = to64(dev.decode(rho, out_dtype=torch.float32))
        o16 = to64(dev.decode(rho))
    torch.cuda.synchronize()
    G = wl.Hq // wl.Hkv
    want0 = np.stack([s.V[0][h // G][:700].double().numpy().mean(0) for h in range(wl.Hq)])
    want1 = np.stack([s.V[1][h // G][0].double().numpy() for h in range(wl.Hq)])
    p_scale = float(np.abs(to64(rho)).sum(-1).max()) * float(np.abs(s.K[0][0][0].double().numpy()).max())
    err0, err1 = max_abs(o32[0], want0), max_abs(o32[1], want1)
    say(f"zero covariance {opts}: max-abs equal keys {err0:.2e}, equal values {err1:.2e}, |p| scale {p_scale:.1f}")
    assert err0 <= 1e-6 * max(p_scale, 1.0) + 1e-5 and err1 <= 1e-6 * max(p_scale, 1.0) + 1e-5
    np.testing.assert_array_equal(o16, bf16_rne(o32))
    # sequence 2 is untouched: ordinary parity
    ref2 = oracle_out(s, oracle_rho(s), [(2, h) for h in range(wl.Hq)])
    assert max_abs(o32[2], ref2) <= F32OUT_MAX_ABS
