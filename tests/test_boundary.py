"""C-ABI boundary on the CPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call
(so no GPU is needed). Also the host-side split planner."""
import ctypes

import pytest

from parallax_covariance_corrected_amd import binding as pb


@pytest.fixture(scope="module")
def L():
    return pb.lib()


def test_exports_every_declared_function(L):
    names = pb.header_functions()
    assert {"parallax_probe", "parallax_decode", "parallax_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def _decode(L, *, q=16, rho=16, k=16, v=16, lens=16, out=16, B=2, Hq=4, Hkv=2, d=128,
            max_ctx=64, dtype=pb.BF16):
    # fake, never-dereferenced addresses: validation rejects before any use
    return L.parallax_decode(q, rho, k, v, lens, out, B, Hq, Hkv, d, max_ctx, dtype, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(Hq=3, Hkv=2), pb.ERR_INVALID_ARG, "multiple"),
    (dict(d=96), pb.ERR_UNSUPPORTED, "64 or 128"),
    (dict(dtype=7), pb.ERR_UNSUPPORTED, "dtype"),
    (dict(B=0), pb.ERR_INVALID_ARG, ">= 1"),
    (dict(max_ctx=0), pb.ERR_INVALID_ARG, ">= 1"),
    (dict(Hkv=0), pb.ERR_INVALID_ARG, ">= 1"),
    (dict(q=0), pb.ERR_INVALID_ARG, "null"),
    (dict(lens=0), pb.ERR_INVALID_ARG, "null"),
    (dict(k=24), pb.ERR_INVALID_ARG, "aligned"),
    (dict(lens=18), pb.ERR_INVALID_ARG, "aligned"),
    (dict(max_ctx=1 << 24), pb.ERR_UNSUPPORTED, "max_ctx"),
    # the kernels receive Hq and Hkv packed into one 32-bit argument
    (dict(Hq=65536, Hkv=2), pb.ERR_UNSUPPORTED, "65535"),
])
def test_decode_rejects_bad_arguments(L, kw, code, msg):
    assert _decode(L, **kw) == code
    assert msg in L.parallax_last_error().decode()


@pytest.mark.parametrize("args,code", [
    ((16, 16, 16, 1, 2, 128, 64, 9), pb.ERR_UNSUPPORTED),     # dtype
    ((0, 16, 16, 1, 2, 128, 64, pb.BF16), pb.ERR_INVALID_ARG),  # null W_R
    ((16, 16, 16, 1, 2, 100, 64, pb.BF16), pb.ERR_UNSUPPORTED),  # d
    ((16, 16, 16, 1, 2, 128, 60, pb.BF16), pb.ERR_INVALID_ARG),  # d_model % 8
    ((16, 16, 16, 0, 2, 128, 64, pb.BF16), pb.ERR_INVALID_ARG),  # B
    ((16, 16, 8, 1, 2, 128, 64, pb.BF16), pb.ERR_INVALID_ARG),   # misaligned rho
])
def test_probe_rejects_bad_arguments(L, args, code):
    assert L.parallax_probe(*args, None) == code
    assert L.parallax_last_error().decode()


def _probe_decode(L, *, W=16, x=16, q=16, k=16, v=16, lens=16, out=16, B=2, Hq=4, Hkv=2, d=128,
                  d_model=64, max_ctx=64, dtype=pb.BF16):
    return L.parallax_probe_decode(W, x, q, k, v, lens, out, B, Hq, Hkv, d, d_model, max_ctx,
                                   dtype, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(W=0), pb.ERR_INVALID_ARG, "null"),
    (dict(x=24), pb.ERR_INVALID_ARG, "aligned"),
    (dict(d_model=60), pb.ERR_INVALID_ARG, "multiple of 8"),
    (dict(d_model=0), pb.ERR_INVALID_ARG, ">= 1"),
    (dict(Hq=3, Hkv=2), pb.ERR_INVALID_ARG, "multiple"),
    (dict(d=96), pb.ERR_UNSUPPORTED, "64 or 128"),
    (dict(dtype=7), pb.ERR_UNSUPPORTED, "dtype"),
    (dict(q=0), pb.ERR_INVALID_ARG, "null"),
    (dict(lens=18), pb.ERR_INVALID_ARG, "aligned"),
    (dict(max_ctx=1 << 24), pb.ERR_UNSUPPORTED, "max_ctx"),
])
def test_probe_decode_rejects_bad_arguments(L, kw, code, msg):
    assert _probe_decode(L, **kw) == code
    assert msg in L.parallax_last_error().decode()


def test_probe_decode_plan():
    # the tiny fp32 workload: W_R is 32 KB per work item, the probe runs inside the decode
    assert pb.probe_decode_plan(1, 2, 2, 64, 128, 128, pb.F32)
    # the bf16 workloads (d_model 2048 / 2560): a separate probe launch
    for shape in [(16, 16, 8, 128, 2048, 4096), (1, 16, 8, 128, 2048, 32768),
                  (2048, 16, 8, 128, 2048, 128), (64, 32, 8, 128, 2560, 32768)]:
        assert not pb.probe_decode_plan(*shape, pb.BF16)
    # small d_model and few items: fused (32 KiB per item up to 16 MiB in all,
    # 64 KiB up to 8 MiB, 128 KiB up to 4 MiB); more: separate
    assert pb.probe_decode_plan(4, 16, 8, 128, 64, 1024, pb.BF16)          # 32 KiB x 256
    assert pb.probe_decode_plan(64, 16, 8, 128, 64, 128, pb.BF16)          # 32 KiB x 512
    assert pb.probe_decode_plan(1, 16, 8, 128, 128, 128, pb.BF16)          # 64 KiB x 8
    assert pb.probe_decode_plan(16, 16, 8, 128, 128, 128, pb.BF16)         # 64 KiB x 128
    assert not pb.probe_decode_plan(4, 16, 8, 128, 128, 4096, pb.BF16)     # 64 KiB x 256
    assert pb.probe_decode_plan(4, 16, 8, 128, 256, 128, pb.BF16)          # 128 KiB x 32
    assert not pb.probe_decode_plan(1, 16, 8, 128, 256, 1024, pb.BF16)     # 128 KiB x 64
    assert not pb.probe_decode_plan(64, 16, 8, 128, 64, 4096, pb.BF16)     # 32 KiB x 1024
    assert not pb.probe_decode_plan(1, 16, 8, 128, 512, 128, pb.BF16)      # 256 KiB
    assert not pb.probe_decode_plan(256, 16, 8, 128, 64, 1024, pb.BF16)
    # the generic kernel (fp32): up to 128 KiB per item, 8 MiB in all
    assert pb.probe_decode_plan(4, 2, 2, 64, 512, 1024, pb.F32)            # 128 KiB x 64
    assert not pb.probe_decode_plan(4, 2, 2, 64, 1024, 128, pb.F32)
    # fp32 rows of d_model elements must be whole 16-byte pieces
    assert not pb.probe_decode_plan(1, 2, 2, 64, 130, 128, pb.F32)
    with pb.options(fuse=1):
        assert not pb.probe_decode_plan(1, 2, 2, 64, 128, 128, pb.F32)
    with pb.options(fuse=2):
        assert pb.probe_decode_plan(16, 16, 8, 128, 2048, 4096, pb.BF16)
        assert pb.get_option(pb.OPT_FUSE) == 2
        # one wave per item (many short sequences) and the compacted numbering
        # (ragged batch in a large cache) keep the separate probe
        assert pb.decode_plan(2048, 16, 8, 128, 128)[2] == 3
        assert not pb.probe_decode_plan(2048, 16, 8, 128, 2048, 128, pb.BF16)
        assert not pb.probe_decode_plan(64, 32, 8, 128, 2560, 32768, pb.BF16)
    assert pb.get_option(pb.OPT_FUSE) == 0
    assert pb.lib().parallax_set_option(pb.OPT_FUSE, 3) == pb.ERR_INVALID_ARG


def _prefill(L, *, q=16, rho=16, k=16, v=16, pre=16, out=16, B=2, T=8, Hq=4, Hkv=2, d=128,
             max_ctx=64, dtype=pb.BF16):
    return L.parallax_prefill(q, rho, k, v, pre, out, B, T, Hq, Hkv, d, max_ctx, dtype, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dtype=9), pb.ERR_UNSUPPORTED, "dtype"),
    (dict(T=0), pb.ERR_INVALID_ARG, "T must"),
    (dict(T=65), pb.ERR_INVALID_ARG, "T must"),
    (dict(Hq=3, Hkv=2), pb.ERR_INVALID_ARG, "multiple"),
    (dict(d=32), pb.ERR_UNSUPPORTED, "64 or 128"),
    (dict(rho=0), pb.ERR_INVALID_ARG, "null"),
    (dict(out=0), pb.ERR_INVALID_ARG, "null"),
    (dict(q=24), pb.ERR_INVALID_ARG, "aligned"),
    (dict(pre=18), pb.ERR_INVALID_ARG, "aligned"),
    (dict(B=70000), pb.ERR_UNSUPPORTED, "range"),
    (dict(Hq=65536, Hkv=1), pb.ERR_UNSUPPORTED, "65535"),
])
def test_prefill_rejects_bad_arguments(L, kw, code, msg):
    assert _prefill(L, **kw) == code
    assert msg in L.parallax_last_error().decode()


def test_read_bandwidth_rejects_bad_arguments(L):
    assert L.parallax_read_bandwidth(0, 1 << 20, 16, None) == pb.ERR_INVALID_ARG
    assert L.parallax_read_bandwidth(24, 1 << 20, 16, None) == pb.ERR_INVALID_ARG
    assert L.parallax_read_bandwidth(16, (1 << 20) + 4096, 16, None) == pb.ERR_INVALID_ARG
    assert L.parallax_read_bandwidth(16, 0, 16, None) == pb.ERR_INVALID_ARG
    assert "1 MiB" in L.parallax_last_error().decode()


def test_softmax_decode_rejects_bad_arguments(L):
    assert L.parallax_softmax_decode(16, 16, 16, 16, 16, 2, 3, 2, 128, 64, pb.BF16, None) == pb.ERR_INVALID_ARG
    assert L.parallax_softmax_decode(0, 16, 16, 16, 16, 2, 4, 2, 128, 64, pb.BF16, None) == pb.ERR_INVALID_ARG
    assert L.parallax_softmax_decode(16, 16, 16, 16, 16, 2, 4, 2, 96, 64, pb.BF16, None) == pb.ERR_UNSUPPORTED
    # the Parallax entry point requires rho
    assert L.parallax_decode(16, 0, 16, 16, 16, 16, 2, 4, 2, 128, 64, pb.BF16, None) == pb.ERR_INVALID_ARG
    assert "rho" in L.parallax_last_error().decode()


def test_options_and_profile_on_host(L):
    assert L.parallax_set_option(pb.OPT_CHUNK, 100) == pb.ERR_INVALID_ARG
    assert L.parallax_set_option(pb.OPT_ITEMS, 3) == pb.ERR_INVALID_ARG
    assert L.parallax_set_option(99, 0) == pb.ERR_INVALID_ARG
    assert L.parallax_set_option(pb.OPT_ORDER, 3) == pb.ERR_INVALID_ARG
    assert L.parallax_set_option(pb.OPT_PROBE, 3) == pb.ERR_INVALID_ARG
    assert L.parallax_set_option(pb.OPT_PROBE, -1) == pb.ERR_INVALID_ARG
    with pb.options(probe=2):
        assert pb.get_option(pb.OPT_PROBE) == 2
    assert pb.get_option(pb.OPT_PROBE) == 0
    with pb.options(chunk=512, kernel=1):
        assert pb.get_option(pb.OPT_CHUNK) == 512 and pb.get_option(pb.OPT_KERNEL) == 1
        assert pb.decode_plan(16, 16, 8, 128, 4096) == (512, 8, 1)
    with pb.options(items=2, chunk=256):
        assert pb.decode_plan(16, 16, 8, 128, 4096) == (256, 16, 3)
    with pb.options(order=2):
        assert pb.get_option(pb.OPT_ORDER) == 2
    assert pb.get_option(pb.OPT_CHUNK) == 0 and pb.get_option(pb.OPT_KERNEL) == 0
    assert pb.get_option(pb.OPT_ORDER) == 0
    pb.profile_reset()
    assert pb.profile_read(pb.KERNEL_DECODE) == (0.0, 0)
    with pytest.raises(pb.ParallaxError):
        pb.profile_read(5)


def test_plan_covers_context_and_picks_kernels():
    # (B, Hq, Hkv, d, max_ctx, dtype)
    for shape in [(16, 16, 8, 128, 4096, pb.BF16), (1, 16, 8, 128, 32768, pb.BF16),
                  (2048, 16, 8, 128, 128, pb.BF16), (64, 32, 8, 128, 32768, pb.BF16),
                  (1, 2, 2, 64, 128, pb.F32), (3, 4, 4, 64, 1000, pb.BF16_F32OUT)]:
        chunk, splits, kernel = pb.decode_plan(*shape)
        max_ctx = shape[4]
        assert chunk % 64 == 0 and 64 <= chunk <= 2048
        assert (splits - 1) * chunk < max_ctx <= splits * chunk
        assert kernel == 1 if shape[5] == pb.F32 else kernel in (2, 3)
    # many short sequences: one wave per item; long ones: four waves per item
    assert pb.decode_plan(2048, 16, 8, 128, 128)[2] == 3
    assert pb.decode_plan(16, 16, 8, 128, 4096)[2] == 2
    # about one workgroup per compute unit on the mid-context workload
    chunk, splits, _ = pb.decode_plan(16, 16, 8, 128, 4096)
    assert 16 * 8 * splits >= 256
    # short caches take one split (no merge launch)
    for B, ctx in ((1, 256), (8, 512), (2, 100)):
        assert pb.decode_plan(B, 16, 8, 128, ctx)[1] == 1


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(pb, "_lib", None)
    monkeypatch.setattr(pb, "LIB_PATH", str(tmp_path / "libparallax.so"))
    with pytest.raises(RuntimeError, match="not built"):
        pb.lib()


# ---------------------------------------------------------------- Python binding checks
# The C ABI sees only pointers, so the binding checks every tensor's shape,
# dtype and device against the sizes it passes; a mismatch raises ValueError
# before the library is touched (here: CPU tensors and a library that fails the
# test if it is called).
@pytest.fixture
def no_lib(monkeypatch):
    def _fail():
        raise AssertionError("the library was called")
    monkeypatch.setattr(pb, "lib", _fail)


def _dec_args(B=2, Hq=4, Hkv=2, d=64, ctx=32, dt=None):
    import torch
    dt = dt or torch.bfloat16
    return dict(q=torch.zeros(B, Hq, d, dtype=dt), rho=torch.zeros(B, Hq, d),
                k_cache=torch.zeros(B, Hkv, ctx, d, dtype=dt),
                v_cache=torch.zeros(B, Hkv, ctx, d, dtype=dt),
                seq_lens=torch.zeros(B, dtype=torch.int32))


def _bad_decode_cases():
    import torch
    return [
        ("rho", lambda a: a.update(rho=torch.zeros(2, 4, 32)), "rho must have shape"),
        ("rho", lambda a: a.update(rho=torch.zeros(2, 4, 64, dtype=torch.bfloat16)), "rho must be"),
        ("v_cache", lambda a: a.update(v_cache=torch.zeros(2, 2, 16, 64, dtype=torch.bfloat16)),
         "v_cache must have shape"),
        ("k_cache", lambda a: a.update(k_cache=torch.zeros(3, 2, 32, 64, dtype=torch.bfloat16),
                                       v_cache=torch.zeros(3, 2, 32, 64, dtype=torch.bfloat16)),
         "k_cache must have shape"),
        ("k_cache", lambda a: a.update(k_cache=torch.zeros(2, 2, 32, 128, dtype=torch.bfloat16)),
         "k_cache must have shape"),
        ("k_cache", lambda a: a.update(k_cache=torch.zeros(2, 2, 32, 64)), "k_cache must be"),
        ("seq_lens", lambda a: a.update(seq_lens=torch.zeros(3, dtype=torch.int32)),
         "seq_lens must have shape"),
        ("seq_lens", lambda a: a.update(seq_lens=torch.zeros(2, dtype=torch.int64)),
         "seq_lens must be"),
        ("out", lambda a: a.update(out=torch.zeros(2, 4, 32, dtype=torch.bfloat16)),
         "out must have shape"),
        ("out", lambda a: a.update(out=torch.zeros(2, 4, 64, dtype=torch.float16)),
         "out must be bfloat16 or float32"),
    ]


@pytest.mark.parametrize("i", range(10))
def test_binding_decode_rejects_mismatched_tensors(no_lib, i):
    name, mutate, msg = _bad_decode_cases()[i]
    a = _dec_args()
    mutate(a)
    with pytest.raises(ValueError, match=msg):
        pb.decode(**a)
    a.pop("rho")
    if name != "rho":
        with pytest.raises(ValueError, match=msg):
            pb.softmax_decode(**a)


def test_binding_rejects_before_the_library(no_lib):
    import torch
    a = _dec_args()
    with pytest.raises(ValueError, match="device tensor"):   # right shapes, host memory
        pb.decode(**a)
    with pytest.raises(ValueError, match="rho is required"):
        pb.decode(**{**a, "rho": None})
    f = _dec_args(dt=torch.float32)
    with pytest.raises(ValueError, match="fp32 inputs produce an fp32 output"):
        pb.decode(**f, out=torch.zeros(2, 4, 64, dtype=torch.bfloat16))
    # probe: a bf16 rho buffer would be written at 4 bytes per element
    W, x = torch.zeros(4 * 64, 128, dtype=torch.bfloat16), torch.zeros(2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="rho must be torch.float32"):
        pb.probe(W, x, 4, 64, out=torch.zeros(2, 4, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="rho must have shape"):
        pb.probe(W, x, 4, 64, out=torch.zeros(2, 4, 32))
    with pytest.raises(ValueError, match="W_R must have shape"):
        pb.probe(W[:, :64], x, 4, 64)
    with pytest.raises(ValueError, match="W_R must be"):
        pb.probe(W.float(), x, 4, 64)
    # probe_decode: x and W_R against q
    a.pop("rho")
    with pytest.raises(ValueError, match="x must have shape"):
        pb.probe_decode(W, torch.zeros(3, 128, dtype=torch.bfloat16), **a)
    with pytest.raises(ValueError, match="W_R must have shape"):
        pb.probe_decode(torch.zeros(4 * 32, 128, dtype=torch.bfloat16), x, **a)
    with pytest.raises(ValueError, match="seq_lens must have shape"):
        pb.probe_decode(W, x, **{**a, "seq_lens": torch.zeros(1, dtype=torch.int32)})
    # prefill: q [B, T, Hq, d]
    q = torch.zeros(2, 5, 4, 64, dtype=torch.bfloat16)
    K = torch.zeros(2, 2, 32, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="rho must have shape"):
        pb.prefill(q, torch.zeros(2, 4, 4, 64), K, K)
    with pytest.raises(ValueError, match="prefix_lens must have shape"):
        pb.prefill(q, None, K, K, prefix_lens=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="out must have shape"):
        pb.prefill(q, None, K, K, out=torch.zeros(2, 5, 4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="device tensor"):
        pb.prefill(q, None, K, K)
    with pytest.raises(ValueError, match="sink must hold"):
        pb.read_bandwidth(torch.zeros(1 << 20, dtype=torch.uint8), torch.zeros(0, dtype=torch.int32))


def test_noalloc_rejects_shapes_beyond_its_scratch_array(L):
    """parallax_probe_decode_noalloc refuses, on the host, a plan whose rho and
    split states exceed its static scratch array (B = 2048 at 8192 keys: four
    splits of 16 heads, 136 MB of states), and names the sizes."""
    args = (16, 16, 16, 16, 16, 16, 16)      # fake, never-dereferenced addresses
    rc = L.parallax_probe_decode_noalloc(*args, 2048, 16, 8, 128, 2048, 8192, pb.BF16, None)
    assert rc == pb.ERR_UNSUPPORTED
    msg = L.parallax_last_error().decode()
    assert "static scratch array" in msg and str(64 << 20) in msg
    assert L.parallax_noalloc_scratch_bytes() == 64 << 20
    # the same shape checks as parallax_probe_decode
    assert L.parallax_probe_decode_noalloc(*args, 2, 3, 2, 128, 64, 64, pb.BF16, None) == \
        pb.ERR_INVALID_ARG
