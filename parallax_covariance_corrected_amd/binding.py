"""ctypes binding of libparallax.so: argument marshalling only.

Every computation runs in the HIP library; this module only turns torch
tensors into device pointers, sizes and the current HIP stream. If the library
is missing, every call raises — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libparallax.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "parallax.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_NO_MEMORY = 0, 1, 2, 3, 4
F32, BF16, BF16_F32OUT = 0, 1, 2
OPT_CHUNK, OPT_KERNEL, OPT_PROFILE, OPT_ITEMS, OPT_ORDER, OPT_FUSE, OPT_PREFETCH, OPT_PROBE = (
    1, 2, 3, 4, 5, 6, 7, 8)
KERNEL_PROBE, KERNEL_DECODE, KERNEL_MERGE, KERNEL_PREFILL, KERNEL_READ = 0, 1, 2, 3, 4

_lib = None


class ParallaxError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"parallax error {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libparallax.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m parallax_covariance_corrected_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.parallax_probe.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
        L.parallax_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
        L.parallax_softmax_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
        L.parallax_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
        L.parallax_softmax_prefill.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
        L.parallax_read_bandwidth.argtypes = [vp, ctypes.c_longlong, vp, vp]
        L.parallax_decode_plan.argtypes = [i, i, i, i, i, i, ctypes.POINTER(i),
                                           ctypes.POINTER(i), ctypes.POINTER(i)]
        L.parallax_probe_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
        L.parallax_probe_decode_plan.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(i)]
        L.parallax_probe_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp,
                                                    i, i, i, i, i, i, i, vp]
        L.parallax_noalloc_scratch_bytes.argtypes = []
        L.parallax_noalloc_scratch_bytes.restype = ctypes.c_longlong
        L.parallax_set_option.argtypes = [i, i]
        L.parallax_get_option.argtypes = [i, ctypes.POINTER(i)]
        L.parallax_profile_read.argtypes = [i, ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_longlong)]
        L.parallax_profile_reset.argtypes = []
        for name in ("parallax_probe", "parallax_decode", "parallax_softmax_decode",
                     "parallax_prefill", "parallax_softmax_prefill", "parallax_read_bandwidth",
                     "parallax_decode_plan", "parallax_probe_decode", "parallax_probe_decode_plan",
                     "parallax_probe_decode_noalloc",
                     "parallax_set_option", "parallax_get_option", "parallax_profile_read",
                     "parallax_profile_reset"):
            getattr(L, name).restype = i
        L.parallax_last_error.argtypes = []
        L.parallax_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/parallax.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|long long|const char\*)\s+(parallax_\w+)\s*\(",
                                 txt, re.M)))


def _check(rc: int):
    if rc != OK:
        raise ParallaxError(rc, lib().parallax_last_error().decode())


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _dtype_code(t: torch.dtype, out_dtype: torch.dtype) -> int:
    if t == torch.float32:
        if out_dtype != torch.float32:
            raise ValueError("fp32 inputs produce an fp32 output")
        return F32
    if t == torch.bfloat16:
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError(f"out must be bfloat16 or float32, got {out_dtype}")
        return BF16 if out_dtype == torch.bfloat16 else BF16_F32OUT
    raise ValueError(f"unsupported dtype {t}")


def _shape(t: torch.Tensor, name: str, shape, dtype=None):
    """Raise ValueError unless t has exactly this shape (and dtype)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _rank(t: torch.Tensor, name: str, n: int):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")


def _stream_of(tensors) -> int:
    """Check that every tensor is a contiguous tensor on one GPU and return the
    HIP stream handle of that GPU's current stream (the library launches on the
    calling thread's current device, so the call runs under that device)."""
    dev = None
    for t, name in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    if dev.index is not None and dev.index != torch.cuda.current_device():
        raise ValueError(f"the tensors are on {dev}; make it the current device "
                         "(torch.cuda.device) before the call")
    return torch.cuda.current_stream(dev).cuda_stream


def _out(out, shape, dtype, like: torch.Tensor) -> torch.Tensor:
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    return out


def probe(W_R: torch.Tensor, x: torch.Tensor, Hq: int, d: int,
          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """rho[B, Hq, d] (fp32) = x[B, d_model] . W_R[Hq*d, d_model]^T on the current stream."""
    _rank(x, "x", 2)
    B, d_model = x.shape
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"unsupported dtype {x.dtype}")
    _shape(W_R, "W_R", (Hq * d, d_model), x.dtype)
    if out is not None:
        _shape(out, "rho", (B, Hq, d), torch.float32)
    st = _stream_of([(W_R, "W_R"), (x, "x"), (out, "rho")])
    out = _out(out, (B, Hq, d), torch.float32, x)
    code = F32 if x.dtype == torch.float32 else BF16
    _check(lib().parallax_probe(_ptr(W_R), _ptr(x), _ptr(out), B, Hq, d, d_model, code, st))
    return out


def _decode_shapes(q, k_cache, v_cache, seq_lens, rho=None):
    """Sizes of a decode call from q [B, Hq, d] and k_cache [B, Hkv, max_ctx, d];
    every other tensor is checked against them."""
    _rank(q, "q", 3)
    _rank(k_cache, "k_cache", 4)
    B, Hq, d = q.shape
    Hkv, max_ctx = k_cache.shape[1], k_cache.shape[2]
    _shape(k_cache, "k_cache", (B, Hkv, max_ctx, d), q.dtype)
    _shape(v_cache, "v_cache", (B, Hkv, max_ctx, d), q.dtype)
    _shape(seq_lens, "seq_lens", (B,), torch.int32)
    if rho is not None:
        _shape(rho, "rho", (B, Hq, d), torch.float32)
    return B, Hq, Hkv, d, max_ctx


def decode(q: torch.Tensor, rho: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           seq_lens: torch.Tensor, out: Optional[torch.Tensor] = None,
           out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Parallax decode: out[B, Hq, d] from q[B, Hq, d], rho[B, Hq, d] (fp32),
    k_cache/v_cache[B, Hkv, max_ctx, d], seq_lens[B] (int32), on the current stream."""
    if rho is None:
        raise ValueError("rho is required (softmax_decode runs without the correction)")
    B, Hq, Hkv, d, max_ctx = _decode_shapes(q, k_cache, v_cache, seq_lens, rho)
    odt = out.dtype if out is not None else (out_dtype or q.dtype)
    code = _dtype_code(q.dtype, odt)
    if out is not None:
        _shape(out, "out", (B, Hq, d))
    st = _stream_of([(q, "q"), (rho, "rho"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                     (seq_lens, "seq_lens"), (out, "out")])
    out = _out(out, (B, Hq, d), odt, q)
    _check(lib().parallax_decode(_ptr(q), _ptr(rho), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(seq_lens), _ptr(out), B, Hq, Hkv, d, max_ctx, code, st))
    return out


def probe_decode(W_R: torch.Tensor, x: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                 v_cache: torch.Tensor, seq_lens: torch.Tensor,
                 out: Optional[torch.Tensor] = None,
                 out_dtype: Optional[torch.dtype] = None, noalloc: bool = False) -> torch.Tensor:
    """One whole decode step (probe rho = W_R x, then the Parallax decode):
    out[B, Hq, d] from W_R[Hq*d, d_model], x[B, d_model], q[B, Hq, d],
    k_cache/v_cache[B, Hkv, max_ctx, d] and seq_lens[B] (int32), on the
    current stream. noalloc=True calls parallax_probe_decode_noalloc (the
    library's static scratch array instead of its workspace; pass `out` too
    so that nothing is allocated on the Python side either)."""
    B, Hq, Hkv, d, max_ctx = _decode_shapes(q, k_cache, v_cache, seq_lens)
    _rank(x, "x", 2)
    d_model = x.shape[1]
    _shape(x, "x", (B, d_model), q.dtype)
    _shape(W_R, "W_R", (Hq * d, d_model), q.dtype)
    odt = out.dtype if out is not None else (out_dtype or q.dtype)
    code = _dtype_code(q.dtype, odt)
    if out is not None:
        _shape(out, "out", (B, Hq, d))
    st = _stream_of([(W_R, "W_R"), (x, "x"), (q, "q"), (k_cache, "k_cache"),
                     (v_cache, "v_cache"), (seq_lens, "seq_lens"), (out, "out")])
    out = _out(out, (B, Hq, d), odt, q)
    fn = lib().parallax_probe_decode_noalloc if noalloc else lib().parallax_probe_decode
    _check(fn(_ptr(W_R), _ptr(x), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(out),
              B, Hq, Hkv, d, d_model, max_ctx, code, st))
    return out


def softmax_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   seq_lens: torch.Tensor, out: Optional[torch.Tensor] = None,
                   out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Plain softmax attention decode (the same kernel without the correction
    branch): out[B, Hq, d] from q, k_cache/v_cache [B, Hkv, max_ctx, d], seq_lens."""
    B, Hq, Hkv, d, max_ctx = _decode_shapes(q, k_cache, v_cache, seq_lens)
    odt = out.dtype if out is not None else (out_dtype or q.dtype)
    code = _dtype_code(q.dtype, odt)
    if out is not None:
        _shape(out, "out", (B, Hq, d))
    st = _stream_of([(q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                     (seq_lens, "seq_lens"), (out, "out")])
    out = _out(out, (B, Hq, d), odt, q)
    _check(lib().parallax_softmax_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                         _ptr(out), B, Hq, Hkv, d, max_ctx, code, st))
    return out


def prefill(q: torch.Tensor, rho: Optional[torch.Tensor], k_cache: torch.Tensor,
            v_cache: torch.Tensor, prefix_lens: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None,
            out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Causal many-query forward: out[B, T, Hq, d] for q [B, T, Hq, d] (bf16),
    rho [B, T, Hq, d] (fp32) and a cache [B, Hkv, max_ctx, d] holding each
    sequence's prefix_lens[b] cached tokens followed by its T new ones.
    rho=None runs plain softmax attention (parallax_softmax_prefill)."""
    _rank(q, "q", 4)
    _rank(k_cache, "k_cache", 4)
    B, T, Hq, d = q.shape
    Hkv, max_ctx = k_cache.shape[1], k_cache.shape[2]
    _shape(k_cache, "k_cache", (B, Hkv, max_ctx, d), q.dtype)
    _shape(v_cache, "v_cache", (B, Hkv, max_ctx, d), q.dtype)
    if rho is not None:
        _shape(rho, "rho", (B, T, Hq, d), torch.float32)
    if prefix_lens is not None:
        _shape(prefix_lens, "prefix_lens", (B,), torch.int32)
    odt = out.dtype if out is not None else (out_dtype or q.dtype)
    code = _dtype_code(q.dtype, odt)
    if out is not None:
        _shape(out, "out", (B, T, Hq, d))
    st = _stream_of([(q, "q"), (rho, "rho"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                     (prefix_lens, "prefix_lens"), (out, "out")])
    out = _out(out, (B, T, Hq, d), odt, q)
    pp = _ptr(prefix_lens) if prefix_lens is not None else None
    if rho is None:
        _check(lib().parallax_softmax_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), pp, _ptr(out),
                                              B, T, Hq, Hkv, d, max_ctx, code, st))
    else:
        _check(lib().parallax_prefill(_ptr(q), _ptr(rho), _ptr(k_cache), _ptr(v_cache), pp,
                                      _ptr(out), B, T, Hq, Hkv, d, max_ctx, code, st))
    return out


def read_bandwidth(buf: torch.Tensor, sink: torch.Tensor):
    """Measurement hook: stream `buf` (contiguous, device, size a multiple of
    1 MiB) once with the decode's load shape; time it with options(profile=1)
    and profile_read(KERNEL_READ). sink: at least 4 bytes the kernel may write."""
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    st = _stream_of([(buf, "buf"), (sink, "sink")])
    nbytes = buf.numel() * buf.element_size()
    _check(lib().parallax_read_bandwidth(_ptr(buf), nbytes, _ptr(sink), st))


def decode_plan(B: int, Hq: int, Hkv: int, d: int, max_ctx: int, dtype: int = BF16):
    """(chunk, splits, kernel) the library would use for this shape."""
    c, s, k = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().parallax_decode_plan(B, Hq, Hkv, d, max_ctx, dtype, ctypes.byref(c),
                                      ctypes.byref(s), ctypes.byref(k)))
    return c.value, s.value, k.value


def probe_decode_plan(B: int, Hq: int, Hkv: int, d: int, d_model: int, max_ctx: int,
                      dtype: int = BF16) -> bool:
    """Whether probe_decode computes the probe inside the decode kernel for this shape."""
    f = ctypes.c_int()
    _check(lib().parallax_probe_decode_plan(B, Hq, Hkv, d, d_model, max_ctx, dtype,
                                            ctypes.byref(f)))
    return bool(f.value)


def noalloc_scratch_bytes() -> int:
    """Size of the static scratch array behind probe_decode(noalloc=True)."""
    return int(lib().parallax_noalloc_scratch_bytes())


def set_option(option: int, value: int):
    _check(lib().parallax_set_option(option, value))


def get_option(option: int) -> int:
    v = ctypes.c_int()
    _check(lib().parallax_get_option(option, ctypes.byref(v)))
    return v.value


def profile_read(kernel: int):
    """(total_ms, launches) recorded for a kernel since the last reset."""
    ms, n = ctypes.c_double(), ctypes.c_longlong()
    _check(lib().parallax_profile_read(kernel, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def profile_reset():
    _check(lib().parallax_profile_reset())


class options:
    """Context manager that sets library options and restores them on exit."""

    def __init__(self, **kw):
        self.kw = {{"chunk": OPT_CHUNK, "kernel": OPT_KERNEL, "profile": OPT_PROFILE,
                    "items": OPT_ITEMS, "order": OPT_ORDER, "fuse": OPT_FUSE,
                    "prefetch": OPT_PREFETCH, "probe": OPT_PROBE}[k]: v
                   for k, v in kw.items()}
        self.saved = {}

    def __enter__(self):
        for o, v in self.kw.items():
            self.saved[o] = get_option(o)
            set_option(o, v)
        return self

    def __exit__(self, *exc):
        for o, v in self.saved.items():
            set_option(o, v)
        return False
