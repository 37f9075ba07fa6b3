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
OPT_CHUNK, OPT_KERNEL, OPT_PROFILE, OPT_ITEMS, OPT_ORDER, OPT_FUSE = 1, 2, 3, 4, 5, 6
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
        L.parallax_set_option.argtypes = [i, i]
        L.parallax_get_option.argtypes = [i, ctypes.POINTER(i)]
        L.parallax_profile_read.argtypes = [i, ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_longlong)]
        L.parallax_profile_reset.argtypes = []
        for name in ("parallax_probe", "parallax_decode", "parallax_softmax_decode",
                     "parallax_prefill", "parallax_softmax_prefill", "parallax_read_bandwidth",
                     "parallax_decode_plan", "parallax_probe_decode", "parallax_probe_decode_plan",
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
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(parallax_\w+)\s*\(", txt, re.M)))


def _check(rc: int):
    if rc != OK:
        raise ParallaxError(rc, lib().parallax_last_error().decode())


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.dtype, out_dtype: torch.dtype) -> int:
    if t == torch.float32:
        if out_dtype != torch.float32:
            raise ValueError("fp32 inputs produce an fp32 output")
        return F32
    if t == torch.bfloat16:
        return BF16 if out_dtype == torch.bfloat16 else BF16_F32OUT
    raise ValueError(f"unsupported dtype {t}")


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def probe(W_R: torch.Tensor, x: torch.Tensor, Hq: int, d: int,
          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """rho[B, Hq, d] (fp32) = x[B, d_model] . W_R[Hq*d, d_model]^T on the current stream."""
    _need(W_R, "W_R"); _need(x, "x")
    B, d_model = x.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=x.device)
    _need(out, "rho")
    code = F32 if x.dtype == torch.float32 else BF16
    if W_R.dtype != x.dtype:
        raise ValueError("W_R and x must share a dtype")
    _check(lib().parallax_probe(_ptr(W_R), _ptr(x), _ptr(out), B, Hq, d, d_model, code, _stream()))
    return out


def decode(q: torch.Tensor, rho: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           seq_lens: torch.Tensor, out: Optional[torch.Tensor] = None,
           out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Parallax decode: out[B, Hq, d] from q[B, Hq, d], rho[B, Hq, d] (fp32),
    k_cache/v_cache[B, Hkv, max_ctx, d], seq_lens[B] (int32), on the current stream."""
    for t, nm in ((q, "q"), (rho, "rho"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                  (seq_lens, "seq_lens")):
        _need(t, nm)
    B, Hq, d = q.shape
    _, Hkv, max_ctx, _ = k_cache.shape
    if rho.dtype != torch.float32 or seq_lens.dtype != torch.int32:
        raise ValueError("rho must be fp32 and seq_lens int32")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, k_cache and v_cache must share a dtype")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    code = _dtype_code(q.dtype, out.dtype)
    _check(lib().parallax_decode(_ptr(q), _ptr(rho), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(seq_lens), _ptr(out), B, Hq, Hkv, d, max_ctx, code,
                                 _stream()))
    return out


def probe_decode(W_R: torch.Tensor, x: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                 v_cache: torch.Tensor, seq_lens: torch.Tensor,
                 out: Optional[torch.Tensor] = None,
                 out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """One whole decode step (probe rho = W_R x, then the Parallax decode):
    out[B, Hq, d] from W_R[Hq*d, d_model], x[B, d_model], q[B, Hq, d],
    k_cache/v_cache[B, Hkv, max_ctx, d] and seq_lens[B] (int32), on the
    current stream."""
    for t, nm in ((W_R, "W_R"), (x, "x"), (q, "q"), (k_cache, "k_cache"),
                  (v_cache, "v_cache"), (seq_lens, "seq_lens")):
        _need(t, nm)
    B, Hq, d = q.shape
    _, Hkv, max_ctx, _ = k_cache.shape
    d_model = x.shape[1]
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    if any(t.dtype != q.dtype for t in (W_R, x, k_cache, v_cache)):
        raise ValueError("W_R, x, q, k_cache and v_cache must share a dtype")
    if tuple(W_R.shape) != (Hq * d, d_model) or x.shape[0] != B:
        raise ValueError("W_R must be [Hq*d, d_model] and x [B, d_model]")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    code = _dtype_code(q.dtype, out.dtype)
    _check(lib().parallax_probe_decode(_ptr(W_R), _ptr(x), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(seq_lens), _ptr(out), B, Hq, Hkv, d, d_model, max_ctx,
                                       code, _stream()))
    return out


def softmax_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   seq_lens: torch.Tensor, out: Optional[torch.Tensor] = None,
                   out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Plain softmax attention decode (the same kernel without the correction
    branch): out[B, Hq, d] from q, k_cache/v_cache [B, Hkv, max_ctx, d], seq_lens."""
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens")):
        _need(t, nm)
    B, Hq, d = q.shape
    _, Hkv, max_ctx, _ = k_cache.shape
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, k_cache and v_cache must share a dtype")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    code = _dtype_code(q.dtype, out.dtype)
    _check(lib().parallax_softmax_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                         _ptr(out), B, Hq, Hkv, d, max_ctx, code, _stream()))
    return out


def prefill(q: torch.Tensor, rho: Optional[torch.Tensor], k_cache: torch.Tensor,
            v_cache: torch.Tensor, prefix_lens: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None,
            out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Causal many-query forward: out[B, T, Hq, d] for q [B, T, Hq, d] (bf16),
    rho [B, T, Hq, d] (fp32) and a cache [B, Hkv, max_ctx, d] holding each
    sequence's prefix_lens[b] cached tokens followed by its T new ones.
    rho=None runs plain softmax attention (parallax_softmax_prefill)."""
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm)
    B, T, Hq, d = q.shape
    _, Hkv, max_ctx, _ = k_cache.shape
    if rho is not None:
        _need(rho, "rho")
        if rho.dtype != torch.float32 or tuple(rho.shape) != (B, T, Hq, d):
            raise ValueError("rho must be float32 [B, T, Hq, d]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, k_cache and v_cache must share a dtype")
    pp = None
    if prefix_lens is not None:
        _need(prefix_lens, "prefix_lens")
        if prefix_lens.dtype != torch.int32:
            raise ValueError("prefix_lens must be int32")
        pp = _ptr(prefix_lens)
    if out is None:
        out = torch.empty((B, T, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out")
    code = _dtype_code(q.dtype, out.dtype)
    if rho is None:
        _check(lib().parallax_softmax_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), pp, _ptr(out),
                                              B, T, Hq, Hkv, d, max_ctx, code, _stream()))
    else:
        _check(lib().parallax_prefill(_ptr(q), _ptr(rho), _ptr(k_cache), _ptr(v_cache), pp,
                                      _ptr(out), B, T, Hq, Hkv, d, max_ctx, code, _stream()))
    return out


def read_bandwidth(buf: torch.Tensor, sink: torch.Tensor):
    """Measurement hook: stream `buf` (contiguous, device, size a multiple of
    1 MiB) once with the decode's load shape; time it with options(profile=1)
    and profile_read(KERNEL_READ)."""
    _need(buf, "buf")
    _need(sink, "sink")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().parallax_read_bandwidth(_ptr(buf), nbytes, _ptr(sink), _stream()))


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
                    "items": OPT_ITEMS, "order": OPT_ORDER, "fuse": OPT_FUSE}[k]: v
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
