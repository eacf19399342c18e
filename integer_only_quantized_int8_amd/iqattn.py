"""Thin ctypes binding of libiqattn.so (argument marshalling only).

The four functions carry the C-ABI names and arguments of include/iqattn.h.
Tensors are torch int8 tensors on the HIP device; streams are
torch.cuda.Stream objects (HIP streams under ROCm) or None for the current
stream.  Every step of the attention runs in the library's kernels; if the
library is missing this module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libiqattn.so")

IQATTN_OK = 0
IQATTN_E_INVAL = -1
IQATTN_E_SHAPE = -2
IQATTN_E_ALLOC = -3
IQATTN_E_LAUNCH = -4
IQATTN_E_NULL = -5
IQATTN_E_ALIGN = -6
IQATTN_E_DEVICE = -7
IQATTN_E_INCOMPLETE = -8
IQATTN_E_TOOBIG = -9
IQATTN_SHIFTMAX = 0
IQATTN_LIS = 1
IQATTN_OUT_HEADS = 0
IQATTN_OUT_TOKENS = 1
IQATTN_LIS_VALU = 0
IQATTN_LIS_MFMA = 1
IQATTN_MAX_SEQ = 1024
IQLINEAR_PLAIN = 0
IQLINEAR_QKV_HEADS = 1

EXPORTED = ("iqattn_create", "iqattn_forward", "iqattn_destroy", "iqattn_strerror",
            "iqattn_check", "iqattn_set_spin_limit", "iqattn_forward_noalloc",
            "iqlinear_create", "iqlinear_forward", "iqlinear_destroy",
            "iqgelu_create", "iqgelu_forward", "iqgelu_destroy",
            "iqlayernorm_create", "iqlayernorm_forward", "iqlayernorm_destroy",
            "iqlinattn_create", "iqlinattn_forward", "iqlinattn_destroy")


class iqattn_params(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "batch", "heads", "seq_len", "head_dim", "qk_b", "qk_c", "pv_b", "pv_c", "i0",
        "exp_frac_bits", "intdiv_m", "k_out", "variant", "lis_bits", "lis_engine", "window",
        "out_layout")] + [("rel_bias", C.POINTER(C.c_int32))]


class iqlinear_params(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "rows", "in_features", "out_features", "layout", "batch", "seq_len", "heads",
        "head_dim")] + [("b", C.c_int32 * 3), ("c", C.c_int32 * 3)]


class iqgelu_params(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "rows", "cols", "i0", "exp_frac_bits", "intdiv_m", "k_out", "b", "c")]


class iqlayernorm_params(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "rows", "cols", "norm_frac_bits", "intdiv_m", "b", "c")]


class iqlinattn_params(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "batch", "heads", "seq_len", "head_dim", "kv_b", "kv_c", "ks_b", "ks_c", "out_b",
        "out_c")]


class IQAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {iqattn_strerror(code)} ({code})")


_lib = None


def load_library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with integer_only_quantized_int8_amd/build.py "
                "(hipcc --offload-arch=gfx950); there is no fallback path")
        lib = C.CDLL(LIB_PATH)
        lib.iqattn_create.argtypes = [C.POINTER(iqattn_params), C.POINTER(C.c_void_p)]
        lib.iqattn_create.restype = C.c_int
        lib.iqattn_forward.argtypes = [C.c_void_p] * 6
        lib.iqattn_forward.restype = C.c_int
        lib.iqattn_destroy.argtypes = [C.c_void_p]
        lib.iqattn_destroy.restype = C.c_int
        lib.iqattn_strerror.argtypes = [C.c_int]
        lib.iqattn_strerror.restype = C.c_char_p
        lib.iqattn_check.argtypes = [C.c_void_p, C.c_void_p]
        lib.iqattn_check.restype = C.c_int
        lib.iqattn_set_spin_limit.argtypes = [C.c_void_p, C.c_int32]
        lib.iqattn_set_spin_limit.restype = C.c_int
        lib.iqattn_forward_noalloc.argtypes = [C.POINTER(iqattn_params)] + [C.c_void_p] * 5
        lib.iqattn_forward_noalloc.restype = C.c_int
        lib.iqlinear_create.argtypes = [C.POINTER(iqlinear_params), C.POINTER(C.c_void_p)]
        lib.iqlinear_create.restype = C.c_int
        lib.iqlinear_forward.argtypes = [C.c_void_p] * 7
        lib.iqlinear_forward.restype = C.c_int
        lib.iqlinear_destroy.argtypes = [C.c_void_p]
        lib.iqlinear_destroy.restype = C.c_int
        lib.iqgelu_create.argtypes = [C.POINTER(iqgelu_params), C.POINTER(C.c_void_p)]
        lib.iqgelu_create.restype = C.c_int
        lib.iqgelu_forward.argtypes = [C.c_void_p] * 4
        lib.iqgelu_forward.restype = C.c_int
        lib.iqgelu_destroy.argtypes = [C.c_void_p]
        lib.iqgelu_destroy.restype = C.c_int
        lib.iqlayernorm_create.argtypes = [C.POINTER(iqlayernorm_params), C.POINTER(C.c_void_p)]
        lib.iqlayernorm_create.restype = C.c_int
        lib.iqlayernorm_forward.argtypes = [C.c_void_p] * 6
        lib.iqlayernorm_forward.restype = C.c_int
        lib.iqlayernorm_destroy.argtypes = [C.c_void_p]
        lib.iqlayernorm_destroy.restype = C.c_int
        lib.iqlinattn_create.argtypes = [C.POINTER(iqlinattn_params), C.POINTER(C.c_void_p)]
        lib.iqlinattn_create.restype = C.c_int
        lib.iqlinattn_forward.argtypes = [C.c_void_p] * 6
        lib.iqlinattn_forward.restype = C.c_int
        lib.iqlinattn_destroy.argtypes = [C.c_void_p]
        lib.iqlinattn_destroy.restype = C.c_int
        _lib = lib
    return _lib


def make_params(shape, params: Dict[str, object]):
    """Fill an iqattn_params from (B, H, N, d) and a parameter dict.  Returns the
    struct and the int32 array that backs rel_bias (keep it alive until create
    returns)."""
    B, H, N, d = shape
    p = iqattn_params()
    p.batch, p.heads, p.seq_len, p.head_dim = int(B), int(H), int(N), int(d)
    for name in ("qk_b", "qk_c", "pv_b", "pv_c", "i0", "exp_frac_bits", "intdiv_m", "k_out",
                 "variant", "lis_bits", "lis_engine", "window", "out_layout"):
        setattr(p, name, int(params.get(name, 0) or 0))
    keep = None
    rb = params.get("rel_bias")
    if rb is not None:
        keep = np.ascontiguousarray(np.asarray(rb, dtype=np.int32))
        p.rel_bias = keep.ctypes.data_as(C.POINTER(C.c_int32))
    return p, keep


def iqattn_strerror(code: int) -> str:
    return load_library().iqattn_strerror(int(code)).decode()


def iqattn_create(p: iqattn_params) -> int:
    """Returns the context handle (an integer address); raises IQAttnError."""
    ctx = C.c_void_p()
    rc = load_library().iqattn_create(C.byref(p), C.byref(ctx))
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqattn_create")
    return ctx.value


def _stream_handle(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def iqattn_forward(ctx: int, q, k, v, out, stream=None) -> None:
    """Enqueue the fused attention on `stream` (default: torch's current stream)."""
    rc = load_library().iqattn_forward(C.c_void_p(ctx), C.c_void_p(q.data_ptr()),
                                       C.c_void_p(k.data_ptr()), C.c_void_p(v.data_ptr()),
                                       C.c_void_p(out.data_ptr()),
                                       C.c_void_p(_stream_handle(stream)))
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqattn_forward")


def iqattn_destroy(ctx: Optional[int]) -> None:
    rc = load_library().iqattn_destroy(C.c_void_p(ctx) if ctx else None)
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqattn_destroy")


def iqattn_check(ctx: int, stream=None) -> int:
    """Synchronise `stream` and return the context's completion status
    (IQATTN_OK or IQATTN_E_INCOMPLETE); raises on other errors."""
    rc = load_library().iqattn_check(C.c_void_p(ctx), C.c_void_p(_stream_handle(stream)))
    if rc not in (IQATTN_OK, IQATTN_E_INCOMPLETE):
        raise IQAttnError(rc, "iqattn_check")
    return rc


def iqattn_forward_noalloc(shape, params: Dict[str, object], q, k, v, out, stream=None) -> None:
    """The attention of (shape, params) in one call that allocates nothing
    (static device memory of the library; calls that overlap on one GPU race)."""
    p, keep = make_params(shape, params)
    ptr = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    rc = load_library().iqattn_forward_noalloc(C.byref(p), ptr(q), ptr(k), ptr(v), ptr(out),
                                               C.c_void_p(_stream_handle(stream)))
    del keep
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqattn_forward_noalloc")


def iqattn_set_spin_limit(ctx: int, polls: int) -> None:
    rc = load_library().iqattn_set_spin_limit(C.c_void_p(ctx), int(polls))
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqattn_set_spin_limit")


class IQAttn:
    """Owns one context for a fixed shape and parameter set."""

    def __init__(self, shape, params: Dict[str, object]):
        self.shape = tuple(int(x) for x in shape)
        self.out_layout = int(params.get("out_layout", IQATTN_OUT_HEADS) or 0)
        B, H, N, d = self.shape
        self.out_shape = (B, N, H, d) if self.out_layout == IQATTN_OUT_TOKENS else self.shape
        p, keep = make_params(self.shape, params)
        self.ctx = iqattn_create(p)
        del keep

    def forward(self, q, k, v, out=None, stream=None):
        """out: [B, H, N, d], or [B, N, H, d] for out_layout IQATTN_OUT_TOKENS
        (any contiguous int8 device tensor of that many elements)."""
        import torch
        for name, t in (("q", q), ("k", k), ("v", v)):
            if t.dtype != torch.int8 or not t.is_cuda or not t.is_contiguous() \
                    or tuple(t.shape) != self.shape:
                raise ValueError(f"{name} must be a contiguous int8 device tensor of shape "
                                 f"{self.shape}")
        if out is None:
            out = torch.empty(self.out_shape, dtype=torch.int8, device=q.device)
        elif out.dtype != torch.int8 or not out.is_cuda or not out.is_contiguous() \
                or out.numel() != q.numel():
            raise ValueError(f"out must be a contiguous int8 device tensor of shape {self.out_shape}")
        iqattn_forward(self.ctx, q, k, v, out, stream)
        return out

    __call__ = forward

    def check(self, stream=None) -> int:
        """IQATTN_OK, or IQATTN_E_INCOMPLETE if a launch since the last check
        left output rows unwritten (synchronises the stream)."""
        return iqattn_check(self.ctx, stream)

    def close(self):
        if self.ctx:
            iqattn_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- linear layer
def make_linear_params(params: Dict[str, object]) -> iqlinear_params:
    """Fill an iqlinear_params from a dict (rows, in_features, out_features,
    layout, batch, seq_len, heads, head_dim, b, c; b and c are 1- or 3-tuples)."""
    p = iqlinear_params()
    for name in ("rows", "in_features", "out_features", "layout", "batch", "seq_len", "heads",
                 "head_dim"):
        setattr(p, name, int(params.get(name, 0) or 0))
    b = list(params["b"]) + [1] * 3
    c = list(params["c"]) + [0] * 3
    for i in range(3):
        p.b[i] = int(b[i])
        p.c[i] = int(c[i])
    return p


def iqlinear_create(p: iqlinear_params) -> int:
    ctx = C.c_void_p()
    rc = load_library().iqlinear_create(C.byref(p), C.byref(ctx))
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqlinear_create")
    return ctx.value


def iqlinear_forward(ctx: int, x, w, out0, out1=None, out2=None, stream=None) -> None:
    """Enqueue the int8 linear layer on `stream` (default: torch's current stream)."""
    ptr = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    rc = load_library().iqlinear_forward(C.c_void_p(ctx), ptr(x), ptr(w), ptr(out0), ptr(out1),
                                         ptr(out2), C.c_void_p(_stream_handle(stream)))
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqlinear_forward")


def iqlinear_destroy(ctx: Optional[int]) -> None:
    rc = load_library().iqlinear_destroy(C.c_void_p(ctx) if ctx else None)
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqlinear_destroy")


class IQLinear:
    """Owns one linear-layer context: x [rows, in] int8, w [out, in] int8."""

    def __init__(self, params: Dict[str, object]):
        self.params = dict(params)
        self.ctx = iqlinear_create(make_linear_params(self.params))

    def forward(self, x, w, outs=None, stream=None):
        import torch
        P = self.params
        rows, fin, fout = P["rows"], P["in_features"], P["out_features"]
        for name, t, shape in (("x", x, (rows, fin)), ("w", w, (fout, fin))):
            if t.dtype != torch.int8 or not t.is_cuda or not t.is_contiguous() \
                    or tuple(t.shape) != shape:
                raise ValueError(f"{name} must be a contiguous int8 device tensor of shape {shape}")
        if P["layout"] == IQLINEAR_QKV_HEADS:
            shape = (P["batch"], P["heads"], P["seq_len"], P["head_dim"])
            if outs is None:
                outs = tuple(torch.empty(shape, dtype=torch.int8, device=x.device) for _ in range(3))
            iqlinear_forward(self.ctx, x, w, outs[0], outs[1], outs[2], stream)
            return outs
        out = outs if outs is not None else torch.empty((rows, fout), dtype=torch.int8,
                                                        device=x.device)
        iqlinear_forward(self.ctx, x, w, out, None, None, stream)
        return out

    __call__ = forward

    def close(self):
        if self.ctx:
            iqlinear_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- ShiftGELU / I-LayerNorm
def _fill(struct_cls, fields, params: Dict[str, object]):
    p = struct_cls()
    for name in fields:
        setattr(p, name, int(params[name]))
    return p


def make_gelu_params(params: Dict[str, object]) -> iqgelu_params:
    return _fill(iqgelu_params, ("rows", "cols", "i0", "exp_frac_bits", "intdiv_m", "k_out",
                                 "b", "c"), params)


def make_layernorm_params(params: Dict[str, object]) -> iqlayernorm_params:
    return _fill(iqlayernorm_params, ("rows", "cols", "norm_frac_bits", "intdiv_m", "b", "c"),
                 params)


def _create(fn, p, where) -> int:
    ctx = C.c_void_p()
    rc = fn(C.byref(p), C.byref(ctx))
    if rc != IQATTN_OK:
        raise IQAttnError(rc, where)
    return ctx.value


def iqgelu_create(p: iqgelu_params) -> int:
    return _create(load_library().iqgelu_create, p, "iqgelu_create")


def iqgelu_forward(ctx: int, x, out, stream=None) -> None:
    ptr = lambda t: None if t is None else C.c_void_p(t.data_ptr())  # noqa: E731
    rc = load_library().iqgelu_forward(C.c_void_p(ctx), ptr(x), ptr(out),
                                       C.c_void_p(_stream_handle(stream)))
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqgelu_forward")


def iqgelu_destroy(ctx: Optional[int]) -> None:
    rc = load_library().iqgelu_destroy(C.c_void_p(ctx) if ctx else None)
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqgelu_destroy")


def iqlayernorm_create(p: iqlayernorm_params) -> int:
    return _create(load_library().iqlayernorm_create, p, "iqlayernorm_create")


def iqlayernorm_forward(ctx: int, x, gamma, beta, out, stream=None) -> None:
    ptr = lambda t: None if t is None else C.c_void_p(t.data_ptr())  # noqa: E731
    rc = load_library().iqlayernorm_forward(C.c_void_p(ctx), ptr(x), ptr(gamma), ptr(beta),
                                            ptr(out), C.c_void_p(_stream_handle(stream)))
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqlayernorm_forward")


def iqlayernorm_destroy(ctx: Optional[int]) -> None:
    rc = load_library().iqlayernorm_destroy(C.c_void_p(ctx) if ctx else None)
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqlayernorm_destroy")


def _check(name, t, dtype, shape):
    import torch
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shape:
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor of shape {shape}")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")
    del torch


class _Owner:
    _destroy = None

    def close(self):
        if self.ctx:
            type(self)._destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class IQGelu(_Owner):
    """Owns one ShiftGELU context: x [rows, cols] int8 -> int8."""
    _destroy = staticmethod(iqgelu_destroy)

    def __init__(self, params: Dict[str, object]):
        self.params = dict(params)
        self.ctx = iqgelu_create(make_gelu_params(self.params))

    def forward(self, x, out=None, stream=None):
        import torch
        shape = (self.params["rows"], self.params["cols"])
        _check("x", x, torch.int8, shape)
        out = out if out is not None else torch.empty(shape, dtype=torch.int8, device=x.device)
        _check("out", out, torch.int8, shape)
        iqgelu_forward(self.ctx, x, out, stream)
        return out

    __call__ = forward


class IQLayerNorm(_Owner):
    """Owns one I-LayerNorm context: x [rows, cols] int8, gamma [cols] int8,
    beta [cols] int32 -> int8."""
    _destroy = staticmethod(iqlayernorm_destroy)

    def __init__(self, params: Dict[str, object]):
        self.params = dict(params)
        self.ctx = iqlayernorm_create(make_layernorm_params(self.params))

    def forward(self, x, gamma, beta, out=None, stream=None):
        import torch
        rows, cols = self.params["rows"], self.params["cols"]
        _check("x", x, torch.int8, (rows, cols))
        _check("gamma", gamma, torch.int8, (cols,))
        _check("beta", beta, torch.int32, (cols,))
        out = out if out is not None else torch.empty((rows, cols), dtype=torch.int8,
                                                      device=x.device)
        _check("out", out, torch.int8, (rows, cols))
        iqlayernorm_forward(self.ctx, x, gamma, beta, out, stream)
        return out

    __call__ = forward


# ---------------------------------------------------------------- linear attention
def make_linattn_params(shape, params: Dict[str, object]) -> iqlinattn_params:
    B, H, N, d = shape
    return _fill(iqlinattn_params, ("batch", "heads", "seq_len", "head_dim", "kv_b", "kv_c",
                                    "ks_b", "ks_c", "out_b", "out_c"),
                 dict(params, batch=B, heads=H, seq_len=N, head_dim=d))


def iqlinattn_create(p: iqlinattn_params) -> int:
    return _create(load_library().iqlinattn_create, p, "iqlinattn_create")


def iqlinattn_forward(ctx: int, q, k, v, out, stream=None) -> None:
    ptr = lambda t: None if t is None else C.c_void_p(t.data_ptr())  # noqa: E731
    rc = load_library().iqlinattn_forward(C.c_void_p(ctx), ptr(q), ptr(k), ptr(v), ptr(out),
                                          C.c_void_p(_stream_handle(stream)))
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqlinattn_forward")


def iqlinattn_destroy(ctx: Optional[int]) -> None:
    rc = load_library().iqlinattn_destroy(C.c_void_p(ctx) if ctx else None)
    if rc != IQATTN_OK:
        raise IQAttnError(rc, "iqlinattn_destroy")


class IQLinAttn(_Owner):
    """Owns one softmax-free linear-attention context: Q, K, V [B, H, N, d] int8."""
    _destroy = staticmethod(iqlinattn_destroy)

    def __init__(self, shape, params: Dict[str, object]):
        self.shape = tuple(int(x) for x in shape)
        self.params = dict(params)
        self.ctx = iqlinattn_create(make_linattn_params(self.shape, self.params))

    def forward(self, q, k, v, out=None, stream=None):
        import torch
        for name, t in (("q", q), ("k", k), ("v", v)):
            _check(name, t, torch.int8, self.shape)
        out = out if out is not None else torch.empty(self.shape, dtype=torch.int8,
                                                      device=q.device)
        _check("out", out, torch.int8, self.shape)
        iqlinattn_forward(self.ctx, q, k, v, out, stream)
        return out

    __call__ = forward
