"""ctypes binding of the C oracle (iqattn_oracle.c).

TEST INFRASTRUCTURE ONLY.  Builds liboracle.so with plain gcc -O2 (no
intrinsics, no threads) and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iqattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def library_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle (single-threaded, -O2, C99)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        # the compiler's temporaries go to the repository's untracked _build/
        scratch = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(_SRC))), "_build")
        os.makedirs(scratch, exist_ok=True)
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC",
                               "-shared", "-o", tmp, _SRC], env=dict(os.environ, TMPDIR=scratch))
        os.replace(tmp, _LIB)
    return _LIB


class _Params(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "batch", "heads", "seq_len", "head_dim", "qk_b", "qk_c", "pv_b", "pv_c",
        "i0", "exp_frac_bits", "intdiv_m", "k_out", "variant", "lis_bits", "window")] + \
        [("rel_bias", C.POINTER(C.c_int32))]


class _Dump(C.Structure):
    _fields_ = [("acc", C.POINTER(C.c_int64)), ("logit", C.POINTER(C.c_int32)),
                ("expv", C.POINTER(C.c_int64)), ("rowsum", C.POINTER(C.c_int64)),
                ("prob", C.POINTER(C.c_int64)), ("code", C.POINTER(C.c_int32)),
                ("pv", C.POINTER(C.c_int64))]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = C.CDLL(_LIB)
        lib.orc_check_params.argtypes = [C.POINTER(_Params)]
        lib.orc_forward.argtypes = [C.POINTER(_Params), C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_int64, C.c_int64, C.POINTER(_Dump)]
        lib.orc_requant.argtypes = [C.c_int64, C.c_int32, C.c_int32]
        lib.orc_linear.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int64,
                                   C.c_int32, C.c_int32, C.c_void_p, C.c_int64, C.c_int64]
        lib.orc_linear.restype = C.c_int
        lib.orc_shiftgelu.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                                      C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                      C.c_int64, C.c_int64, C.c_void_p]
        lib.orc_shiftgelu.restype = C.c_int
        lib.orc_isqrt10.argtypes = [C.c_int64]
        lib.orc_isqrt10.restype = C.c_int64
        lib.orc_ilayernorm.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
                                       C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                       C.c_int64, C.c_int64, C.c_void_p]
        lib.orc_ilayernorm.restype = C.c_int
        lib.orc_linattn.argtypes = [C.c_void_p] * 5 + [C.c_int64, C.c_int64, C.c_void_p]
        lib.orc_linattn.restype = C.c_int
        lib.orc_requant.restype = C.c_int32
        lib.orc_requant_array.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_int32,
                                          C.c_void_p]
        lib.orc_shift_exp.argtypes = [C.c_int32, C.c_int32, C.c_int32]
        lib.orc_shift_exp.restype = C.c_int64
        lib.orc_ilog2r.argtypes = [C.c_int64]
        lib.orc_ilog2r.restype = C.c_int32
        lib.orc_softmax_row.argtypes = [C.POINTER(_Params), C.c_void_p, C.c_int32,
                                        C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        _lib = lib
    return _lib


def _make_params(shape, params: Dict[str, object]):
    B, H, N, d = shape
    p = _Params()
    p.batch, p.heads, p.seq_len, p.head_dim = B, H, N, d
    for name in ("qk_b", "qk_c", "pv_b", "pv_c", "i0", "exp_frac_bits", "intdiv_m",
                 "k_out", "variant", "lis_bits", "window"):
        setattr(p, name, int(params.get(name, 0) or 0))
    keep = None
    rb = params.get("rel_bias")
    if rb is not None:
        keep = np.ascontiguousarray(np.asarray(rb, dtype=np.int32))
        p.rel_bias = keep.ctypes.data_as(C.POINTER(C.c_int32))
    return p, keep


def check_params(shape, params) -> int:
    p, _keep = _make_params(shape, params)
    return _load().orc_check_params(C.byref(p))


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(C.POINTER(ctype))


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, params: Dict[str, object],
            heads: Optional[tuple] = None, dump: bool = False):
    """Run the oracle on int8 [B, H, N, d] tensors.

    heads = (begin, end) restricts the work to flattened heads [begin, end);
    the returned `out` is then shaped [end - begin, N, d].  With dump=True a
    dict of intermediates for those heads is returned as well.
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    k = np.ascontiguousarray(k, dtype=np.int8)
    v = np.ascontiguousarray(v, dtype=np.int8)
    B, H, N, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    p, keep = _make_params(q.shape, params)
    total = B * H
    h0, h1 = (0, total) if heads is None else heads
    out = np.zeros((B, H, N, d), dtype=np.int8)
    dumps = None
    dstruct = None
    if dump:
        nh = h1 - h0
        dumps = dict(acc=np.zeros((nh, N, N), np.int64), logit=np.zeros((nh, N, N), np.int32),
                     expv=np.zeros((nh, N, N), np.int64), rowsum=np.zeros((nh, N), np.int64),
                     prob=np.zeros((nh, N, N), np.int64), code=np.zeros((nh, N, N), np.int32),
                     pv=np.zeros((nh, N, d), np.int64))
        dstruct = _Dump(_ptr(dumps["acc"], C.c_int64), _ptr(dumps["logit"], C.c_int32),
                        _ptr(dumps["expv"], C.c_int64), _ptr(dumps["rowsum"], C.c_int64),
                        _ptr(dumps["prob"], C.c_int64), _ptr(dumps["code"], C.c_int32),
                        _ptr(dumps["pv"], C.c_int64))
    rc = lib.orc_forward(C.byref(p), q.ctypes.data, k.ctypes.data, v.ctypes.data,
                         out.ctypes.data, h0, h1, C.byref(dstruct) if dstruct else None)
    del keep
    if rc != 0:
        raise ValueError(f"oracle rejected the parameters (code {rc})")
    res = out.reshape(total, N, d)[h0:h1]
    return (res, dumps) if dump else res


def softmax_row(logits, params: Dict[str, object]):
    """Shiftmax / LIS on one row of int8 logits -> (e, s, prob, code)."""
    lib = _load()
    L = np.ascontiguousarray(np.asarray(logits, dtype=np.int32))
    n = L.shape[0]
    p, keep = _make_params((1, 1, n, 1), params)
    e = np.zeros(n, np.int64)
    s = np.zeros(1, np.int64)
    prob = np.zeros(n, np.int64)
    code = np.zeros(n, np.int32)
    rc = lib.orc_softmax_row(C.byref(p), L.ctypes.data, n, e.ctypes.data, s.ctypes.data,
                             prob.ctypes.data, code.ctypes.data)
    del keep
    if rc != 0:
        raise ValueError(f"oracle softmax_row failed ({rc})")
    return e, int(s[0]), prob, code


def requant(x: int, b: int, c: int) -> int:
    return int(_load().orc_requant(int(x), int(b), int(c)))


def requant_array(x: np.ndarray, b: int, c: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.int64)
    out = np.zeros(x.shape, np.int32)
    _load().orc_requant_array(x.ctypes.data, x.size, int(b), int(c), out.ctypes.data)
    return out


def shift_exp(delta: int, i0: int, n: int) -> int:
    return int(_load().orc_shift_exp(int(delta), int(i0), int(n)))


def ilog2r(x: int) -> int:
    return int(_load().orc_ilog2r(int(x)))


def linear(x: np.ndarray, w: np.ndarray, b: int, c: int, rows=None) -> np.ndarray:
    """Integer-only linear layer: x [rows, in] int8, w [out, in] int8 ->
    [rows, out] int8 (or [r1 - r0, out] for rows=(r0, r1))."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.int8)
    w = np.ascontiguousarray(w, dtype=np.int8)
    M, K = x.shape
    Nc, K2 = w.shape
    if K != K2:
        raise ValueError("x and w disagree on in_features")
    r0, r1 = (0, M) if rows is None else rows
    out = np.zeros((M, Nc), dtype=np.int8)
    rc = lib.orc_linear(x.ctypes.data, w.ctypes.data, M, K, Nc, int(b), int(c),
                        out.ctypes.data, r0, r1)
    if rc != 0:
        raise ValueError(f"orc_linear: invalid arguments ({rc})")
    return out[r0:r1]


def shiftgelu(x: np.ndarray, params: Dict[str, int], rows=None, dump=False):
    """ShiftGELU of x [rows, cols] int8 -> int8 (and, with dump, an int64 array
    [rows, cols, 4] of (Ip, e1, e2, sigmoid code) per element)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.int8)
    M, N = x.shape
    r0, r1 = (0, M) if rows is None else rows
    out = np.zeros((M, N), np.int8)
    sig = np.zeros((M, N, 4), np.int64) if dump else None
    rc = lib.orc_shiftgelu(x.ctypes.data, M, N, params["i0"], params["exp_frac_bits"],
                           params["intdiv_m"], params["k_out"], params["b"], params["c"],
                           out.ctypes.data, r0, r1, sig.ctypes.data if dump else None)
    if rc != 0:
        raise ValueError(f"orc_shiftgelu: invalid arguments ({rc})")
    return (out[r0:r1], sig[r0:r1]) if dump else out[r0:r1]


def isqrt10(v: int) -> int:
    return int(_load().orc_isqrt10(int(v)))


def ilayernorm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, params: Dict[str, int],
               rows=None, dump=False):
    """I-LayerNorm of x [rows, cols] int8 with gamma int8 [cols], beta int32
    [cols] -> int8 (and per-row mean, var, sd, floor(2^M / sd))."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.int8)
    g = np.ascontiguousarray(gamma, dtype=np.int8)
    be = np.ascontiguousarray(beta, dtype=np.int32)
    M, N = x.shape
    r0, r1 = (0, M) if rows is None else rows
    out = np.zeros((M, N), np.int8)
    st = np.zeros((M, 4), np.int64) if dump else None
    rc = lib.orc_ilayernorm(x.ctypes.data, g.ctypes.data, be.ctypes.data, M, N,
                            params["norm_frac_bits"], params["intdiv_m"], params["b"],
                            params["c"], out.ctypes.data, r0, r1,
                            st.ctypes.data if dump else None)
    if rc != 0:
        raise ValueError(f"orc_ilayernorm: invalid arguments ({rc})")
    return (out[r0:r1], st[r0:r1]) if dump else out[r0:r1]


class _LinattnParams(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("batch", "heads", "seq_len", "head_dim")] + \
        [(n, C.c_int32) for n in ("kv_b", "kv_c", "ks_b", "ks_c", "out_b", "out_c")]


def linattn(q: np.ndarray, k: np.ndarray, v: np.ndarray, params: Dict[str, int], heads=None,
            dump=False):
    """Softmax-free integer linear attention of int8 Q, K, V [B, H, N, d] -> int8
    [B, H, N, d] (and, with dump, the int64 requantised KV [d, d] and ks [d] per
    head, shaped [B * H, d * d + d]).  heads = (begin, end) over the flattened
    B * H limits the heads computed; the others stay 0."""
    lib = _load()
    q, k, v = (np.ascontiguousarray(t, dtype=np.int8) for t in (q, k, v))
    B, H, N, d = q.shape
    pp = _LinattnParams(B, H, N, d, *(int(params[n]) for n in
                                     ("kv_b", "kv_c", "ks_b", "ks_c", "out_b", "out_c")))
    h0, h1 = (0, B * H) if heads is None else heads
    out = np.zeros(q.shape, np.int8)
    dm = np.zeros((max(h1 - h0, 0), d * d + d), np.int64) if dump else None
    rc = lib.orc_linattn(C.addressof(pp), q.ctypes.data, k.ctypes.data, v.ctypes.data,
                         out.ctypes.data, h0, h1, dm.ctypes.data if dump else None)
    if rc != 0:
        raise ValueError(f"orc_linattn: invalid arguments ({rc})")
    return (out, dm) if dump else out
