"""The C-ABI library: loads, exports every declared symbol, rejects bad
parameters before touching a device (no GPU needed)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from integer_only_quantized_int8_amd import iqattn as IQ
from integer_only_quantized_int8_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(iq(?:attn|linear|gelu|layernorm|linattn)_\w+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(IQ.LIB_PATH):
        from integer_only_quantized_int8_amd import build
        build.build()
    return IQ.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared == set(IQ.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(os.path.join(ROOT, "include", "iqattn.h")).read()
    for name in ("IQATTN_OK", "IQATTN_E_INVAL", "IQATTN_E_SHAPE", "IQATTN_E_ALLOC",
                 "IQATTN_E_LAUNCH", "IQATTN_E_NULL", "IQATTN_E_ALIGN", "IQATTN_E_DEVICE",
                 "IQATTN_SHIFTMAX", "IQATTN_LIS", "IQATTN_LIS_VALU", "IQATTN_LIS_MFMA",
                 "IQATTN_OUT_HEADS", "IQATTN_OUT_TOKENS", "IQATTN_MAX_SEQ",
                 "IQATTN_E_INCOMPLETE", "IQATTN_E_TOOBIG"):
        m = re.search(r"#define\s+%s\s+(-?\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(IQ, name), name
    text = open(os.path.join(ROOT, "include", "iqlinear.h")).read()
    for name in ("IQLINEAR_PLAIN", "IQLINEAR_QKV_HEADS"):
        m = re.search(r"#define\s+%s\s+(-?\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(IQ, name), name


def _create_rc(lib, shape, **over):
    params = W.default_params(3)
    params.update(over)
    p, keep = IQ.make_params(shape, params)
    ctx = C.c_void_p(12345)
    rc = lib.iqattn_create(C.byref(p), C.byref(ctx))
    del keep
    return rc, ctx.value


@pytest.mark.parametrize("shape,over,code", [
    ((1, 1, 0, 64), {}, IQ.IQATTN_E_SHAPE),
    ((1, 1, 1025, 64), {}, IQ.IQATTN_E_SHAPE),
    ((1, 40000, 1024, 64), {"out_layout": 1}, IQ.IQATTN_E_SHAPE),
    ((1, 1, 16, 48), {}, IQ.IQATTN_E_SHAPE),
    ((-1, 1, 16, 64), {}, IQ.IQATTN_E_SHAPE),
    ((1, 0, 16, 64), {}, IQ.IQATTN_E_SHAPE),
    ((1, 1, 16, 64), {"qk_b": 0}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"pv_c": 63}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"i0": 0}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"i0": 16, "exp_frac_bits": 19}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"k_out": 9}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"intdiv_m": 32}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"variant": 2}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"variant": 1, "lis_bits": 5}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"variant": 1, "intdiv_m": 14}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"variant": 1, "lis_engine": 2}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"variant": 1, "lis_engine": -1}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"window": 4}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"out_layout": 2}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"out_layout": -1}, IQ.IQATTN_E_INVAL),
    ((1, 1, 16, 64), {"window": 3, "rel_bias": np.zeros((1, 25), np.int32)}, IQ.IQATTN_E_SHAPE),
    ((1, 1, 16, 64), {"window": 4, "rel_bias": np.full((1, 49), (1 << 30) + 1, np.int32)},
     IQ.IQATTN_E_INVAL),
])
def test_create_rejects_bad_parameters_before_any_device_call(lib, shape, over, code):
    rc, ctx = _create_rc(lib, shape, **over)
    assert rc == code
    assert ctx is None  # *out is cleared on every error


def test_null_pointers_and_destroy_null(lib):
    assert lib.iqattn_create(None, None) == IQ.IQATTN_E_NULL
    p, _ = IQ.make_params((1, 1, 16, 64), W.default_params(1))
    assert lib.iqattn_create(C.byref(p), None) == IQ.IQATTN_E_NULL
    assert lib.iqattn_destroy(None) == IQ.IQATTN_OK
    assert lib.iqattn_forward(None, None, None, None, None, None) == IQ.IQATTN_E_NULL
    assert lib.iqattn_check(None, None) == IQ.IQATTN_E_NULL
    assert lib.iqattn_set_spin_limit(None, 1) == IQ.IQATTN_E_NULL


def test_strerror_texts(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -99):
        s = IQ.iqattn_strerror(code)
        assert isinstance(s, str) and s


def _linear_rc(lib, **over):
    p = dict(rows=4, in_features=64, out_features=64, layout=IQ.IQLINEAR_PLAIN, batch=0,
             seq_len=0, heads=0, head_dim=0, b=(20000, 1, 1), c=(20, 1, 1))
    p.update(over)
    s = IQ.make_linear_params(p)
    ctx = C.c_void_p(12345)
    rc = lib.iqlinear_create(C.byref(s), C.byref(ctx))
    return rc, ctx.value


@pytest.mark.parametrize("over,code", [
    (dict(rows=-1), IQ.IQATTN_E_SHAPE),
    (dict(in_features=48), IQ.IQATTN_E_SHAPE),
    (dict(in_features=0), IQ.IQATTN_E_SHAPE),
    (dict(out_features=72), IQ.IQATTN_E_SHAPE),
    (dict(layout=2), IQ.IQATTN_E_INVAL),
    (dict(b=(0, 1, 1)), IQ.IQATTN_E_INVAL),
    (dict(c=(63, 1, 1)), IQ.IQATTN_E_INVAL),
    (dict(layout=IQ.IQLINEAR_QKV_HEADS, rows=6, out_features=192, batch=2, seq_len=3, heads=1,
          head_dim=64, b=(1, 1, 0), c=(1, 1, 1)), IQ.IQATTN_E_INVAL),
    (dict(layout=IQ.IQLINEAR_QKV_HEADS, rows=7, out_features=192, batch=2, seq_len=3, heads=1,
          head_dim=64, b=(1, 1, 1), c=(1, 1, 1)), IQ.IQATTN_E_SHAPE),
    (dict(layout=IQ.IQLINEAR_QKV_HEADS, rows=6, out_features=24, batch=2, seq_len=3, heads=1,
          head_dim=8, b=(1, 1, 1), c=(1, 1, 1)), IQ.IQATTN_E_SHAPE),
])
def test_linear_create_rejects_bad_parameters_before_any_device_call(lib, over, code):
    rc, ctx = _linear_rc(lib, **over)
    assert rc == code
    assert ctx is None


def test_linear_null_arguments(lib):
    assert lib.iqlinear_create(None, None) == IQ.IQATTN_E_NULL
    assert lib.iqlinear_destroy(None) == IQ.IQATTN_OK
    assert lib.iqlinear_forward(None, None, None, None, None, None, None) == IQ.IQATTN_E_NULL


def _gelu_rc(lib, **over):
    p = dict(rows=4, cols=64, i0=16, exp_frac_bits=22, intdiv_m=40, k_out=8, b=20000, c=22)
    p.update(over)
    ctx = C.c_void_p(12345)
    rc = lib.iqgelu_create(C.byref(IQ.make_gelu_params(p)), C.byref(ctx))
    return rc, ctx.value


@pytest.mark.parametrize("over,code", [
    (dict(rows=-1), IQ.IQATTN_E_SHAPE), (dict(cols=0), IQ.IQATTN_E_SHAPE),
    (dict(cols=8), IQ.IQATTN_E_SHAPE), (dict(cols=72), IQ.IQATTN_E_SHAPE),
    (dict(cols=16400), IQ.IQATTN_E_SHAPE), (dict(rows=1 << 20, cols=4096), IQ.IQATTN_E_SHAPE),
    (dict(i0=0), IQ.IQATTN_E_INVAL), (dict(i0=32769), IQ.IQATTN_E_INVAL),
    (dict(exp_frac_bits=31), IQ.IQATTN_E_INVAL), (dict(k_out=1), IQ.IQATTN_E_INVAL),
    (dict(k_out=9), IQ.IQATTN_E_INVAL), (dict(intdiv_m=6), IQ.IQATTN_E_INVAL),
    (dict(intdiv_m=41), IQ.IQATTN_E_INVAL), (dict(b=0), IQ.IQATTN_E_INVAL),
    (dict(c=63), IQ.IQATTN_E_INVAL), (dict(c=-1), IQ.IQATTN_E_INVAL),
])
def test_gelu_create_rejects_bad_parameters_before_any_device_call(lib, over, code):
    rc, ctx = _gelu_rc(lib, **over)
    assert rc == code
    assert ctx is None


def _ln_rc(lib, **over):
    p = dict(rows=4, cols=64, norm_frac_bits=7, intdiv_m=22, b=20000, c=22)
    p.update(over)
    ctx = C.c_void_p(12345)
    rc = lib.iqlayernorm_create(C.byref(IQ.make_layernorm_params(p)), C.byref(ctx))
    return rc, ctx.value


@pytest.mark.parametrize("over,code", [
    (dict(rows=-1), IQ.IQATTN_E_SHAPE), (dict(cols=0), IQ.IQATTN_E_SHAPE),
    (dict(cols=40), IQ.IQATTN_E_SHAPE), (dict(cols=16384 + 16), IQ.IQATTN_E_SHAPE),
    (dict(norm_frac_bits=-1), IQ.IQATTN_E_INVAL), (dict(norm_frac_bits=9), IQ.IQATTN_E_INVAL),
    (dict(intdiv_m=6), IQ.IQATTN_E_INVAL), (dict(intdiv_m=23), IQ.IQATTN_E_INVAL),
    (dict(b=0), IQ.IQATTN_E_INVAL), (dict(c=63), IQ.IQATTN_E_INVAL),
])
def test_layernorm_create_rejects_bad_parameters_before_any_device_call(lib, over, code):
    rc, ctx = _ln_rc(lib, **over)
    assert rc == code
    assert ctx is None


def test_block_null_arguments(lib):
    assert lib.iqgelu_create(None, None) == IQ.IQATTN_E_NULL
    assert lib.iqgelu_destroy(None) == IQ.IQATTN_OK
    assert lib.iqgelu_forward(None, None, None, None) == IQ.IQATTN_E_NULL
    assert lib.iqlayernorm_create(None, None) == IQ.IQATTN_E_NULL
    assert lib.iqlayernorm_destroy(None) == IQ.IQATTN_OK
    assert lib.iqlayernorm_forward(None, None, None, None, None, None) == IQ.IQATTN_E_NULL


def _la_rc(lib, **over):
    p = dict(batch=2, heads=3, seq_len=40, head_dim=16, kv_b=20000, kv_c=20, ks_b=20000,
             ks_c=12, out_b=20000, out_c=8)
    p.update(over)
    shape = (p.pop("batch"), p.pop("heads"), p.pop("seq_len"), p.pop("head_dim"))
    ctx = C.c_void_p(12345)
    rc = lib.iqlinattn_create(C.byref(IQ.make_linattn_params(shape, p)), C.byref(ctx))
    return rc, ctx.value


@pytest.mark.parametrize("over,code", [
    (dict(batch=-1), IQ.IQATTN_E_SHAPE), (dict(heads=0), IQ.IQATTN_E_SHAPE),
    (dict(seq_len=0), IQ.IQATTN_E_SHAPE), (dict(seq_len=65537), IQ.IQATTN_E_SHAPE),
    (dict(head_dim=8), IQ.IQATTN_E_SHAPE), (dict(head_dim=48), IQ.IQATTN_E_SHAPE),
    (dict(head_dim=128), IQ.IQATTN_E_SHAPE),
    (dict(batch=1024, heads=64, seq_len=1024, head_dim=64), IQ.IQATTN_E_SHAPE),
    (dict(kv_b=0), IQ.IQATTN_E_INVAL), (dict(ks_c=63), IQ.IQATTN_E_INVAL),
    (dict(out_c=-1), IQ.IQATTN_E_INVAL), (dict(out_b=0), IQ.IQATTN_E_INVAL),
])
def test_linattn_create_rejects_bad_parameters_before_any_device_call(lib, over, code):
    rc, ctx = _la_rc(lib, **over)
    assert rc == code
    assert ctx is None


def test_linattn_null_arguments(lib):
    assert lib.iqlinattn_create(None, None) == IQ.IQATTN_E_NULL
    assert lib.iqlinattn_destroy(None) == IQ.IQATTN_OK
    assert lib.iqlinattn_forward(None, None, None, None, None, None) == IQ.IQATTN_E_NULL


def test_struct_layouts_match_headers():
    """Every parameter struct of include/*.h has the size and field offsets of
    its ctypes twin in the binding (a small C program, built in the
    repository's untracked _build/, prints them)."""
    import pathlib
    import subprocess
    tmp_path = pathlib.Path(ROOT) / "_build" / "layout_check"
    tmp_path.mkdir(parents=True, exist_ok=True)
    structs = {
        "iqattn_params": (IQ.iqattn_params, "iqattn.h"),
        "iqlinear_params": (IQ.iqlinear_params, "iqlinear.h"),
        "iqgelu_params": (IQ.iqgelu_params, "iqblock.h"),
        "iqlayernorm_params": (IQ.iqlayernorm_params, "iqblock.h"),
        "iqlinattn_params": (IQ.iqlinattn_params, "iqlinattn.h"),
    }
    lines = ["#include <stdio.h>", "#include <stddef.h>"]
    lines += sorted({f'#include "{h}"' for _, h in structs.values()})
    lines.append("int main(void) {")
    for name, (cls, _) in structs.items():
        lines.append(f'  printf("{name} size %zu\\n", sizeof({name}));')
        for field, _ in cls._fields_:
            lines.append(f'  printf("{name} {field} %zu\\n", offsetof({name}, {field}));')
    lines.append("  return 0;\n}")
    src = tmp_path / "layout.c"
    exe = tmp_path / "layout"
    src.write_text("\n".join(lines) + "\n")
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), "-o",
                           str(exe), str(src)])
    out = subprocess.check_output([str(exe)]).decode().split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for name, (cls, _) in structs.items():
        assert got[(name, "size")] == C.sizeof(cls), name
        for field, _ in cls._fields_:
            assert got[(name, field)] == getattr(cls, field).offset, (name, field)


def test_noalloc_rejects_before_any_device_call(lib):
    """iqattn_forward_noalloc checks ranges, pointers and its static-memory
    limits before any HIP call (no device here)."""
    params = W.default_params(3)
    fake = C.c_void_p(16 * 1024)
    def call(shape, **over):
        p, keep = IQ.make_params(shape, dict(params, **over))
        rc = lib.iqattn_forward_noalloc(C.byref(p), fake, fake, fake, fake, None)
        del keep
        return rc
    assert call((1, 1, 1025, 64)) == IQ.IQATTN_E_SHAPE
    assert call((1, 1, 16, 64), qk_b=0) == IQ.IQATTN_E_INVAL
    assert call((0, 1, 16, 64)) == IQ.IQATTN_OK          # empty batch: nothing to do
    p, keep = IQ.make_params((1, 1, 16, 64), params)
    assert lib.iqattn_forward_noalloc(C.byref(p), None, fake, fake, fake, None) == IQ.IQATTN_E_NULL
    bad = C.c_void_p(16 * 1024 + 3)
    assert lib.iqattn_forward_noalloc(C.byref(p), bad, fake, fake, fake, None) == IQ.IQATTN_E_ALIGN
    # the windowed bias: relative tables of more than 960 entries
    assert call((1, 20, 49, 32), window=7, rel_bias=np.zeros((20, 169), np.int32)) == \
        IQ.IQATTN_E_TOOBIG
    assert call((1, 2, 400, 32), window=20, rel_bias=np.zeros((2, 39 * 39), np.int32)) == \
        IQ.IQATTN_E_TOOBIG
    # within the limits the call gets as far as the device
    assert call((1, 3, 49, 32), window=7, rel_bias=np.zeros((3, 169), np.int32)) == \
        IQ.IQATTN_E_DEVICE
    assert call((2, 3, 197, 64)) == IQ.IQATTN_E_DEVICE
