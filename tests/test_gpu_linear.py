"""Bit-exact parity of the int8 linear layer (through the C-ABI) with the
CPU oracle: plain and head-split layouts, ragged row counts, half-width column
tiles, extreme dyadic pairs, and the ViT-B projection shapes (sampled rows)."""
import sys

import numpy as np
import pytest

import oracle
from integer_only_quantized_int8_amd import workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "no GPU visible"
    return torch


def run_gpu(torch, lw, params=None):
    from integer_only_quantized_int8_amd.iqattn import IQLinear
    P = lw.params if params is None else params
    lin = IQLinear(P)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(lw.x).to(dev)
    w = torch.from_numpy(lw.w).to(dev)
    if P["layout"] == 1:
        shape = (P["batch"], P["heads"], P["seq_len"], P["head_dim"])
        outs = tuple(torch.full(shape, 99, dtype=torch.int8, device=dev) for _ in range(3))
        lin.forward(x, w, outs)
        torch.cuda.synchronize()
        res = [o.cpu().numpy() for o in outs]
    else:
        out = torch.full((P["rows"], P["out_features"]), 99, dtype=torch.int8, device=dev)
        lin.forward(x, w, out)
        torch.cuda.synchronize()
        res = out.cpu().numpy()
    lin.close()
    return res


def oracle_rows(lw, rows, params=None):
    """Oracle result of the given rows: [len(rows), out] per (b, c) pair."""
    P = lw.params if params is None else params
    res = []
    for r in rows:
        if P["layout"] == 1:
            C3 = P["out_features"] // 3
            parts = [oracle.linear(lw.x[r:r + 1], lw.w[i * C3:(i + 1) * C3], P["b"][i], P["c"][i])[0]
                     for i in range(3)]
            res.append(np.concatenate(parts))
        else:
            res.append(oracle.linear(lw.x[r:r + 1], lw.w, P["b"][0], P["c"][0])[0])
    return np.stack(res)


def check(torch, lw, rows=None, params=None, label=""):
    P = lw.params if params is None else params
    _say(f"[linear] {label} rows={P['rows']} in={P['in_features']} out={P['out_features']} "
         f"layout={P['layout']}")
    got = run_gpu(torch, lw, P)
    M = P["rows"]
    sel = np.arange(M) if rows is None else np.asarray(rows)
    ref = oracle_rows(lw, sel, P)
    if P["layout"] == 1:
        B, N, H, d = P["batch"], P["seq_len"], P["heads"], P["head_dim"]
        for which in range(3):
            g = got[which].transpose(0, 2, 1, 3).reshape(B * N, H * d)[sel]
            r = ref[:, which * H * d:(which + 1) * H * d]
            if not np.array_equal(g, r):
                bad = np.argwhere(g != r)
                raise AssertionError(f"{label}: tensor {which} differs at {len(bad)} entries, "
                                     f"first {bad[:4].tolist()}")
    else:
        g = got[sel]
        if not np.array_equal(g, ref):
            bad = np.argwhere(g != ref)
            raise AssertionError(f"{label}: {len(bad)} entries differ, first {bad[:4].tolist()}")


@pytest.mark.parametrize("rows,fin,fout", [
    (1, 64, 64), (128, 64, 128), (129, 128, 64), (300, 192, 192), (64, 768, 320),
    (257, 256, 128), (5, 64, 1024), (33, 64, 48), (130, 128, 208),
])
def test_linear_plain_shapes(torch_dev, rows, fin, fout):
    lw = W.make_linear(rows, fin, fout, seed=rows + fin + fout)
    check(torch_dev, lw, label=f"plain {rows}x{fin}x{fout}")


@pytest.mark.parametrize("B,N,H,d", [(1, 197, 3, 64), (2, 49, 3, 32), (3, 50, 2, 64), (1, 7, 1, 64),
                                     (2, 33, 4, 20), (1, 130, 4, 4)])
def test_linear_qkv_head_split(torch_dev, B, N, H, d):
    lw = W.make_linear(B * N, 128, 3 * H * d, seed=B * 100 + N, qkv_heads=(B, N, H, d))
    check(torch_dev, lw, label=f"qkv B{B} N{N} H{H} d{d}")


@pytest.mark.parametrize("rows,fin,fout", [
    (4229, 512, 1152), (8200, 768, 640), (16387, 256, 2048),
])
def test_linear_several_tiles_per_workgroup(torch_dev, rows, fin, fout):
    """More 128 x 128 tiles than compute units, so that each persistent
    workgroup walks a run of tiles and meets a new 128-row block of X inside
    its run; every element against the oracle."""
    lw = W.make_linear(rows, fin, fout, seed=rows ^ fin ^ fout)
    check(torch_dev, lw, label=f"multi-tile {rows}x{fin}x{fout}")


def test_linear_qkv_head_split_several_tiles(torch_dev):
    B, N, H, d = 32, 197, 4, 64
    lw = W.make_linear(B * N, 768, 3 * H * d, seed=77, qkv_heads=(B, N, H, d))
    check(torch_dev, lw, label=f"qkv multi-tile B{B} N{N} H{H} d{d}")


def test_linear_extreme_dyadic_pairs(torch_dev):
    lw = W.make_linear(70, 128, 64, seed=3, sigma_x=127.0, sigma_w=127.0)
    for b, c in ((1, 0), ((1 << 31) - 1, 62), ((1 << 31) - 1, 40), ((1 << 15) - 1, 32),
                 (1 << 14, 1), (3, 12)):
        check(torch_dev, lw, params=dict(lw.params, b=(b,), c=(c,)), label=f"b={b} c={c}")


def _extreme_operands(rows, fin, fout, seed):
    """x and w whose products reach the int32 accumulator's extremes for this
    depth (+-fin 127 128 and +-fin 127 127) in some rows and columns, random
    Gaussians elsewhere."""
    lw = W.make_linear(rows, fin, fout, seed=seed, sigma_x=60.0, sigma_w=60.0)
    x, w = lw.x.copy(), lw.w.copy()
    x[0], x[1], x[2] = 127, -128, -127
    x[3, ::2], x[3, 1::2] = 127, -128
    w[0], w[1], w[2] = 127, -128, -127
    w[5, ::2], w[5, 1::2] = -128, 127
    lw.x, lw.w = x, w
    return lw


@pytest.mark.parametrize("b,c", [
    (65536, 32),        # the window reaches 2^23 - 1 exactly: the 24-bit path
    (65535, 32),        # one step outside: the general path
    ((1 << 23) - 1, 32), (2047, 20), (1 << 22, 31), (3, 12), (1, 10), (5, 16),
])
def test_linear_requant_window_edges(torch_dev, b, c):
    """Pairs on both sides of the 24-bit window path's limits, with
    accumulators at the int32 extremes of a 1024-deep product so that both
    ends of the window saturate."""
    lw = _extreme_operands(140, 1024, 96, seed=b % 1000 + c)
    check(torch_dev, lw, params=dict(lw.params, b=(b,), c=(c,)), label=f"window b={b} c={c}")


def test_linear_qkv_mixed_pair_paths(torch_dev):
    """Head split with one pair outside the window path (the whole launch
    takes the general path) and with three different window pairs."""
    B, N, H, d = 2, 70, 4, 32
    base = W.make_linear(B * N, 256, 3 * H * d, seed=91, sigma_x=60.0, sigma_w=60.0,
                         qkv_heads=(B, N, H, d))
    for pairs in (((1 << 14) + 3, 24), (5000, 20), ((1 << 31) - 1, 45)), \
                 (((1 << 14) + 3, 24), (2000, 22), (3, 12)):
        P = dict(base.params, b=tuple(p[0] for p in pairs), c=tuple(p[1] for p in pairs))
        check(torch_dev, base, params=P, label=f"qkv pairs {pairs}")


@pytest.mark.parametrize("B,N,H,d", [(2, 33, 4, 20), (1, 130, 4, 4)])
def test_linear_qkv_narrow_heads_general_pairs(torch_dev, B, N, H, d):
    """Head dims that are not a multiple of 16 (per-lane 4-byte stores) with
    pairs outside the 24-bit window path: the 32-bit multiply-high form, the
    64-bit form, and a mix of both over Q, K and V."""
    lw = W.make_linear(B * N, 128, 3 * H * d, seed=B * 31 + N, sigma_x=80.0, sigma_w=80.0,
                       qkv_heads=(B, N, H, d))
    for pairs in (((1 << 31) - 1, 45), (((1 << 31) - 1, 40), ((1 << 31) - 1, 40), (5000, 20))):
        if isinstance(pairs[0], int):
            pairs = (pairs, pairs, pairs)
        P = dict(lw.params, b=tuple(x[0] for x in pairs), c=tuple(x[1] for x in pairs))
        check(torch_dev, lw, params=P, label=f"qkv narrow B{B} N{N} H{H} d{d} pairs {pairs}")


def test_linear_vitb_projections_sampled_rows(torch_dev):
    for name in W.LINEAR_CONFIGS:
        lw = W.linear_workload(name)
        M = lw.params["rows"]
        rows = sorted(set([0, 1, 127, 128, M - 1] +
                          list(np.random.default_rng(1).choice(M, 24, replace=False))))
        check(torch_dev, lw, rows=rows, label=name)


@pytest.mark.parametrize("rows,fin,fout", [(100864, 768, 2304), (40000, 192, 1040),
                                           (100864, 192, 1040)])
def test_linear_many_tiles_per_workgroup(torch_dev, rows, fin, fout):
    # more than twice as many output tiles as the persistent grid has
    # workgroups (up to 14 per workgroup), an odd k-block count and a column
    # count that leaves a partial column tile: the tile table, the load ring
    # across tile boundaries and the ragged edges, on sampled rows (the first
    # and the last shape take 256 x 256 tiles, the second 256 x 128)
    lw = W.make_linear(rows, fin, fout, seed=rows + fin + fout)
    M = lw.params["rows"]
    pick = sorted(set([0, 255, 256, M - 257, M - 1] +
                      list(np.random.default_rng(7).choice(M, 40, replace=False))))
    check(torch_dev, lw, rows=pick, label=f"{rows}x{fin}x{fout}")
