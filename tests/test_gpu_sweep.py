"""Seeded random sweeps over each operator's documented parameter domain,
bit-exact against the oracle.

The hand-picked cases of the other parity tests sit at chosen corners; these
draws mix shapes, dyadic pairs, exponent constants, variants, engines, bias
ranges and output layouts at random, so that each of the host's choices of
kernel and arithmetic form (specialised or generic kernel, 24-bit or 32-bit
products, fast or wide requantisation) meets many neighbours.  Most pairs
are drawn so that the results spread over the int8 range (the scale of the
accumulator is estimated from the input spread); the others are drawn
anywhere in the domain, where results mostly saturate or vanish."""
import math
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


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.device("cuda:0"))


def draw_pair(rng, acc_sd, lo_target=2.0, hi_target=100.0, wild=0.25):
    """(b, c) with 1 <= b < 2^31, 0 <= c <= 62.  Mostly b / 2^c maps an
    accumulator of spread acc_sd to an int8 spread in [lo, hi]; with
    probability `wild` anywhere in the domain."""
    if rng.random() < wild:
        b = int(min((1 << 31) - 1, math.floor(2.0 ** rng.uniform(0.0, 31.0))))
        return max(1, b), int(rng.integers(0, 63))
    kb = int(rng.integers(0, 31))
    b = int(rng.integers(1 << kb, (1 << (kb + 1)) if kb < 30 else (1 << 31) - 1))
    target = rng.uniform(lo_target, hi_target)
    c = int(round(math.log2(max(b * max(acc_sd, 1e-9) / target, 1e-30))))
    return b, min(62, max(0, c))


# ------------------------------------------------------------------ attention

# (head_dim, key tiles of 16, relative bias, variant) of specialised kernels:
# the workload shapes (N = 197, 577, 49 with and without bias) and short ones
SPECIALISED = ([(64, kt, False, 0) for kt in (1, 2, 4, 12, 13, 37)]
               + [(64, 4, True, 0), (32, 4, True, 0), (32, 4, False, 0), (32, 13, False, 0)]
               + [(64, kt, False, 1) for kt in (1, 5, 13, 37)] + [(32, 4, False, 1)])

def draw_attention(i):
    rng = np.random.default_rng(70000 + i)
    # three draws in four are "tame": the exponent constants leave the row sum
    # room below 2^M (else the IntDiv factor is 0 and every probability
    # vanishes), the bias stays near the accumulator's scale and both pairs
    # aim at a useful int8 spread; the rest draw all of these anywhere
    tame = rng.random() < 0.75
    # shapes: six draws in ten take the head size, key-tile count (16 keys),
    # bias and variant of a kernel specialised for the workload shapes, the
    # rest anything in the domain (mostly the generic kernel)
    window = 0
    d_kt_fixed = rng.random() < 0.6
    if d_kt_fixed:
        d, kt, bias, variant = SPECIALISED[int(rng.integers(0, len(SPECIALISED)))]
        if bias:
            window = int(rng.choice([w for w in range(1, 26) if (w * w + 15) // 16 == kt]))
            N = window * window
        else:
            N = int(rng.integers(16 * (kt - 1) + 1, 16 * kt + 1))
    else:
        variant = int(rng.integers(0, 2))
        d = int(rng.choice([32, 64]))
        if rng.random() < 0.25:
            window = int(rng.integers(1, 26))
            N = window * window
        else:
            N = int(rng.integers(1, 1025))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    # inputs: spread 1 to 128 (specialised shapes 8 to 128: below that the
    # logit pair b / 2^c passes 1/2 and the generic kernel takes the call)
    sigma = float(2.0 ** rng.uniform(3.0 if d_kt_fixed else 0.0, 7.0))
    bias_range = int(rng.choice([1, 64, 512, 4000] + ([] if tame else [1 << 20, 1 << 30])))
    w = W.make_workload(B, H, N, d, seed=80000 + i, sigma=sigma, variant=variant,
                        window=window, bias_range=bias_range,
                        k_outlier_p=float(rng.choice([0.0, 0.05])))
    p = dict(w.params)
    k_out = int(rng.integers(2, 9))
    lis_bits = int(rng.integers(1, 5))
    m_lo = max(k_out - 1, (1 << lis_bits) - 1 if variant == 1 else 0)
    lg = lambda x: int(math.ceil(math.log2(x))) if x > 1 else 0
    # exponent constants: i0 * 2^n <= 2^22
    if tame:
        i0 = int(math.floor(2.0 ** rng.uniform(0.0, 5.0)))
        M = int(rng.integers(min(31, max(m_lo, k_out + lg(N) + lg(i0))), 32))
        n_hi = max(0, min(22 - lg(i0), M - k_out - lg(N) - lg(i0)))
    else:
        i0 = int(math.floor(2.0 ** rng.uniform(0.0, 12.0)))
        M = int(rng.integers(m_lo, 32))
        n_hi = 22 - lg(i0)
    n = int(rng.integers(0, n_hi + 1))
    wild = 0.0 if tame else 1.0
    # logits: the raw Q.K accumulator has spread ~ sqrt(d) sigma^2; aim the
    # int8 logit at a spread of a few units of i0 (capped by the int8 range)
    s = min(sigma, 127.0)
    lt = min(120.0, i0 * rng.uniform(0.5, 6.0))
    qk_b, qk_c = draw_pair(rng, math.sqrt(d) * s * s, lo_target=max(1.0, lt / 3),
                           hi_target=max(2.0, lt), wild=wild)
    p.update(qk_b=qk_b, qk_c=qk_c, i0=i0, exp_frac_bits=n, intdiv_m=M, k_out=k_out,
             lis_bits=lis_bits, lis_engine=int(rng.integers(0, 2)),
             out_layout=int(rng.integers(0, 2)))
    # P.V pair: the spread of the P.V accumulator (which the pair does not
    # change) is read from the oracle on the first head
    pv = oracle.forward(w.q, w.k, w.v, dict(p, pv_b=1, pv_c=0), heads=(0, 1), dump=True)[1]["pv"]
    p["pv_b"], p["pv_c"] = draw_pair(rng, float(pv.std()), wild=wild)
    return w, p


ATT_CASES = 256


@pytest.mark.parametrize("i", range(ATT_CASES))
def test_attention_sweep(torch_dev, i):
    from integer_only_quantized_int8_amd.iqattn import IQAttn
    torch = torch_dev
    w, p = draw_attention(i)
    B, H, N, d = w.q.shape
    shown = {k: v for k, v in p.items() if k != "rel_bias"}
    _say(f"[sweep] attention draw {i} shape {w.q.shape} {shown}")
    att = IQAttn(w.q.shape, p)
    q, k, v = (_dev(torch, t) for t in (w.q, w.k, w.v))
    oshape = (B, N, H, d) if p["out_layout"] == 1 else (B, H, N, d)
    buf = torch.full((B * H * N * d + 64,), 99, dtype=torch.int8, device="cuda:0")
    out = buf[:B * H * N * d].view(oshape)
    att.forward(q, k, v, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    tail = buf[B * H * N * d:].cpu().numpy()
    att.close()
    assert np.all(tail == 99), "write past the output"
    if p["out_layout"] == 1:
        got = got.transpose(0, 2, 1, 3)
    ref = oracle.forward(w.q, w.k, w.v, p).reshape(B, H, N, d)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"draw {i}: {len(bad)} entries differ, first {bad[:4].tolist()}")


# ------------------------------------------------------------------ linear

def draw_linear(i):
    rng = np.random.default_rng(71000 + i)
    K = 64 * int(rng.integers(1, 17))
    sx, sw = float(2.0 ** rng.uniform(0.0, 7.0)), float(2.0 ** rng.uniform(0.0, 7.0))
    if rng.random() < 0.5:
        B, N = int(rng.integers(1, 4)), int(rng.integers(1, 260))
        H = int(rng.integers(1, 7))
        d = 4 * int(rng.integers(1, 33))
        while (H * d) % 16:
            d += 4
        lw = W.make_linear(B * N, K, 3 * H * d, seed=81000 + i, sigma_x=sx, sigma_w=sw,
                           qkv_heads=(B, N, H, d))
        npairs = 3
    else:
        M = int(rng.choice([int(rng.integers(1, 130)), int(rng.integers(130, 1200))]))
        C = 16 * int(rng.integers(1, 49))
        lw = W.make_linear(M, K, C, seed=81000 + i, sigma_x=sx, sigma_w=sw)
        npairs = 1
    acc = math.sqrt(K) * min(sx, 127.0) * min(sw, 127.0)
    pairs = [draw_pair(rng, acc) for _ in range(npairs)]
    p = dict(lw.params, b=tuple(b for b, _ in pairs), c=tuple(c for _, c in pairs))
    return lw, p


LIN_CASES = 96


@pytest.mark.parametrize("i", range(LIN_CASES))
def test_linear_sweep(torch_dev, i):
    from integer_only_quantized_int8_amd.iqattn import IQLinear
    torch = torch_dev
    lw, p = draw_linear(i)
    _say(f"[sweep] linear draw {i} {p}")
    lin = IQLinear(p)
    x, wt = _dev(torch, lw.x), _dev(torch, lw.w)
    M, C = p["rows"], p["out_features"]
    if p["layout"] == 1:
        B, N, H, d = p["batch"], p["seq_len"], p["heads"], p["head_dim"]
        outs = tuple(torch.full((B, H, N, d), 99, dtype=torch.int8, device="cuda:0")
                     for _ in range(3))
        lin.forward(x, wt, outs)
        torch.cuda.synchronize()
        got = [o.cpu().numpy().transpose(0, 2, 1, 3).reshape(M, H * d) for o in outs]
        C3 = C // 3
        refs = [oracle.linear(lw.x, lw.w[j * C3:(j + 1) * C3], p["b"][j], p["c"][j]) for j in range(3)]
    else:
        out = torch.full((M, C), 99, dtype=torch.int8, device="cuda:0")
        lin.forward(x, wt, out)
        torch.cuda.synchronize()
        got = [out.cpu().numpy()]
        refs = [oracle.linear(lw.x, lw.w, p["b"][0], p["c"][0])]
    lin.close()
    for j, (g, r) in enumerate(zip(got, refs)):
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"draw {i} tensor {j}: {len(bad)} differ, first {bad[:4].tolist()}")


# ------------------------------------------------------------------ ShiftGELU, I-LayerNorm

def draw_gelu(i):
    rng = np.random.default_rng(72000 + i)
    tame = rng.random() < 0.75          # as for the attention draws
    rows, cols = int(rng.integers(1, 300)), 16 * int(rng.integers(1, 257))
    sigma = float(2.0 ** rng.uniform(0.0, 7.0))
    gw = W.make_gelu(rows, cols, seed=82000 + i, sigma=sigma)
    k_out = int(rng.integers(2, 9))
    i0 = int(min(32768, math.floor(2.0 ** rng.uniform(0.0, 15.0))))
    lg = int(math.ceil(math.log2(i0))) if i0 > 1 else 0
    if tame:
        # 2^M above the pair sum e1 + e2 <= 2 i0 2^n, with k_out bits to spare
        M = int(rng.integers(min(40, k_out + lg + 1), 41))
        n = int(rng.integers(0, max(0, min(30, M - k_out - lg - 1)) + 1))
    else:
        M = int(rng.integers(k_out - 1, 41))
        n = int(rng.integers(0, 31))
    p = dict(gw.params, i0=i0, exp_frac_bits=n, k_out=k_out, intdiv_m=M)
    # output accumulator x * sig: the positive half has spread ~ sigma 2^(k_out - 1)
    p["b"], p["c"] = draw_pair(rng, min(sigma, 127.0) * (1 << (k_out - 1)) / 2,
                               wild=0.0 if tame else 1.0)
    return gw, p


def draw_layernorm(i):
    rng = np.random.default_rng(73000 + i)
    tame = rng.random() < 0.75
    rows, cols = int(rng.integers(1, 300)), 16 * int(rng.integers(1, 257))
    beta_range = int(rng.choice([1, 1 << 8, 1 << 14, 1 << 24]))
    lw = W.make_layernorm(rows, cols, seed=83000 + i,
                          sigma_range=(float(rng.uniform(0.0, 4.0)), float(rng.uniform(4.0, 60.0))),
                          beta_range=beta_range)
    F = int(rng.integers(0, 9))
    p = dict(lw.params, norm_frac_bits=F, intdiv_m=int(rng.integers(F, 23)))
    # nrm * gamma + beta: nrm ~ 2^F z, gamma spread 48, beta uniform
    acc = math.sqrt((48.0 * (1 << F)) ** 2 + beta_range ** 2 / 3.0)
    p["b"], p["c"] = draw_pair(rng, acc, wild=0.0 if tame else 1.0)
    return lw, p


GELU_CASES = LN_CASES = 48


@pytest.mark.parametrize("i", range(GELU_CASES))
def test_gelu_sweep(torch_dev, i):
    from integer_only_quantized_int8_amd.iqattn import IQGelu
    torch = torch_dev
    gw, p = draw_gelu(i)
    _say(f"[sweep] gelu draw {i} {gw.x.shape} {p}")
    op = IQGelu(dict(p, rows=gw.rows, cols=gw.cols))
    x = _dev(torch, gw.x)
    out = torch.full_like(x, 99)
    op.forward(x, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    op.close()
    ref = oracle.shiftgelu(gw.x, p)
    assert np.array_equal(got, ref), f"draw {i}: {np.argwhere(got != ref)[:4].tolist()}"


@pytest.mark.parametrize("i", range(LN_CASES))
def test_layernorm_sweep(torch_dev, i):
    from integer_only_quantized_int8_amd.iqattn import IQLayerNorm
    torch = torch_dev
    lw, p = draw_layernorm(i)
    _say(f"[sweep] layernorm draw {i} {lw.x.shape} {p}")
    op = IQLayerNorm(dict(p, rows=lw.rows, cols=lw.cols))
    x, g, b = _dev(torch, lw.x), _dev(torch, lw.gamma), _dev(torch, lw.beta)
    out = torch.full_like(x, 99)
    op.forward(x, g, b, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    op.close()
    ref = oracle.ilayernorm(lw.x, lw.gamma, lw.beta, p)
    assert np.array_equal(got, ref), f"draw {i}: {np.argwhere(got != ref)[:4].tolist()}"


# ------------------------------------------------------------------ linear attention

def draw_linattn(i):
    rng = np.random.default_rng(74000 + i)
    d = int(rng.choice([16, 32, 64]))
    N = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 3000))]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    sigma = float(2.0 ** rng.uniform(0.0, 7.0))
    wl = W.make_linattn(B, H, N, d, seed=84000 + i, sigma=sigma)
    p = dict(wl.params)
    if rng.random() < 0.3:
        for name in ("kv", "ks", "out"):
            p[name + "_b"], p[name + "_c"] = draw_pair(rng, 1.0, wild=1.0)
    return wl, p


LA_CASES = 48


@pytest.mark.parametrize("i", range(LA_CASES))
def test_linattn_sweep(torch_dev, i):
    from integer_only_quantized_int8_amd.iqattn import IQLinAttn
    torch = torch_dev
    wl, p = draw_linattn(i)
    _say(f"[sweep] linear attention draw {i} {wl.q.shape} {p}")
    op = IQLinAttn(wl.q.shape, p)
    q, k, v = (_dev(torch, t) for t in (wl.q, wl.k, wl.v))
    out = torch.full_like(q, 99)
    op.forward(q, k, v, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    op.close()
    ref = oracle.linattn(wl.q, wl.k, wl.v, p)
    assert np.array_equal(got, ref), f"draw {i}: {np.argwhere(got != ref)[:4].tolist()}"
