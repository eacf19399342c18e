"""Bit-exact parity of the HIP path (through the C-ABI) with the CPU oracle.

Every output is an integer, so the GPU result must equal the oracle byte for
byte.  Full-size workloads are compared on every head the oracle finishes in
seconds, and on sampled heads otherwise.
"""
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


def run_gpu(torch, w, params=None, stream=None):
    from integer_only_quantized_int8_amd.iqattn import IQAttn
    params = w.params if params is None else params
    att = IQAttn(w.q.shape, params)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(w.q).to(dev)
    k = torch.from_numpy(w.k).to(dev)
    v = torch.from_numpy(w.v).to(dev)
    out = torch.full_like(q, 99)
    att.forward(q, k, v, out, stream=stream)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    from integer_only_quantized_int8_amd.iqattn import IQATTN_OK
    assert att.check(stream) == IQATTN_OK, "a bounded wait gave up"
    att.close()
    return res


def check(torch, w, params=None, heads=None, label=""):
    """Compare the GPU output with the oracle.  A Log-Int-Softmax case runs both
    P.V engines (VALU shift-add and MFMA bit planes) against the same oracle
    result."""
    params = w.params if params is None else params
    engines = [0, 1] if params["variant"] == 1 else [None]
    total = w.batch * w.heads
    N, d = w.seq_len, w.head_dim
    gots = []
    for eng in engines:
        pe = params if eng is None else dict(params, lis_engine=eng)
        _say(f"[parity] {label} {w.q.shape} variant={params['variant']} engine={eng} "
             f"heads={heads}")
        gots.append((eng, run_gpu(torch, w, pe).reshape(total, N, d)))
    if heads is None:
        ref = oracle.forward(w.q, w.k, w.v, params)
        for eng, got in gots:
            if not np.array_equal(got, ref):
                bad = np.argwhere(got != ref)
                raise AssertionError(f"{label} engine={eng}: {len(bad)} entries differ, "
                                     f"first {bad[:4].tolist()}")
        return
    for u in heads:
        ref = oracle.forward(w.q, w.k, w.v, params, heads=(int(u), int(u) + 1))[0]
        for eng, got in gots:
            if not np.array_equal(got[u], ref):
                bad = np.argwhere(got[u] != ref)
                raise AssertionError(f"{label} engine={eng}: head {u} differs at {len(bad)} "
                                     f"entries, first {bad[:4].tolist()}")


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_config_full(torch_dev, cfg):
    w = W.config_workload(cfg)
    check(torch_dev, w, label=f"shape {cfg} seed {1000 + cfg}")


def test_headline_config_all_heads(torch_dev):
    w = W.config_workload(2)
    check(torch_dev, w, label="shape 2 seed 1002 (all 1536 heads)")


def test_lis_config_all_heads(torch_dev):
    w = W.config_workload(4)
    check(torch_dev, w, label="shape 4 seed 1004 (all 512 heads, both P.V engines)")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_configs_other_seeds_reduced_batch(torch_dev, cfg, seed):
    spec = dict(W.CONFIGS[cfg])
    spec["batch"] = {0: 1, 1: 4, 2: 2, 3: 24, 4: 1}[cfg]
    w = W.make_workload(seed=seed, **spec)
    check(torch_dev, w, label=f"shape {cfg} seed {seed}")


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("N", [1, 2, 15, 16, 17, 31, 33, 49, 63, 64, 65, 130, 197, 208, 209,
                               400, 577, 640, 641, 768, 1000, 1024])
def test_edge_shapes(torch_dev, N, d, variant):
    w = W.make_workload(2, 3, N, d, seed=N * 7 + d + variant, variant=variant)
    check(torch_dev, w, label=f"edge N={N} d={d}")


@pytest.mark.parametrize("w,d", [(26, 64), (32, 32), (32, 64)])
@pytest.mark.parametrize("variant", [0, 1])
def test_long_rows_with_window_bias(torch_dev, w, d, variant):
    wl = W.make_workload(1, 2, w * w, d, seed=w * 3 + d + variant, variant=variant, window=w)
    check(torch_dev, wl, label=f"long row with bias w={w} d={d}")


@pytest.mark.parametrize("N,d,window", [(2, 64, 0), (37, 64, 0), (197, 64, 0), (25, 32, 5),
                                        (49, 64, 7), (700, 64, 0)])
@pytest.mark.parametrize("variant", [0, 1])
def test_int8_extremes(torch_dev, N, d, window, variant):
    """Inputs at both ends of int8 (-128 included, which the header accepts
    although the workloads clip to +-127), a small requantisation scale and
    i0 = 3, so that accumulators reach d * 128 * 128 in magnitude: padded keys
    must still stay below every real key of the row."""
    wl = W.make_workload(2, 2, N, d, seed=N + d + window + variant, variant=variant,
                         window=window)
    rng = np.random.default_rng(N * 7 + variant)
    ext = np.array([-128, 127, -127, 0], dtype=np.int8)
    for t in (wl.q, wl.k, wl.v):
        t[:] = rng.choice(ext, size=t.shape, p=[0.45, 0.45, 0.05, 0.05])
    wl.q[0, 0] = -128                       # rows whose every product is -128 * 127
    wl.k[0, 0] = 127
    params = dict(wl.params, qk_b=511, qk_c=22, i0=3)
    if variant == 1:
        params["pv_c"] = 28
    check(torch_dev, wl, params=params, label=f"int8 extremes N={N} d={d} window={window}")
    if N == 2:                              # Q = -128 and K = 127 everywhere
        wl.q[:] = -128
        wl.k[:] = 127
        check(torch_dev, wl, params=params, label="Q=-128 K=127")


def test_all_equal_logits(torch_dev):
    w = W.make_workload(2, 2, 197, 64, seed=5)
    w.q[:] = 0
    check(torch_dev, w, label="Q=0")
    p = dict(w.params, variant=1, pv_c=28)
    check(torch_dev, w, params=p, label="Q=0 LIS")


def test_saturated_logits_and_dyadic_extremes(torch_dev):
    w = W.make_workload(2, 2, 197, 64, seed=6, sigma=127.0)
    for qk_b, qk_c in ((1 << 14, 22), ((1 << 15) - 1, 22), ((1 << 15) - 1, 12), (1, 1),
                       ((1 << 31) - 1, 30)):
        p = dict(w.params, qk_b=qk_b, qk_c=qk_c)
        check(torch_dev, w, params=p, label=f"qk b={qk_b} c={qk_c}")
    for pv_b, pv_c in ((1 << 14, 20), ((1 << 15) - 1, 20), ((1 << 31) - 1, 40)):
        p = dict(w.params, pv_b=pv_b, pv_c=pv_c)
        check(torch_dev, w, params=p, label=f"pv b={pv_b} c={pv_c}")


def test_outlier_rows_and_bias(torch_dev):
    w = W.make_workload(2, 3, 197, 64, seed=9, per_head_sigma=(8.0, 40.0), k_outlier_p=0.05)
    check(torch_dev, w, label="outliers")
    w = W.make_workload(5, 2, 49, 32, seed=10, window=7, bias_range=4000)
    check(torch_dev, w, label="large bias")
    w = W.make_workload(2, 2, 64, 64, seed=11, window=8)
    check(torch_dev, w, label="bias w=8 d=64")


@pytest.mark.parametrize("over", [dict(i0=1, exp_frac_bits=0), dict(i0=5, exp_frac_bits=3),
                                  dict(i0=16, exp_frac_bits=8, intdiv_m=31),
                                  dict(k_out=4, intdiv_m=20), dict(i0=64, exp_frac_bits=16),
                                  dict(k_out=2)])
def test_other_exponent_parameters(torch_dev, over):
    w = W.make_workload(2, 2, 100, 64, seed=12)
    check(torch_dev, w, params=dict(w.params, **over), label=f"params {over}")
    pl = dict(w.params, variant=1, pv_c=28, **over)
    if pl["intdiv_m"] >= 15:
        check(torch_dev, w, params=pl, label=f"LIS params {over}")


def test_lis_bits(torch_dev):
    w = W.make_workload(2, 2, 77, 64, seed=13, variant=1)
    for bits in (1, 2, 3, 4):
        check(torch_dev, w, params=dict(w.params, lis_bits=bits), label=f"lis_bits={bits}")


def test_deterministic_repeat_and_streams(torch_dev):
    torch = torch_dev
    from integer_only_quantized_int8_amd.iqattn import IQAttn
    w = W.make_workload(16, 12, 197, 64, seed=14)
    att = IQAttn(w.q.shape, w.params)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    torch.cuda.synchronize()
    att.forward(q, k, v, o1, stream=s1)
    att.forward(q, k, v, o2, stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    o3 = att.forward(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3)
    att.close()
    ref = oracle.forward(w.q, w.k, w.v, w.params, heads=(0, 12))
    assert np.array_equal(o1.cpu().numpy().reshape(-1, 197, 64)[:12], ref)


def test_empty_batch_and_alignment_errors(torch_dev):
    torch = torch_dev
    from integer_only_quantized_int8_amd import iqattn as IQ
    w = W.make_workload(1, 2, 33, 64, seed=15)
    att = IQ.IQAttn((0, 2, 33, 64), w.params)
    e = torch.empty((0, 2, 33, 64), dtype=torch.int8, device="cuda:0")
    att.forward(e, e, e)
    att.close()
    att = IQ.IQAttn((1, 2, 33, 64), w.params)
    buf = torch.zeros(2 * 33 * 64 + 1, dtype=torch.int8, device="cuda:0")
    mis = buf[1:].view(1, 2, 33, 64)
    with pytest.raises(IQ.IQAttnError) as ei:
        att.forward(mis, mis, mis)
    assert ei.value.code == IQ.IQATTN_E_ALIGN
    att.close()


@pytest.mark.parametrize("spec,engine", [
    (dict(W.CONFIGS[0]), None),                                   # specialised, 13 key tiles
    (dict(W.CONFIGS[3], batch=8), None),                          # windowed, bias, d = 32
    (dict(W.CONFIGS[4], batch=1, heads=3), 0),                    # LIS, VALU P.V, 577 keys
    (dict(W.CONFIGS[4], batch=1, heads=3), 1),                    # LIS, MFMA P.V
    (dict(batch=2, heads=3, seq_len=400, head_dim=64), None),     # generic kernel
    (dict(batch=2, heads=3, seq_len=400, head_dim=32, variant=1), 0),  # generic LIS
])
def test_token_major_output(torch_dev, spec, engine):
    """out_layout IQATTN_OUT_TOKENS writes [B, N, H, d] (rows of H d features
    per token): the same bytes as the head-major result, transposed."""
    torch = torch_dev
    from integer_only_quantized_int8_amd.iqattn import IQAttn, IQATTN_OUT_TOKENS
    spec = {k: v for k, v in spec.items() if k != "name"}
    w = W.make_workload(seed=77, **spec)
    params = dict(w.params, out_layout=IQATTN_OUT_TOKENS)
    if engine is not None:
        params["lis_engine"] = engine
    _say(f"[parity] token-major {w.q.shape} variant={w.params['variant']} engine={engine}")
    att = IQAttn(w.q.shape, params)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
    B, H, N, d = w.q.shape
    buf = torch.full((B * N * H * d + 64,), 99, dtype=torch.int8, device=dev)
    out = buf[:B * N * H * d].view(B, N, H, d)
    att.forward(q, k, v, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    att.close()
    assert np.all(buf[B * N * H * d:].cpu().numpy() == 99), "write past the output"
    ref = oracle.forward(w.q, w.k, w.v, w.params if engine is None else params)
    ref = ref.reshape(B, H, N, d).transpose(0, 2, 1, 3)
    assert np.array_equal(got, ref), f"{np.argwhere(got != ref)[:4].tolist()}"


def test_msa_block_without_transposes(torch_dev):
    """Q/K/V projection (head-split output), attention (token-major output) and
    output projection chained on the GPU, no reshaping copy in between, against
    the oracle chain."""
    torch = torch_dev
    from integer_only_quantized_int8_amd.iqattn import IQAttn, IQLinear, IQATTN_OUT_TOKENS
    B, N, H, d = 2, 197, 4, 64
    C = H * d
    qkv = W.make_linear(B * N, C, 3 * C, seed=81, qkv_heads=(B, N, H, d))
    proj = W.make_linear(B * N, C, C, seed=82)
    att_w = W.make_workload(seed=83, batch=B, heads=H, seq_len=N, head_dim=d)
    _say("[parity] MSA block: qkv -> attention (token-major) -> proj")
    dev = torch.device("cuda:0")
    lq = IQLinear(qkv.params)
    att = IQAttn((B, H, N, d), dict(att_w.params, out_layout=IQATTN_OUT_TOKENS))
    lp = IQLinear(proj.params)
    x = torch.from_numpy(qkv.x).to(dev)
    wq = torch.from_numpy(qkv.w).to(dev)
    wp = torch.from_numpy(proj.w).to(dev)
    q, k, v = lq.forward(x, wq)
    a = att.forward(q, k, v)                     # [B, N, H, d] = [B N, C] rows
    y = lp.forward(a.view(B * N, C), wp)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    for o in (lq, att, lp):
        o.close()
    # oracle chain
    P = qkv.params
    parts = [oracle.linear(qkv.x, qkv.w[i * C:(i + 1) * C], P["b"][i], P["c"][i]) for i in range(3)]
    heads = [t.reshape(B, N, H, d).transpose(0, 2, 1, 3).copy() for t in parts]
    o = oracle.forward(heads[0], heads[1], heads[2], att_w.params)
    tok = o.reshape(B, H, N, d).transpose(0, 2, 1, 3).reshape(B * N, C)
    ref = oracle.linear(tok, proj.w, proj.params["b"][0], proj.params["c"][0])
    assert np.array_equal(got, ref)
