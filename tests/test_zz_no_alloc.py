"""iqattn_forward_noalloc (the entry point for callers that cannot allocate)
against iqattn_create + iqattn_forward with the same parameters: byte-equal
outputs on two calls in a row, the second with a smaller input, on every
kernel family (specialised, windowed bias in LDS, Log-Int-Softmax on both
engines, rows of 641+ keys, generic 64-bit requantisation, token-major
output), and inside a captured HIP graph.
"""
import sys

import numpy as np
import pytest

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


def _ctx_result(torch, w, params):
    from integer_only_quantized_int8_amd.iqattn import IQAttn, IQATTN_OK
    dev = torch.device("cuda:0")
    att = IQAttn(w.q.shape, params)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
    out = att.forward(q, k, v)
    torch.cuda.synchronize()
    assert att.check() == IQATTN_OK
    res = out.cpu().numpy()
    att.close()
    return res


CASES = [
    ("specialised", dict(batch=4, heads=12, seq_len=197, head_dim=64), {}),
    ("windowed bias", dict(batch=24, heads=3, seq_len=49, head_dim=32, window=7), {}),
    ("LIS VALU", dict(batch=1, heads=3, seq_len=577, head_dim=64, variant=1), dict(lis_engine=0)),
    ("LIS MFMA", dict(batch=1, heads=3, seq_len=577, head_dim=64, variant=1), dict(lis_engine=1)),
    ("long rows", dict(batch=1, heads=2, seq_len=700, head_dim=32), {}),
    ("generic", dict(batch=2, heads=3, seq_len=100, head_dim=64), dict(qk_b=(1 << 31) - 1, qk_c=40)),
    ("token-major", dict(batch=2, heads=4, seq_len=130, head_dim=64), dict(out_layout=1)),
]


@pytest.mark.parametrize("name,spec,over", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_context_path(torch_dev, name, spec, over):
    torch = torch_dev
    from integer_only_quantized_int8_amd.iqattn import iqattn_forward_noalloc
    dev = torch.device("cuda:0")
    big = W.make_workload(seed=101, **spec)
    small_spec = dict(spec, batch=max(1, spec["batch"] // 2))
    if spec["seq_len"] > 64 and not spec.get("window"):
        small_spec["seq_len"] = spec["seq_len"] - 37          # fewer keys too
    small = W.make_workload(seed=102, **small_spec)
    pb, ps = dict(big.params, **over), dict(small.params, **over)
    _say(f"[noalloc] {name}: {big.q.shape} then {small.q.shape}")
    refs = [_ctx_result(torch, big, pb), _ctx_result(torch, small, ps)]
    outs = []
    for w, p in ((big, pb), (small, ps)):
        q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
        out = torch.full_like(q, 99)
        iqattn_forward_noalloc(w.q.shape, p, q, k, v, out)      # no synchronisation between
        outs.append((q, k, v, out))
    torch.cuda.synchronize()
    for (q, k, v, out), ref in zip(outs, refs):
        got = out.cpu().numpy().reshape(ref.shape)
        assert np.array_equal(got, ref), f"{name}: {int((got != ref).sum())} bytes differ"


def test_noalloc_in_a_captured_graph(torch_dev):
    """Captured once, replayed three times with eager work in between: every
    replay equals the context path's result."""
    torch = torch_dev
    from integer_only_quantized_int8_amd.iqattn import iqattn_forward_noalloc
    dev = torch.device("cuda:0")
    w = W.make_workload(seed=103, batch=8, heads=3, seq_len=49, head_dim=32, window=7)
    ref = _ctx_result(torch, w, w.params)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
    out = torch.zeros_like(q)
    iqattn_forward_noalloc(w.q.shape, w.params, q, k, v, out)   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iqattn_forward_noalloc(w.q.shape, w.params, q, k, v, out)
    for rep in range(3):
        out.fill_(99)
        other = W.make_workload(seed=104 + rep, batch=2, heads=12, seq_len=197, head_dim=64)
        oq, ok, ov = (torch.from_numpy(x).to(dev) for x in (other.q, other.k, other.v))
        scratch_user = torch.empty_like(oq)
        iqattn_forward_noalloc(other.q.shape, other.params, oq, ok, ov, scratch_user)  # eager call
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref), f"replay {rep}"
