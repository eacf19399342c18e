"""Every sequence length the header allows, on every back end: a context can
be created for each (the kernel choice and its LDS plan fit the device), and
one length per 16-key tile count runs byte-exact against the oracle, so every
specialised instance and the generic kernel around them are exercised."""
import sys

import numpy as np
import pytest

import oracle
from integer_only_quantized_int8_amd import workloads as W

pytestmark = pytest.mark.gpu

ENGINES = [(0, 0), (1, 0), (1, 1)]  # (variant, lis_engine): Shiftmax, LIS VALU, LIS MFMA


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "no GPU visible"
    return torch


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("variant,engine", ENGINES)
def test_create_every_length(torch_dev, d, variant, engine):
    from integer_only_quantized_int8_amd.iqattn import IQAttn
    _say(f"[coverage] create N = 1..640, d = {d}, variant {variant}, engine {engine}")
    params = dict(W.default_params(5, variant), lis_engine=engine)
    for n in range(1, 641):
        att = IQAttn((1, 2, n, d), params)
        att.close()


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("variant,engine", ENGINES)
def test_every_tile_count(torch_dev, d, variant, engine):
    from integer_only_quantized_int8_amd.iqattn import IQAttn
    torch = torch_dev
    dev = torch.device("cuda:0")
    for kt in range(1, 41):
        n = 16 * kt - (kt % 3) * 5  # full last tiles and ragged ones
        w = W.make_workload(1, 2, n, d, seed=900 + kt, variant=variant)
        params = dict(w.params, lis_engine=engine)
        _say(f"[coverage] N = {n} (KT = {kt}), d = {d}, variant {variant}, engine {engine}")
        att = IQAttn(w.q.shape, params)
        q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
        out = torch.full_like(q, 99)
        att.forward(q, k, v, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(2, n, d)
        att.close()
        ref = oracle.forward(w.q, w.k, w.v, params)
        assert np.array_equal(got, ref), f"N = {n}: {np.argwhere(got != ref)[:4].tolist()}"


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("variant,engine", ENGINES)
def test_every_window_with_bias(torch_dev, d, variant, engine):
    """Windowed attention with the relative-position bias for every window
    w = 1..25 (N = w^2), byte-exact, Shiftmax and both LIS engines."""
    from integer_only_quantized_int8_amd.iqattn import IQAttn
    torch = torch_dev
    dev = torch.device("cuda:0")
    for win in range(1, 26):
        w = W.make_workload(2, 2, win * win, d, seed=950 + win, window=win, variant=variant)
        _say(f"[coverage] window {win} (N = {win * win}), d = {d}, bias, variant {variant}, "
             f"engine {engine}")
        att = IQAttn(w.q.shape, dict(w.params, lis_engine=engine))
        q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
        out = torch.full_like(q, 99)
        att.forward(q, k, v, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(4, win * win, d)
        att.close()
        ref = oracle.forward(w.q, w.k, w.v, dict(w.params, lis_engine=engine))
        assert np.array_equal(got, ref), f"window {win}: {np.argwhere(got != ref)[:4].tolist()}"
