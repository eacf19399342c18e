"""HIP-graph capture and replay of every entry point.

A graph holding two launches of an operator (different inputs, separate
outputs) is replayed several times, with eager work (a fill kernel over the
outputs, an eager launch of the same operator) and host synchronisation
between the replays; every replay must give the eager result byte for byte,
and the eager result must equal the oracle.  The kernels keep all their
scheduling state (work queues, stage counters) in LDS and take every
parameter by value, so a replay has nothing to reset."""
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


def replay_check(torch, launch, outs, label, reps=4):
    """launch() enqueues the operator's launches (writing outs) on the
    current stream."""
    launch()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    for rep in range(reps):
        for o in outs:
            o.fill_(99)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"{label}: replay {rep}, output {i} differs from eager"
        launch()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"{label}: eager launch after replay {rep}, output {i}"
    del graph
    return ref


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.device("cuda:0"))


@pytest.mark.parametrize("cfg,engine", [(0, None), (3, None), (4, 0), (4, 1)])
def test_graph_attention(torch_dev, cfg, engine):
    from integer_only_quantized_int8_amd.iqattn import IQAttn
    torch = torch_dev
    spec = dict(W.CONFIGS[cfg])
    spec["batch"] = {0: 1, 3: 2, 4: 1}[cfg]
    if cfg == 4:
        spec["heads"] = 2
    ws = [W.make_workload(seed=s, **spec) for s in (11, 12)]
    params = ws[0].params if engine is None else dict(ws[0].params, lis_engine=engine)
    _say(f"[graph] attention shape {cfg} engine {engine} {ws[0].q.shape}")
    att = IQAttn(ws[0].q.shape, params)
    ins = [tuple(_dev(torch, t) for t in (w.q, w.k, w.v)) for w in ws]
    outs = [torch.empty_like(i[0]) for i in ins]

    def launch():
        for (q, k, v), o in zip(ins, outs):
            att.forward(q, k, v, o)

    got = replay_check(torch, launch, outs, f"attention shape {cfg}")
    for w, g in zip(ws, got):
        # every head against the oracle (same parameters: the pairs are per call)
        ref = oracle.forward(w.q, w.k, w.v, params)
        total = w.batch * w.heads
        assert np.array_equal(g.cpu().numpy().reshape(total, w.seq_len, w.head_dim), ref)
    att.close()


def test_graph_linear(torch_dev):
    from integer_only_quantized_int8_amd.iqattn import IQLinear
    torch = torch_dev
    B, N, H, d = 2, 197, 4, 64
    qkv = W.make_linear(B * N, 256, 3 * H * d, seed=5, qkv_heads=(B, N, H, d))
    plain = W.make_linear(300, 256, 192, seed=6)
    _say("[graph] linear qkv + plain")
    lq, lp = IQLinear(qkv.params), IQLinear(plain.params)
    xq, wq = _dev(torch, qkv.x), _dev(torch, qkv.w)
    xp, wp = _dev(torch, plain.x), _dev(torch, plain.w)
    shape = (B, H, N, d)
    oq = tuple(torch.empty(shape, dtype=torch.int8, device="cuda:0") for _ in range(3))
    op = torch.empty((300, 192), dtype=torch.int8, device="cuda:0")

    def launch():
        lq.forward(xq, wq, oq)
        lp.forward(xp, wp, op)

    got = replay_check(torch, launch, list(oq) + [op], "linear")
    P = plain.params
    assert np.array_equal(got[3].cpu().numpy(), oracle.linear(plain.x, plain.w, P["b"][0], P["c"][0]))
    P = qkv.params
    C3 = 3 * H * d // 3
    for i in range(3):
        ref = oracle.linear(qkv.x, qkv.w[i * C3:(i + 1) * C3], P["b"][i], P["c"][i])
        g = got[i].cpu().numpy().transpose(0, 2, 1, 3).reshape(B * N, H * d)
        assert np.array_equal(g, ref), f"tensor {i}"
    lq.close()
    lp.close()


def test_graph_gelu_and_layernorm(torch_dev):
    from integer_only_quantized_int8_amd.iqattn import IQGelu, IQLayerNorm
    torch = torch_dev
    gw = W.make_gelu(197, 3072, seed=21)
    lw = W.make_layernorm(197, 768, seed=22)
    _say("[graph] gelu + layernorm")
    ge = IQGelu(dict(gw.params, rows=197, cols=3072))
    ln = IQLayerNorm(dict(lw.params, rows=197, cols=768))
    gx = _dev(torch, gw.x)
    lx, lg, lb = _dev(torch, lw.x), _dev(torch, lw.gamma), _dev(torch, lw.beta)
    go = torch.empty_like(gx)
    lo = torch.empty_like(lx)

    def launch():
        ge.forward(gx, go)
        ln.forward(lx, lg, lb, lo)

    got = replay_check(torch, launch, [go, lo], "gelu + layernorm")
    assert np.array_equal(got[0].cpu().numpy(), oracle.shiftgelu(gw.x, gw.params))
    assert np.array_equal(got[1].cpu().numpy(), oracle.ilayernorm(lw.x, lw.gamma, lw.beta, lw.params))
    ge.close()
    ln.close()


def test_graph_linear_attention(torch_dev):
    from integer_only_quantized_int8_amd.iqattn import IQLinAttn
    torch = torch_dev
    wl = W.make_linattn(2, 4, 196, 16, seed=31)
    _say(f"[graph] linear attention {wl.q.shape}")
    op = IQLinAttn(wl.q.shape, wl.params)
    q, k, v = (_dev(torch, t) for t in (wl.q, wl.k, wl.v))
    out = torch.empty_like(q)

    def launch():
        op.forward(q, k, v, out)

    got = replay_check(torch, launch, [out], "linear attention")
    assert np.array_equal(got[0].cpu().numpy(), oracle.linattn(wl.q, wl.k, wl.v, wl.params))
    op.close()


def test_one_context_on_two_streams(torch_dev):
    """A context is immutable after create: launches of one context on two
    streams at once (different inputs, separate outputs) give the results of
    sequential launches."""
    from integer_only_quantized_int8_amd.iqattn import IQAttn, IQLinear
    torch = torch_dev
    ws = [W.make_workload(seed=s, **dict(W.CONFIGS[0], batch=4)) for s in (41, 42)]
    att = IQAttn(ws[0].q.shape, ws[0].params)
    lw = [W.make_linear(500, 256, 384, seed=s) for s in (43, 44)]
    lin = IQLinear(lw[0].params)
    ins = [tuple(_dev(torch, t) for t in (w.q, w.k, w.v)) for w in ws]
    lins = [(_dev(torch, w.x), _dev(torch, w.w)) for w in lw]
    seq = []
    for (q, k, v), (x, w) in zip(ins, lins):
        seq.append((att.forward(q, k, v), lin.forward(x, w)))
    torch.cuda.synchronize()
    _say("[streams] one context, two streams")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [(torch.empty_like(i[0]), torch.empty((500, 384), dtype=torch.int8, device="cuda:0"))
            for i in ins]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for s, (q, k, v), (x, w), (oa, ol) in zip(streams, ins, lins, outs):
            with torch.cuda.stream(s):
                att.forward(q, k, v, oa)
                lin.forward(x, w, ol)
        torch.cuda.synchronize()
        for (ra, rl), (oa, ol) in zip(seq, outs):
            assert torch.equal(oa, ra) and torch.equal(ol, rl), f"repetition {rep}"
    att.close()
    lin.close()
