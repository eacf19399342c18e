"""Failure path of the kernels' bounded waits, forced from the host.

The specialised attention kernel's waves wait for their operands with bounded
polls (the linear layer's waves meet only at workgroup barriers).  A test-only spin
limit of one poll makes waves give up while their data is still on the way:
every kernel must still exit normally, the launch must be reported as
incomplete by the check call, and the next launch with the default limit
must be complete and exact again.
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


def test_attention_giveup_is_reported_and_recovers(torch_dev):
    torch = torch_dev
    from integer_only_quantized_int8_amd import iqattn as IQ
    # the headline shape: six whole heads per workgroup, so the loader wave
    # also waits for buffers to be released
    w = W.config_workload(2)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
    att = IQ.IQAttn(w.q.shape, w.params)
    out = torch.empty_like(q)
    _say("[status] attention, spin limit 1")
    IQ.iqattn_set_spin_limit(att.ctx, 1)
    att.forward(q, k, v, out)
    assert att.check() == IQ.IQATTN_E_INCOMPLETE
    assert att.check() == IQ.IQATTN_OK          # the check clears the word
    _say("[status] attention, default spin limit")
    IQ.iqattn_set_spin_limit(att.ctx, 1 << 22)
    out.fill_(99)
    att.forward(q, k, v, out)
    assert att.check() == IQ.IQATTN_OK
    got = out.cpu().numpy().reshape(-1, w.seq_len, w.head_dim)
    att.close()
    for lo, hi in ((0, 48), (1488, 1536)):
        ref = oracle.forward(w.q, w.k, w.v, w.params, heads=(lo, hi))
        assert np.array_equal(got[lo:hi], ref), (lo, hi)


def test_spin_limit_argument_checks(torch_dev):
    from integer_only_quantized_int8_amd import iqattn as IQ
    w = W.make_workload(1, 2, 33, 64, seed=3)
    att = IQ.IQAttn(w.q.shape, w.params)
    with pytest.raises(IQ.IQAttnError) as ei:
        IQ.iqattn_set_spin_limit(att.ctx, 0)
    assert ei.value.code == IQ.IQATTN_E_INVAL
    att.close()
