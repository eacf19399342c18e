"""Pins of the oracle's softmax-free integer linear attention (CPU).

The two token sums (Trio-ViT's steps i and ii) are pinned to numpy's int64
matrix product and sum; the shift division to float64 Eq. 4 within the bound
the log2 divisor allows (a divisor X and its code L = ilog2r(X) satisfy
0.75 <= X / 2^L < 1.5); the token sums to their invariance under a joint
permutation of K and V; closed forms (ReLU(Q) = 0, one token); tiny shapes to
the brute-force evaluator.
"""
import numpy as np
import pytest

import bruteforce as BF
import oracle
from integer_only_quantized_int8_amd import workloads as W


def _exact_requant(x, b, c):
    return np.array([max(-127, min(127, (int(b) * int(v)) >> c)) for v in x.ravel()],
                    dtype=np.int64).reshape(x.shape)


def test_token_sums_match_numpy():
    wl = W.make_linattn(2, 3, 97, 16, seed=1)
    _, dm = oracle.linattn(wl.q, wl.k, wl.v, wl.params, dump=True)
    P = wl.params
    kr = np.maximum(wl.k.astype(np.int64), 0).reshape(6, 97, 16)
    vv = wl.v.astype(np.int64).reshape(6, 97, 16)
    for h in range(6):
        kv = kr[h].T @ vv[h]
        ks = kr[h].sum(axis=0)
        assert np.array_equal(dm[h, :256].reshape(16, 16), _exact_requant(kv, P["kv_b"], P["kv_c"]))
        assert np.array_equal(dm[h, 256:], _exact_requant(ks, P["ks_b"], P["ks_c"]))
    # the workload's pairs keep the sums inside int8 without mass clipping
    assert np.abs(dm[:, :256]).std() > 10 and (np.abs(dm[:, :256]) == 127).mean() < 0.05
    assert dm[:, 256:].min() > 30 and (dm[:, 256:] == 127).mean() < 0.2


@pytest.mark.parametrize("shape", [(1, 4, 196, 16), (1, 2, 1024, 32), (2, 2, 50, 64)])
def test_shift_division_within_log2_bound_of_eq4(shape):
    """Against float64 Eq. 4 on the requantised sums: (out_b / 2^out_c) num / den
    before the floor; the integer output lies within [0.75, 1.5) of it (the
    divisor's code), minus the floor."""
    B, H, N, d = shape
    wl = W.make_linattn(B, H, N, d, seed=N + d)
    out, dm = oracle.linattn(wl.q, wl.k, wl.v, wl.params, dump=True)
    P = wl.params
    qr = np.maximum(wl.q.astype(np.float64), 0).reshape(B * H, N, d)
    o = out.reshape(B * H, N, d).astype(np.float64)
    checked = 0
    for h in range(B * H):
        kvq = dm[h, :d * d].reshape(d, d).astype(np.float64)
        ksq = dm[h, d * d:].astype(np.float64)
        num = qr[h] @ kvq
        den = qr[h] @ ksq
        ok = den > 0
        ref = P["out_b"] / 2.0 ** P["out_c"] * num[ok] / den[ok, None]
        got = o[h][ok]
        lo = np.minimum(0.75 * ref, 1.5 * ref) - 1
        hi = np.maximum(0.75 * ref, 1.5 * ref) + 1e-9
        inside = np.abs(ref) * 1.5 < 127
        assert np.all((got >= lo) & (got <= hi) | ~inside)
        checked += inside.sum()
        assert np.all(o[h][~ok] == 0)
    assert checked > 0
    # a wrong code (one step off) leaves the bound on most entries
    assert (np.abs(o) > 4).mean() > 0.3


def test_joint_token_permutation_and_query_independence():
    wl = W.make_linattn(1, 2, 120, 16, seed=4)
    out = oracle.linattn(wl.q, wl.k, wl.v, wl.params)
    perm = np.random.default_rng(3).permutation(120)
    out2 = oracle.linattn(wl.q, wl.k[:, :, perm], wl.v[:, :, perm], wl.params)
    assert np.array_equal(out, out2)
    qp = np.random.default_rng(5).permutation(120)
    out3 = oracle.linattn(wl.q[:, :, qp], wl.k, wl.v, wl.params)
    assert np.array_equal(out3, out[:, :, qp])
    single = oracle.linattn(wl.q[:, 1:], wl.k[:, 1:], wl.v[:, 1:], wl.params)
    assert np.array_equal(single[0, 0], out[0, 1])


def test_closed_forms():
    P = dict(kv_b=1, kv_c=0, ks_b=1, ks_c=0, out_b=1, out_c=0)
    rng = np.random.default_rng(8)
    k = rng.integers(-127, 128, (1, 1, 9, 16)).astype(np.int8)
    v = rng.integers(-127, 128, (1, 1, 9, 16)).astype(np.int8)
    q = -np.abs(rng.integers(0, 128, (1, 1, 9, 16))).astype(np.int8)  # ReLU(Q) = 0
    assert np.all(oracle.linattn(q, k, v, P) == 0)
    # one token, unit pairs: KV = relu(k) v^T clipped, ks = relu(k) clipped;
    # q = e_a picks row a: num = KVq[a], den = ksq[a]
    k1 = np.zeros((1, 1, 1, 16), np.int8); k1[..., 3] = 5
    v1 = np.arange(-8, 8, dtype=np.int8).reshape(1, 1, 1, 16) * 3
    q1 = np.zeros((1, 1, 1, 16), np.int8); q1[..., 3] = 1
    out = oracle.linattn(q1, k1, v1, P)[0, 0, 0]
    # den = 5 -> code ilog2r(5) = 2 + bit1(5)=0 -> 2; num = 5 * v
    assert list(out) == [int(np.floor(5 * int(x) / 4)) for x in v1.ravel()]


@pytest.mark.parametrize("shape,p", [
    ((1, 2, 5, 16), dict(kv_b=20000, kv_c=20, ks_b=20000, ks_c=12, out_b=20000, out_c=8)),
    ((1, 1, 33, 32), dict(kv_b=99, kv_c=9, ks_b=7, ks_c=4, out_b=12345, out_c=3)),
    ((2, 1, 3, 16), dict(kv_b=(1 << 31) - 1, kv_c=45, ks_b=1, ks_c=0, out_b=1, out_c=0)),
])
def test_tiny_against_brute_force(shape, p):
    rng = np.random.default_rng(sum(shape))
    q, k, v = (rng.integers(-128, 128, shape).astype(np.int8) for _ in range(3))
    out = oracle.linattn(q, k, v, p)
    B, H, N, d = shape
    for b in range(B):
        for h in range(H):
            ref = BF.linattn_head(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), p)
            assert out[b, h].tolist() == ref


def test_parameter_validation():
    q = np.zeros((1, 1, 4, 16), np.int8)
    P = dict(kv_b=1, kv_c=0, ks_b=1, ks_c=0, out_b=1, out_c=0)
    for bad in (dict(kv_b=0), dict(ks_c=63), dict(out_c=-1), dict(out_b=0)):
        with pytest.raises(ValueError):
            oracle.linattn(q, q, q, dict(P, **bad))
