"""Brute-force evaluator of the integer attention pipeline, for tiny shapes.

Written independently of the C oracle with Python's unbounded integers and
exact rationals: every floor is math.floor of a Fraction, the q/r split is
divmod, the leading-one index is int.bit_length.  It pins the oracle's
integer mechanics (widths, shifts, signs, loops); the readings themselves are
pinned elsewhere (softmax bound, closed forms, worked examples).
"""
from fractions import Fraction
from math import floor


def fl(num, den=1):
    return floor(Fraction(num, den))


def requant(x, b, c):
    return max(-127, min(127, fl(b * x, 2 ** c)))


def shift_exp(delta, i0, n):
    ip = delta + fl(delta, 2) - fl(delta, 16)
    q, r = divmod(-ip, i0)
    mant = i0 + fl(-r, 2)
    return fl(mant * 2 ** n, 2 ** q)


def ilog2r(x):
    k = x.bit_length() - 1
    return k + ((x >> (k - 1)) & 1 if k >= 1 else 0)


def softmax_row(L, p):
    m = max(L)
    e = [shift_exp(x - m, p["i0"], p["exp_frac_bits"]) for x in L]
    s = sum(e)
    f = fl(2 ** p["intdiv_m"], s)
    if p["variant"] == 0:
        pmax = 2 ** (p["k_out"] - 1) - 1
        w = [min(fl(f * x, 2 ** (p["intdiv_m"] - p["k_out"] + 1)), pmax) for x in e]
        return e, w, None
    F = 2 ** p["lis_bits"] - 1
    ph = [fl(f * x, 2 ** (p["intdiv_m"] - F)) for x in e]
    codes = [F if v == 0 else max(0, min(F, F - ilog2r(v))) for v in ph]
    return e, [2 ** (F - c) for c in codes], codes


def attention(q, k, v, p):
    """q, k, v: nested lists / arrays [B][H][N][d] of ints.  Returns out."""
    B, H, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    w = p.get("window", 0) or 0
    out = [[[[0] * d for _ in range(N)] for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(N):
                L = []
                for j in range(N):
                    acc = sum(int(q[b][h][i][t]) * int(k[b][h][j][t]) for t in range(d))
                    if w:
                        dr = i // w - j // w
                        dc = i % w - j % w
                        acc += int(p["rel_bias"][h][(dr + w - 1) * (2 * w - 1) + dc + w - 1])
                    L.append(requant(acc, p["qk_b"], p["qk_c"]))
                _, wts, _ = softmax_row(L, p)
                for t in range(d):
                    o = sum(wts[j] * int(v[b][h][j][t]) for j in range(N))
                    out[b][h][i][t] = requant(o, p["pv_b"], p["pv_c"])
    return out


def shiftgelu_row(xs, p):
    """ShiftGELU (I-ViT sec. 3.4) of one row of ints."""
    ip = [x + fl(x, 2) + fl(x, 8) + fl(x, 16) for x in xs]
    imax = max([0] + ip)
    e2 = shift_exp(-imax, p["i0"], p["exp_frac_bits"])
    m, k = p["intdiv_m"], p["k_out"]
    out = []
    for x, v in zip(xs, ip):
        e1 = shift_exp(v - imax, p["i0"], p["exp_frac_bits"])
        sig = 0
        if e1:
            sig = min(fl(fl(2 ** m, e1 + e2) * e1, 2 ** (m - k + 1)), 2 ** (k - 1) - 1)
        out.append(requant(x * sig, p["b"], p["c"]))
    return out


def newton_isqrt10(v):
    if v <= 0:
        return 0
    r = 2 ** (v.bit_length() // 2)
    for _ in range(10):
        r = fl(r + fl(v, r), 2)
    return r


def ilayernorm_row(xs, gamma, beta, p):
    """I-LayerNorm (I-ViT sec. 3.5) of one row of ints."""
    n = len(xs)
    mean = fl(sum(xs), n)
    var = fl(sum((x - mean) ** 2 for x in xs), n)
    sd = newton_isqrt10(var) or 1
    m, f = p["intdiv_m"], p["norm_frac_bits"]
    fs = fl(2 ** m, sd)
    return [requant(fl((x - mean) * fs, 2 ** (m - f)) * int(g) + int(bt), p["b"], p["c"])
            for x, g, bt in zip(xs, gamma, beta)]


def linattn_head(Q, K, V, p):
    """Softmax-free linear attention of one head: Q, K, V nested [N][d] ints."""
    N, d = len(Q), len(Q[0])
    relu = lambda x: x if x > 0 else 0  # noqa: E731
    kvq = [[requant(sum(relu(K[j][a]) * V[j][b] for j in range(N)), p["kv_b"], p["kv_c"])
            for b in range(d)] for a in range(d)]
    ksq = [requant(sum(relu(K[j][a]) for j in range(N)), p["ks_b"], p["ks_c"]) for a in range(d)]
    out = []
    for i in range(N):
        qr = [relu(x) for x in Q[i]]
        den = sum(qr[a] * ksq[a] for a in range(d))
        L = ilog2r(den) if den > 0 else 0
        row = []
        for b in range(d):
            num = sum(qr[a] * kvq[a][b] for a in range(d))
            row.append(max(-127, min(127, fl(p["out_b"] * num, 2 ** (p["out_c"] + L)))))
        out.append(row)
    return out
