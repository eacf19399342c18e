"""Seeded synthetic workloads for the integer-only attention core.

This module draws random numbers and shapes them into int8 Q/K/V tensors,
dyadic parameter pairs and bias tables. It performs none of the attention
arithmetic: the HIP path and the CPU oracle both consume its output, and
neither depends on the other.

Generator definition (one definition, used everywhere):
  * SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014), used counter-based: output i of stream
    (seed, sid) is mix64(state0 + (i + 1) * 0x9E3779B97F4A7C15) with
    state0 = mix64(seed * 0x100000001B3 + sid * 0x9E3779B97F4A7C15 + 1).
  * Uniform in (0, 1]: ((x >> 11) + 1) * 2^-53.
  * Normal by Box-Muller from two consecutive uniforms (u1, u2):
    z = sqrt(-2 ln u1) * cos(2 pi u2).
  * Integer in [lo, hi]: lo + floor(((x >> 11) * 2^-53) * (hi - lo + 1)).
  * int8 value: clip(round_half_away_from_zero(sigma * z), -127, 127)
    (the symmetric int8 range of the uniform symmetric quantiser).
  * Tensors are filled in [B, H, N, d] row-major order.

Workload shapes and distributions are those of the five attention shapes the
method is evaluated on (DeiT-Tiny/Small, ViT-B/DeiT-B, Swin-S stage-1 windows,
ViT-L at 384 px with Log-Int-Softmax).  They stand in for ImageNet/COCO
activations of trained models, which are not available here.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

_GOLDEN = 0x9E3779B97F4A7C15
_MASK64 = (1 << 64) - 1
_CHUNK = 1 << 22

# Stream ids (one independent SplitMix64 stream per use).
S_Q, S_K, S_V, S_PARAMS, S_SIGMA, S_OUTLIER, S_BIAS = 1, 2, 3, 4, 5, 6, 7
S_X, S_W, S_LPARAMS = 8, 9, 10

SHIFTMAX = 0
LIS = 1


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


class Stream:
    """Counter-based SplitMix64 stream keyed by (seed, stream id)."""

    def __init__(self, seed: int, sid: int):
        key = (seed * 0x100000001B3 + sid * _GOLDEN + 1) & _MASK64
        self._state0 = np.uint64(int(_mix64(np.array([key], np.uint64))[0]))
        self._pos = 0

    def u64(self, n: int) -> np.ndarray:
        idx = np.arange(self._pos + 1, self._pos + n + 1, dtype=np.uint64)
        self._pos += n
        with np.errstate(over="ignore"):
            return _mix64(self._state0 + idx * np.uint64(_GOLDEN))

    def uniform01(self, n: int) -> np.ndarray:
        """Uniform doubles in (0, 1]."""
        return ((self.u64(n) >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)

    def uniform_co(self, n: int) -> np.ndarray:
        """Uniform doubles in [0, 1)."""
        return (self.u64(n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)

    def randint(self, lo: int, hi: int, n: int) -> np.ndarray:
        """Integers uniform in [lo, hi] (inclusive)."""
        u = self.uniform_co(n)
        return (lo + np.floor(u * (hi - lo + 1))).astype(np.int64)

    def normal(self, n: int) -> np.ndarray:
        u = self.uniform01(2 * n).reshape(n, 2)
        return np.sqrt(-2.0 * np.log(u[:, 0])) * np.cos(2.0 * np.pi * u[:, 1])


def _round_half_away(x: np.ndarray) -> np.ndarray:
    return np.sign(x) * np.floor(np.abs(x) + 0.5)


def int8_gaussian(stream: Stream, shape, sigma) -> np.ndarray:
    """clip(round(sigma * N(0,1)), -127, 127) as int8, filled row-major.

    `sigma` is a scalar or an array broadcastable to `shape`.
    """
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.int8)
    sig = np.broadcast_to(np.asarray(sigma, dtype=np.float64), shape).reshape(-1) \
        if np.ndim(sigma) else None
    for s in range(0, total, _CHUNK):
        n = min(_CHUNK, total - s)
        z = stream.normal(n)
        scale = sig[s:s + n] if sig is not None else float(sigma)
        out[s:s + n] = np.clip(_round_half_away(scale * z), -127, 127).astype(np.int8)
    return out.reshape(shape)


@dataclass
class Workload:
    """One batch of int8 attention inputs plus the integer parameters."""
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    params: Dict[str, object] = field(default_factory=dict)

    @property
    def n_heads_total(self) -> int:
        return self.batch * self.heads


def default_params(seed: int, variant: int = SHIFTMAX) -> Dict[str, object]:
    """Dyadic pairs and Shiftmax/LIS constants for one workload.

    b1, b2 uniform integers in [2^14, 2^15); c1 = 22, c2 = 20 (LIS: c2 = 28,
    i.e. 20 + 15 - 7, so that the LIS output scale matches the Shiftmax one).
    I0 = 16, 8 extra exponent fraction bits, M = 30, k_out = 8, 4-bit LIS codes.
    """
    st = Stream(seed, S_PARAMS)
    b = st.randint(1 << 14, (1 << 15) - 1, 2)
    return dict(qk_b=int(b[0]), qk_c=22, pv_b=int(b[1]),
                pv_c=28 if variant == LIS else 20,
                i0=16, exp_frac_bits=8, intdiv_m=30, k_out=8,
                variant=variant, lis_bits=4, lis_engine=0, window=0, rel_bias=None)


def make_workload(batch: int, heads: int, seq_len: int, head_dim: int, seed: int,
                  sigma=24.0, variant: int = SHIFTMAX, name: str = "custom",
                  per_head_sigma: Optional[tuple] = None, k_outlier_p: float = 0.0,
                  window: int = 0, bias_range: int = 512) -> Workload:
    shape = (batch, heads, seq_len, head_dim)
    if per_head_sigma is not None:
        lo, hi = per_head_sigma
        sig_h = lo + (hi - lo) * Stream(seed, S_SIGMA).uniform_co(heads)
        sigma = sig_h.reshape(1, heads, 1, 1)
    q = int8_gaussian(Stream(seed, S_Q), shape, sigma)
    k = int8_gaussian(Stream(seed, S_K), shape, sigma)
    v = int8_gaussian(Stream(seed, S_V), shape, sigma)
    if k_outlier_p > 0.0:
        rows = Stream(seed, S_OUTLIER).uniform_co(batch * heads * seq_len)
        sel = (rows < k_outlier_p).reshape(batch, heads, seq_len)
        k3 = np.clip(k.astype(np.int16) * 3, -127, 127).astype(np.int8)
        k = np.where(sel[..., None], k3, k)
    params = default_params(seed, variant)
    if window:
        span = (2 * window - 1) ** 2
        t = Stream(seed, S_BIAS).randint(-bias_range, bias_range, heads * span)
        params["window"] = window
        params["rel_bias"] = t.astype(np.int32).reshape(heads, span)
    return Workload(name, batch, heads, seq_len, head_dim,
                    np.ascontiguousarray(q), np.ascontiguousarray(k),
                    np.ascontiguousarray(v), params)


# The five workload shapes.  Seed 1000 + k gives the headline inputs of shape k.
CONFIGS = {
    0: dict(name="deit_tiny_b1_h3_n197_d64", batch=1, heads=3, seq_len=197, head_dim=64),
    1: dict(name="deit_small_b64_h6_n197_d64", batch=64, heads=6, seq_len=197, head_dim=64),
    2: dict(name="vitb_b128_h12_n197_d64", batch=128, heads=12, seq_len=197, head_dim=64,
            per_head_sigma=(8.0, 40.0), k_outlier_p=0.05),
    3: dict(name="swin_s_stage1_2048win_h3_n49_d32_relbias", batch=32 * 64, heads=3,
            seq_len=49, head_dim=32, window=7),
    4: dict(name="vitl384_b32_h16_n577_d64_lis", batch=32, heads=16, seq_len=577,
            head_dim=64, variant=LIS),
}


def config_workload(cfg: int, seed: Optional[int] = None) -> Workload:
    spec = dict(CONFIGS[cfg])
    if seed is None:
        seed = 1000 + cfg
    return make_workload(seed=seed, **spec)


def config_shape(cfg: int):
    s = CONFIGS[cfg]
    return s["batch"], s["heads"], s["seq_len"], s["head_dim"]


# ---------------------------------------------------------------- linear layers
@dataclass
class LinearWorkload:
    """int8 activations x [rows, in], weights w [out, in] and the layer's
    parameters (a dict accepted by iqattn.IQLinear)."""
    name: str
    x: np.ndarray
    w: np.ndarray
    params: Dict[str, object] = field(default_factory=dict)


def make_linear(rows: int, in_features: int, out_features: int, seed: int, sigma_x=24.0,
                sigma_w=24.0, qkv_heads: Optional[tuple] = None, name: str = "linear",
                target_sigma=32.0) -> LinearWorkload:
    """Seeded int8 x and w (clipped Gaussians) and dyadic pairs: b uniform in
    [2^14, 2^15), c chosen so that b / 2^c maps the accumulator's standard
    deviation sqrt(in) * sigma_x * sigma_w to about target_sigma.
    qkv_heads = (batch, seq_len, heads, head_dim) selects the head-split layout
    (out = 3 * heads * head_dim, one pair per Q, K, V)."""
    x = int8_gaussian(Stream(seed, S_X), (rows, in_features), sigma_x)
    w = int8_gaussian(Stream(seed, S_W), (out_features, in_features), sigma_w)
    st = Stream(seed, S_LPARAMS)
    npairs = 3 if qkv_heads else 1
    b = st.randint(1 << 14, (1 << 15) - 1, npairs)
    sd = float(np.sqrt(in_features)) * sigma_x * sigma_w
    c = [int(np.ceil(np.log2(float(bi) * sd / target_sigma))) for bi in b]
    params = dict(rows=rows, in_features=in_features, out_features=out_features,
                  layout=0, batch=0, seq_len=0, heads=0, head_dim=0,
                  b=tuple(int(v) for v in b), c=tuple(c))
    if qkv_heads:
        B, N, H, d = qkv_heads
        params.update(layout=1, batch=B, seq_len=N, heads=H, head_dim=d)
    return LinearWorkload(name, np.ascontiguousarray(x), np.ascontiguousarray(w), params)


# ViT-B projections at the headline batch: Q/K/V (head-split) and the output one
LINEAR_CONFIGS = {
    "vitb_qkv_b128_n197_c768": dict(rows=128 * 197, in_features=768, out_features=3 * 768,
                                     qkv_heads=(128, 197, 12, 64)),
    "vitb_proj_b128_n197_c768": dict(rows=128 * 197, in_features=768, out_features=768),
}


def linear_workload(name: str, seed: int = 2000) -> LinearWorkload:
    spec = dict(LINEAR_CONFIGS[name])
    return make_linear(seed=seed, name=name, **spec)


# ---------------------------------------------------------------- ShiftGELU / I-LayerNorm
S_G, S_GPARAMS, S_LNX, S_LNMU, S_LNSIG, S_GAMMA, S_BETA, S_LNPARAMS = 11, 12, 13, 14, 15, 16, 17, 18


@dataclass
class GeluWorkload:
    """int8 input of the MLP's GELU, x [rows, cols], plus its parameters."""
    name: str
    rows: int
    cols: int
    x: np.ndarray
    params: Dict[str, int] = field(default_factory=dict)


def gelu_params(seed: int) -> Dict[str, int]:
    """Input scale 1/16 (I0 = 16), 22 extra exponent fraction bits, M = 40,
    k_out = 8; output pair b uniform in [2^14, 2^15), c = 22: b / 2^c in
    [1/256, 1/128) maps x * sigma (scale 1/(16 * 128)) to an output scale in
    (1/16, 1/8], wide enough for the largest input, 127/16."""
    b = Stream(seed, S_GPARAMS).randint(1 << 14, (1 << 15) - 1, 1)
    return dict(i0=16, exp_frac_bits=22, intdiv_m=40, k_out=8, b=int(b[0]), c=22)


def make_gelu(rows: int, cols: int, seed: int, sigma=32.0, name: str = "custom") -> GeluWorkload:
    x = int8_gaussian(Stream(seed, S_G), (rows, cols), sigma)
    return GeluWorkload(name, rows, cols, x, gelu_params(seed))


@dataclass
class LayerNormWorkload:
    """int8 input of a LayerNorm, x [rows, cols], int8 gamma and int32 beta per
    column, plus its parameters."""
    name: str
    rows: int
    cols: int
    x: np.ndarray
    gamma: np.ndarray
    beta: np.ndarray
    params: Dict[str, int] = field(default_factory=dict)


def layernorm_params(seed: int) -> Dict[str, int]:
    """7 fraction bits on the normalised value, M = 22 for floor(2^M / sd);
    output pair b uniform in [2^14, 2^15), c = 22."""
    b = Stream(seed, S_LNPARAMS).randint(1 << 14, (1 << 15) - 1, 1)
    return dict(norm_frac_bits=7, intdiv_m=22, b=int(b[0]), c=22)


def make_layernorm(rows: int, cols: int, seed: int, name: str = "custom",
                   mu_sigma=12.0, sigma_range=(8.0, 40.0), gamma_sigma=48.0,
                   beta_range=1 << 14) -> LayerNormWorkload:
    """LayerNorm inputs with inter-channel variation: column j has its own mean
    mu_j ~ N(0, mu_sigma) and spread sigma_j uniform in sigma_range; element
    x[m, j] = clip(round(mu_j + sigma_j * z), -127, 127).  gamma is int8
    N(0, gamma_sigma), beta uniform in [-beta_range, beta_range]."""
    mu = mu_sigma * Stream(seed, S_LNMU).normal(cols)
    lo, hi = sigma_range
    sg = lo + (hi - lo) * Stream(seed, S_LNSIG).uniform_co(cols)
    z = Stream(seed, S_LNX).normal(rows * cols).reshape(rows, cols)
    x = np.clip(_round_half_away(mu[None, :] + sg[None, :] * z), -127, 127).astype(np.int8)
    gamma = int8_gaussian(Stream(seed, S_GAMMA), (cols,), gamma_sigma)
    beta = Stream(seed, S_BETA).randint(-beta_range, beta_range, cols).astype(np.int32)
    return LayerNormWorkload(name, rows, cols, x, gamma, beta, layernorm_params(seed))


# ViT-B/16 at 224 px, batch 128: 197 tokens, hidden 768, MLP 3072.
GELU_CONFIGS = {"vitb_mlp_b128_n197_c3072": (128 * 197, 3072)}
LAYERNORM_CONFIGS = {"vitb_ln_b128_n197_c768": (128 * 197, 768)}


def gelu_workload(name: str, seed: int = 3000) -> GeluWorkload:
    rows, cols = GELU_CONFIGS[name]
    return make_gelu(rows, cols, seed, name=name)


def layernorm_workload(name: str, seed: int = 4000) -> LayerNormWorkload:
    rows, cols = LAYERNORM_CONFIGS[name]
    return make_layernorm(rows, cols, seed, name=name)


# ---------------------------------------------------------------- linear attention
S_LQ, S_LK, S_LV, S_LAPARAMS = 19, 20, 21, 22


def linattn_params(seed: int, seq_len: int, head_dim: int, sigma=24.0) -> Dict[str, int]:
    """Dyadic pairs for the softmax-free linear attention, from the input
    distribution only (sigma of Q, K, V; N tokens; d features):
      KV entries have std ~ sqrt(N) * (sigma / sqrt 2) * sigma  -> int8 std ~ 32;
      ks entries have mean ~ 0.4 * sigma * N                    -> int8 ~ 96;
      num ~ sqrt(d) * (sigma / sqrt 2) * 32, den ~ d * 0.4 * sigma * 96, and the
      output pair maps num / den to an int8 std of about 32.
    Each b is uniform in [2^14, 2^15); each c the exponent that gives the target."""
    import math
    b = Stream(seed, S_LAPARAMS).randint(1 << 14, (1 << 15) - 1, 3)
    half = sigma / math.sqrt(2.0)
    kv_std = math.sqrt(seq_len) * half * sigma
    ks_mean = 0.4 * sigma * seq_len
    num_std = math.sqrt(head_dim) * half * 32.0
    den = head_dim * 0.4 * sigma * 96.0
    c_kv = max(0, round(math.log2(b[0] * kv_std / 32.0)))
    c_ks = max(0, math.ceil(math.log2(b[1] * ks_mean / 96.0)))
    c_out = max(0, round(math.log2(b[2] * num_std / (den * 32.0))))
    return dict(kv_b=int(b[0]), kv_c=c_kv, ks_b=int(b[1]), ks_c=c_ks, out_b=int(b[2]), out_c=c_out)


def make_linattn(batch: int, heads: int, seq_len: int, head_dim: int, seed: int, sigma=24.0,
                 name: str = "custom") -> Workload:
    shape = (batch, heads, seq_len, head_dim)
    q = int8_gaussian(Stream(seed, S_LQ), shape, sigma)
    k = int8_gaussian(Stream(seed, S_LK), shape, sigma)
    v = int8_gaussian(Stream(seed, S_LV), shape, sigma)
    return Workload(name, batch, heads, seq_len, head_dim, q, k, v,
                    linattn_params(seed, seq_len, head_dim, sigma))


# EfficientViT-style ReLU attention at stage 3 (16-pixel tokens): 224 px -> 196
# tokens, 512 px -> 1024 tokens; head dim 16 (B1-like) and 32 (B3-like), the
# heads doubled by the multi-scale branch.
LINATTN_CONFIGS = {
    "effvit_b64_h16_n196_d16": (64, 16, 196, 16),
    "effvit_b64_h16_n1024_d16": (64, 16, 1024, 16),
    "effvit_b16_h32_n1024_d32": (16, 32, 1024, 32),
}


def linattn_workload(name: str, seed: int = 5000) -> Workload:
    B, H, N, d = LINATTN_CONFIGS[name]
    return make_linattn(B, H, N, d, seed, name=name)
