"""Seeded synthetic inputs for the DSpark draft / verify / schedule path.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no softmax, no sampling, no acceptance test, no scheduling),
so both the fp64 oracle and the HIP library can be fed from it without sharing
any of the computation they are compared on.

Every stream is ``numpy.random.Generator(PCG64(SeedSequence([seed, tensor, *extra])))``,
where ``seed`` is the workload's seed id.
Large per-request tensors use ``extra = [b]`` so one request's rows can be
regenerated alone (the oracle checks sampled requests at full size that way).

Shapes and distributions follow the five workloads of the hot path (seed ids 1 .. 5):

* TINY - B=4, V=1024, r=32, gamma=4, fp32 factors. U ~ N(0, 2^2), W1, W2 ~ N(0, 0.05^2),
  target noise sigma = 0.5.
* SINGLE - B=1, V=151936, r=256, gamma=7, bf16 factors ~ N(0, 0.02^2); U ~ N(0, 3^2) with
  32 distinct ids per row raised by +8.
* BATCHED - as SINGLE with B=64, gamma=16.
* VERIFY - verify only: B=256, gamma=16, V=151936; draft logits as SINGLE's U; target =
  draft + N(0, sigma_k^2) with sigma_k from ``tests/golden/target_sigma.json``.
* ROUND - full round: R=B=512, gamma=16, V=129280, r=256, bf16; confidences
  Beta(8,2) * 0.97^k, temperatures 0.8 .. 1.5, SPS(B) = 1/(0.02 + 1e-5 B), Bmax=4096.

The base-logit rows of a request are ``gamma + 1`` rows: the first ``gamma`` are the
draft's U_k (VERIFY: the draft logits L_d), the last is the extra row the target
needs at the bonus position. Target rows are base rows plus position noise.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field

import numpy as np

# stream ids
T_U, T_W1, T_W2, T_X0, T_UDRAFT, T_TNOISE, T_UACC, T_UFIN, T_CONF, T_BOOST, T_UX, T_A = range(12)

U_MAX = np.float32(1.0 - 2.0 ** -24)

_SIGMA_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "tests", "golden", "target_sigma.json")


def rng(seed: int, tensor: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, *extra])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def uniforms(g: np.random.Generator, shape) -> np.ndarray:
    """fp32 uniforms in [0, 1 - 2^-24]."""
    u = g.random(shape, dtype=np.float32)
    return np.minimum(u, U_MAX)


@dataclass(frozen=True)
class Config:
    seed: int
    name: str
    B: int
    V: int
    r: int
    gamma: int
    w_dtype: str            # "f32" or "bf16"
    u_sigma: float          # std of base logits
    w_sigma: float          # std of the Markov factors
    boost_ids: int = 0      # distinct ids per row raised by boost_val
    boost_val: float = 0.0
    tnoise: tuple = field(default=())   # per-position target noise std (gamma + 1 entries) or ()

    @property
    def rows_per_request(self) -> int:
        return self.gamma + 1


def _sigma_table(V: int, gamma: int) -> tuple:
    with open(_SIGMA_FILE) as f:
        tab = json.load(f)
    s = tab["sigma"][str(V)]
    assert len(s) >= gamma, "sigma table shorter than gamma"
    s = list(s[:gamma])
    return tuple(s + [s[-1]])


# seed ids of the five named workloads
TINY, SINGLE, BATCHED, VERIFY, ROUND = 1, 2, 3, 4, 5


def config(seed: int) -> Config:
    if seed == TINY:
        return Config(1, "tiny fp32 full round", B=4, V=1024, r=32, gamma=4, w_dtype="f32",
                      u_sigma=2.0, w_sigma=0.05, tnoise=(0.5,) * 5)
    if seed == SINGLE:
        return Config(2, "single-request draft", B=1, V=151936, r=256, gamma=7, w_dtype="bf16",
                      u_sigma=3.0, w_sigma=0.02, boost_ids=32, boost_val=8.0,
                      tnoise=(0.5,) * 8)
    if seed == BATCHED:
        return Config(3, "batched draft", B=64, V=151936, r=256, gamma=16, w_dtype="bf16",
                      u_sigma=3.0, w_sigma=0.02, boost_ids=32, boost_val=8.0,
                      tnoise=(0.5,) * 17)
    if seed == VERIFY:
        return Config(4, "batched verify", B=256, V=151936, r=256, gamma=16, w_dtype="bf16",
                      u_sigma=3.0, w_sigma=0.02, boost_ids=32, boost_val=8.0,
                      tnoise=_sigma_table(151936, 16))
    if seed == ROUND:
        return Config(5, "full round with scheduler", B=512, V=129280, r=256, gamma=16,
                      w_dtype="bf16", u_sigma=3.0, w_sigma=0.02, boost_ids=32, boost_val=8.0,
                      tnoise=_sigma_table(129280, 16))
    raise ValueError(f"unknown workload seed id {seed}")


def custom(seed: int, B: int, V: int, r: int, gamma: int, w_dtype: str = "bf16",
           u_sigma: float = 3.0, w_sigma: float = 0.02, boost_ids: int = 32,
           boost_val: float = 8.0, tnoise: float = 0.5) -> Config:
    """A workload of any shape with the SINGLE value recipe (used for ragged / edge sizes)."""
    return Config(seed, f"custom B={B} V={V} r={r} gamma={gamma}", B=B, V=V, r=r, gamma=gamma,
                  w_dtype=w_dtype, u_sigma=u_sigma, w_sigma=w_sigma,
                  boost_ids=min(boost_ids, V), boost_val=boost_val,
                  tnoise=(tnoise,) * (gamma + 1))


# ----------------------------------------------------------------------------- factors
def factors(c: Config):
    """W1 [V][r] and W2 [r][V]: float32 arrays for f32, uint16 bf16 bit patterns for bf16."""
    w1 = rng(c.seed, T_W1).standard_normal((c.V, c.r), dtype=np.float32) * np.float32(c.w_sigma)
    w2 = rng(c.seed, T_W2).standard_normal((c.r, c.V), dtype=np.float32) * np.float32(c.w_sigma)
    if c.w_dtype == "bf16":
        return f32_to_bf16_bits(w1), f32_to_bf16_bits(w2)
    return np.ascontiguousarray(w1), np.ascontiguousarray(w2)


def rnn_factor(c: Config, radius: float = 0.5) -> np.ndarray:
    """The RNN head's recurrence A [r][r] ~ N(0, (radius / sqrt(r))^2): spectral radius about
    `radius`, so the state stays of the size of a W1 row. bf16 bits or float32 as c.w_dtype."""
    a = rng(c.seed, T_A).standard_normal((c.r, c.r), dtype=np.float32) * np.float32(radius / np.sqrt(c.r))
    return f32_to_bf16_bits(a) if c.w_dtype == "bf16" else np.ascontiguousarray(a)


# ----------------------------------------------------------------------------- logits
def base_rows(c: Config, b: int) -> np.ndarray:
    """Request b's gamma+1 base-logit rows, float32 [gamma+1][V]."""
    n = c.gamma + 1
    rows = rng(c.seed, T_U, b).standard_normal((n, c.V), dtype=np.float32) * np.float32(c.u_sigma)
    if c.boost_ids:
        g = rng(c.seed, T_BOOST, b)
        for k in range(n):
            ids = g.choice(c.V, size=c.boost_ids, replace=False)
            rows[k, ids] += np.float32(c.boost_val)
    return rows


def target_rows(c: Config, b: int, base: np.ndarray | None = None) -> np.ndarray:
    """Request b's gamma+1 target rows: base row k plus N(0, tnoise[k]^2), float32."""
    if base is None:
        base = base_rows(c, b)
    n = c.gamma + 1
    z = rng(c.seed, T_TNOISE, b).standard_normal((n, c.V), dtype=np.float32)
    sig = np.asarray(c.tnoise[:n], dtype=np.float32)[:, None]
    return (base + z * sig).astype(np.float32)


def draft_logits_all(c: Config, requests=None) -> np.ndarray:
    """U [B][gamma][V] float32 for the listed requests (default: all)."""
    req = range(c.B) if requests is None else list(requests)
    out = np.empty((len(req), c.gamma, c.V), dtype=np.float32)
    for i, b in enumerate(req):
        out[i] = base_rows(c, b)[: c.gamma]
    return out


def target_padded_all(c: Config, requests=None) -> np.ndarray:
    """Target rows in the padded layout [B][gamma+1][V] float32."""
    req = range(c.B) if requests is None else list(requests)
    out = np.empty((len(req), c.gamma + 1, c.V), dtype=np.float32)
    for i, b in enumerate(req):
        out[i] = target_rows(c, b)
    return out


# ----------------------------------------------------------------------------- small tensors
def x0(c: Config) -> np.ndarray:
    return rng(c.seed, T_X0).integers(0, c.V, size=c.B, dtype=np.int64).astype(np.int32)


def draft_uniforms(c: Config) -> np.ndarray:
    return uniforms(rng(c.seed, T_UDRAFT), (c.B, c.gamma))


def verify_uniforms(c: Config):
    """(u_acc [B][gamma], u_fin [B]) fp32."""
    return uniforms(rng(c.seed, T_UACC), (c.B, c.gamma)), uniforms(rng(c.seed, T_UFIN), (c.B,))


def token_uniforms(c: Config) -> np.ndarray:
    """Uniforms used to draw the VERIFY workload's draft tokens from p_d."""
    return uniforms(rng(c.seed, T_UX), (c.B, c.gamma))


def draft_inputs(c: Config) -> dict:
    w1, w2 = factors(c)
    return dict(U=draft_logits_all(c), W1=w1, W2=w2, x0=x0(c), u=draft_uniforms(c))


# ----------------------------------------------------------------------------- scheduler
def confidences(c: Config) -> np.ndarray:
    """c_{r,k} = Beta(8,2) * 0.97^k, k = 1..gamma, float32 [R][gamma]."""
    g = rng(c.seed, T_CONF)
    base = g.beta(8.0, 2.0, size=(c.B, c.gamma))
    decay = 0.97 ** np.arange(1, c.gamma + 1)
    return (base * decay[None, :]).astype(np.float32)


def temperatures(gamma: int, lo: float = 0.8, hi: float = 1.5) -> np.ndarray:
    if gamma == 1:
        return np.array([lo], dtype=np.float32)
    return (lo + (hi - lo) * np.arange(gamma) / (gamma - 1)).astype(np.float32)


def sps_table(Bmax: int = 4096, a: float = 0.02, b: float = 1e-5, step: int = 0) -> np.ndarray:
    """Synthetic engine speed SPS(B) = 1/(a + b*B') in steps/s for B = 0..Bmax, where
    B' = B (smooth) or B rounded up to a multiple of ``step`` (step-shaped)."""
    B = np.arange(Bmax + 1, dtype=np.float64)
    if step:
        B = np.ceil(B / step) * step
    return (1.0 / (a + b * B)).astype(np.float32)
