"""Pins of the oracle's shared numerics (inverse-CDF draw, uniform clamp) and of its
teacher-forcing options, against values fixed by exact arithmetic.

The inverse-CDF draw takes the smallest token v with F(v) > u, F the running sum of the law
in token-id order; when rounding leaves u at or past the last F, the last token with positive
mass is taken ([P3] "DSpark Speculative Decoding", "Semi-Autoregressive Generation": one draw
from p_k; the one-uniform inverse CDF is the reading adopted for how it is drawn). The pins
use laws whose cumulative sums are exact in binary floating point (dyadic rationals), and a
brute force in exact rational arithmetic on integer weights. Each pin is also run against a
few planted mistakes, to show it would catch them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import numerics

U_MAX = 1.0 - 2.0 ** -24


# ----------------------------------------------------------------------------- inverse CDF
def _pin_inverse_cdf(inverse_cdf):
    """Every fixed case of the draw; raises AssertionError on the first wrong answer."""
    q = np.array([0.25, 0.25, 0.5])                 # F = 1/4, 1/2, 1 exactly
    assert inverse_cdf(q, 0.0) == 0
    assert inverse_cdf(q, 0.2499) == 0
    assert inverse_cdf(q, 0.25) == 1                # F(v) > u is strict: a boundary goes right
    assert inverse_cdf(q, 0.5) == 2
    assert inverse_cdf(q, U_MAX) == 2
    # zero-mass tokens are never drawn, wherever they sit
    z = np.array([0.0, 0.5, 0.0, 0.5, 0.0])         # F = 0, 1/2, 1/2, 1, 1
    assert inverse_cdf(z, 0.0) == 1
    assert inverse_cdf(z, 0.5) == 3
    assert inverse_cdf(z, U_MAX) == 3
    # past the end: u at or beyond F(V-1) takes the last token with positive mass
    short = np.array([0.25, 0.25, 0.0, 0.0])        # mass 1/2 (a law that rounded short)
    assert inverse_cdf(short, 0.9) == 1
    assert inverse_cdf(short, 0.5) == 1
    assert inverse_cdf(short, 0.49) == 1
    assert inverse_cdf(short, 0.2) == 0
    assert inverse_cdf(np.array([0.0, 0.375, 0.0, 0.125, 0.0, 0.0]), 0.75) == 3
    # nothing to draw
    assert inverse_cdf(np.zeros(4), 0.3) == -1
    assert inverse_cdf(np.zeros(1), 0.0) == -1
    # one token
    assert inverse_cdf(np.array([1.0]), U_MAX) == 0


def _brute_force_token(w, num, den):
    """min{v : W(v) / S > num / den} in exact rationals, W the running integer weight sum."""
    S = sum(int(x) for x in w)
    u = Fraction(num, den)
    acc = 0
    for v, x in enumerate(w):
        acc += int(x)
        if Fraction(acc, S) > u:
            return v
    return max(v for v, x in enumerate(w) if x > 0)


def _pin_inverse_cdf_brute_force(inverse_cdf):
    g = np.random.default_rng(41)
    for _ in range(300):
        V = int(g.integers(1, 9))
        w = g.integers(0, 4, size=V)
        if w.sum() == 0:
            w[int(g.integers(0, V))] = 1
        S = int(w.sum())
        p = w / S
        # uniforms on and between the cell boundaries (k / (2 S), exact in binary when S is a
        # power of two; otherwise the comparison is still decided far from the rounding)
        for kk in range(0, 2 * S):
            u = kk / (2 * S)
            if abs(u * S - round(u * S)) < 1e-12 and (S & (S - 1)) != 0:
                continue                            # an inexact boundary: skip, not a pin
            assert inverse_cdf(p, u) == _brute_force_token(w, kk, 2 * S), (w.tolist(), kk, S)


def test_inverse_cdf_fixed_cases():
    _pin_inverse_cdf(oracle.inverse_cdf)


def test_inverse_cdf_brute_force_rationals():
    _pin_inverse_cdf_brute_force(oracle.inverse_cdf)


def _mistake_left(p, u):                 # F(v) >= u instead of F(v) > u
    f = np.cumsum(p)
    v = int(np.searchsorted(f, u, side="left"))
    if v >= p.shape[0]:
        nz = np.nonzero(p > 0)[0]
        return int(nz[-1]) if nz.size else -1
    return v


def _mistake_last_token(p, u):           # fallback returns V - 1 whatever its mass
    f = np.cumsum(p)
    v = int(np.searchsorted(f, u, side="right"))
    return p.shape[0] - 1 if v >= p.shape[0] else v


def _mistake_past_end(p, u):             # no fallback: returns V
    return int(np.searchsorted(np.cumsum(p), u, side="right"))


def _mistake_reversed_order(p, u):       # cumulative sum taken from the top token down
    V = p.shape[0]
    v = numerics.inverse_cdf(p[::-1].copy(), u)
    return V - 1 - v if v >= 0 else -1


def _mistake_zero_law(p, u):             # an all-zero law draws token 0 instead of -1
    v = numerics.inverse_cdf(p, u)
    return 0 if v < 0 else v


@pytest.mark.parametrize("mistake", [_mistake_left, _mistake_last_token, _mistake_past_end,
                                     _mistake_reversed_order, _mistake_zero_law])
def test_inverse_cdf_pins_catch_planted_mistakes(mistake):
    with pytest.raises(AssertionError):
        _pin_inverse_cdf(mistake)


@pytest.mark.parametrize("mistake", [_mistake_left, _mistake_reversed_order])
def test_inverse_cdf_brute_force_catches_planted_mistakes(mistake):
    with pytest.raises(AssertionError):
        _pin_inverse_cdf_brute_force(mistake)


# ----------------------------------------------------------------------------- uniform clamp
def _pin_clamp(clamp):
    """Host uniforms are fp32, widened exactly and clamped into [0, 1 - 2^-24]; NaN -> 0."""
    assert clamp(0.5) == 0.5
    assert clamp(np.float32(0.1)) == float(np.float32(0.1))
    assert clamp(0.1) == float(np.float32(0.1))             # an fp64 input is read as fp32
    assert clamp(1.0) == U_MAX
    assert clamp(1.5) == U_MAX
    assert clamp(np.inf) == U_MAX
    assert clamp(0.99999997) == U_MAX                         # rounds to 1.0 in fp32
    assert clamp(U_MAX) == U_MAX
    assert clamp(np.float32(1.0) - np.float32(2 ** -23)) == 1.0 - 2 ** -23
    assert clamp(0.0) == 0.0
    for v in (-0.0, -0.25, -np.inf, np.nan):
        out = clamp(v)
        assert out == 0.0 and np.copysign(1.0, out) == 1.0, v
    assert clamp(np.float32(1e-45)) == float(np.float32(1e-45))   # denormals pass through


def test_clamp_uniform_fixed_cases():
    _pin_clamp(oracle.clamp_uniform)


def _clamp_no_nan(u):                    # NaN passes through
    u = float(np.float32(u))
    return min(max(u, 0.0), U_MAX)


def _clamp_no_f32(u):                    # no fp32 rounding of the input
    return min(max(float(u), 0.0), U_MAX) if u == u else 0.0


def _clamp_upper_one(u):                 # clamps to 1.0 instead of 1 - 2^-24
    u = float(np.float32(u))
    return min(u, 1.0) if u > 0 else 0.0


def _clamp_abs(u):                       # folds negatives up instead of clamping
    u = abs(float(np.float32(u)))
    return min(u, U_MAX) if u == u else 0.0


@pytest.mark.parametrize("mistake", [_clamp_no_nan, _clamp_no_f32, _clamp_upper_one, _clamp_abs])
def test_clamp_pins_catch_planted_mistakes(mistake):
    with pytest.raises(AssertionError):
        _pin_clamp(mistake)


def test_clamped_uniform_draws_inside_the_law():
    """A uniform of 1.0 (or more, or NaN) never draws past the last positive token."""
    p = np.array([0.5, 0.5, 0.0])
    assert oracle.inverse_cdf(p, oracle.clamp_uniform(1.0)) == 1
    assert oracle.inverse_cdf(p, oracle.clamp_uniform(np.nan)) == 0


# ----------------------------------------------------------------------------- teacher forcing
def _perm_chain(seed=7, B=5, G=6, V=64, r=16):
    g = np.random.default_rng(seed)
    perm = g.permutation(V)[:r]
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V) % r] = 50.0
    W2 = np.zeros((r, V), np.float32)
    W2[np.arange(r), perm] = 1.0
    U = (0.1 * g.standard_normal((B, G, V))).astype(np.float32)
    x0 = g.integers(0, V, size=B)
    u = g.uniform(1e-3, U_MAX, size=(B, G)).astype(np.float32)
    return U, W1, W2, x0, u, perm, r


def test_forced_block_follows_the_given_prefix():
    """Permutation chain: position k+1 must draw g(forced_k mod r) for any forced block."""
    U, W1, W2, x0, u, perm, r = _perm_chain()
    B, G, V = U.shape
    forced = np.random.default_rng(8).integers(0, V, size=(B, G))
    out = oracle.markov_draft(U, W1, W2, x0, u, forced=forced)
    for b in range(B):
        assert out["x"][b, 0] == perm[x0[b] % r]
        for k in range(1, G):
            assert out["x"][b, k] == perm[forced[b, k - 1] % r]


def test_forced_with_own_draws_is_the_plain_draft():
    import synth
    c = synth.config(synth.TINY)
    d = synth.draft_inputs(c)
    a = oracle.markov_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], want_logits=True)
    b = oracle.markov_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], want_logits=True,
                            forced=a["x"])
    for key in ("x", "q", "lse", "L"):
        assert np.array_equal(a[key], b[key])


def test_forced_count_gives_the_rule_at_that_count():
    """Two-point laws where every quantity is exact: the residual at a forced rejection and
    the bonus at a forced full acceptance follow the closed forms."""
    # draft (3/4, 1/4), target (1/4, 3/4) at every position; bonus row (1/2, 1/2)
    V, G = 2, 3
    Ld = np.log(np.array([[[0.75, 0.25]] * G]))
    Lt = np.log(np.array([[0.25, 0.75]] * G + [[0.5, 0.5]]))
    x = np.array([[0, 1, 0]])
    u_acc = np.full((1, G), 0.5, np.float32)
    u_fin = np.array([0.9], np.float32)
    plain = oracle.verify(Ld, Lt, x, u_acc, u_fin)
    # ratios: token 0 -> (1/4)/(3/4) = 1/3, token 1 -> min(1, 3) = 1
    assert plain["ratio"][0] == pytest.approx([1 / 3, 1.0, 1 / 3], rel=1e-12)
    assert plain["n"][0] == 0                       # 0.5 * 3/4 >= 1/4: rejected at once
    for n in range(G + 1):
        f = oracle.verify(Ld, Lt, x, u_acc, u_fin, n_forced=np.array([n]))
        assert f["n"][0] == n
        assert list(f["y"][0, :n]) == list(x[0, :n])
        if n < G:
            # residual max(0, p_t - p_d) = (0, 1/2) -> token 1 for any uniform
            assert f["law"][0] == pytest.approx([0.0, 1.0]) and f["y"][0, n] == 1
        else:
            assert f["law"][0] == pytest.approx([0.5, 0.5]) and f["y"][0, n] == 1   # 0.9 > 1/2
        assert np.all(f["y"][0, n + 1:] == -1)
    with pytest.raises(ValueError):
        oracle.verify(Ld, Lt, x, u_acc, u_fin, n_forced=np.array([G + 1]))
