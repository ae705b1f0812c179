"""Pins of the oracle's TV labels c* = 1 - 1/2 ||p_d - p_t||_1 = sum min(p_d, p_t)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _log(w):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(w, np.float64))


def test_rational_rows_exact_fraction():
    g = np.random.default_rng(4)
    for _ in range(20):
        V = int(g.integers(2, 30))
        wd = g.integers(0, 20, size=V); wd[g.integers(0, V)] += 1
        wt = g.integers(0, 20, size=V); wt[g.integers(0, V)] += 1
        Wd, Wt = int(wd.sum()), int(wt.sum())
        exact = sum(min(Fraction(int(a), Wd), Fraction(int(b), Wt)) for a, b in zip(wd, wt))
        assert oracle.tv_row_pair(_log(wd), _log(wt)) == pytest.approx(float(exact), abs=1e-12)


def test_two_point_closed_form():
    for q, s in [(0.3, 0.7), (0.5, 0.5), (0.01, 0.99), (0.9, 0.2)]:
        c = oracle.tv_row_pair(_log([q, 1 - q]), _log([s, 1 - s]))
        assert c == pytest.approx(1 - abs(q - s), abs=1e-7)


def test_identical_and_disjoint_rows():
    g = np.random.default_rng(8)
    row = (3 * g.standard_normal(500)).astype(np.float32)
    assert oracle.tv_row_pair(row, row) == pytest.approx(1.0, abs=1e-12)
    a = row.copy(); a[250:] = -np.inf
    b = row.copy(); b[:250] = -np.inf
    assert oracle.tv_row_pair(a, b) == 0.0


def test_positions_beyond_length_are_nan():
    g = np.random.default_rng(9)
    B, G, V = 3, 4, 16
    Ld = g.standard_normal((B, G, V)).astype(np.float32)
    length = np.array([0, 2, 4])
    t_off = np.concatenate([[0], np.cumsum(length + 1)])
    Lt = g.standard_normal((int(t_off[-1]), V)).astype(np.float32)
    c = oracle.tv_labels(Ld, Lt, t_off=t_off, length=length)
    for b in range(B):
        assert np.all(np.isfinite(c[b, : length[b]]))
        assert np.all(np.isnan(c[b, length[b]:]))
        assert np.all((c[b, : length[b]] >= 0) & (c[b, : length[b]] <= 1))
