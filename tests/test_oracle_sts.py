"""Pins of the STS oracle (sequential temperature scaling fit and ECE)."""
import numpy as np
import pytest

import oracle
from oracle import sts


def test_outcomes_follow_verify_results():
    o = sts.outcomes([0, 2, 3, 1, -1, 0], [3, 3, 3, 1, 3, 0], 3)
    assert o.tolist() == [[0, -1, -1], [1, 1, 0], [1, 1, 1], [1, -1, -1], [-1, -1, -1],
                          [-1, -1, -1]]
    assert sts.outcomes([2], None, 4).tolist() == [[1, 1, 0, -1]]


def test_ece_hand_example():
    cs = np.array([0.9, 0.9, 0.2, 0.95])
    o = np.array([1, 0, 0, 1])
    # bin 9: scores .9 .9 .95, outcomes 1 0 1 -> |2/3 - 0.91666...| * 3/4; bin 2: |0 - .2| / 4
    expect = abs(2.0 / 3.0 - (0.9 + 0.9 + 0.95) / 3.0) * 0.75 + 0.2 * 0.25
    assert sts.ece(cs, o, 10) == pytest.approx(expect, abs=1e-15)
    assert sts.ece(cs, np.array([-1, -1, -1, -1]), 10) == 0.0
    # a score of exactly 1 lands in the last bin
    assert sts.ece(np.array([1.0]), np.array([1]), 10) == 0.0


def test_scale_matches_scheduler_temperature():
    g = np.random.default_rng(3)
    c = g.random((50, 1)).astype(np.float32)
    c[0, 0], c[1, 0], c[2, 0] = 0.0, 1.0, np.nan
    for T in (0.5, 1.0, 2.3, -1.0):
        ref = oracle.temperature_scale(c, np.array([T], np.float32))[:, 0]
        assert np.array_equal(sts.scale(c[:, 0], T), ref)


def test_nll_optimum_closed_form():
    """A single score c0 observed with accept rate p: the NLL minimiser solves
    sigmoid(logit(c0) / T) = p, i.e. T = logit(c0) / logit(p)."""
    c0, acc, rej = 0.8, 6, 4
    logit = lambda x: np.log(x / (1 - x))
    T_star = np.float32(logit(np.float64(np.float32(c0))) / logit(acc / (acc + rej)))
    grid = np.array([T_star * f for f in (0.8, 0.9, 0.97, 1.0, 1.03, 1.1, 1.25)], np.float32)
    N = acc + rej
    conf = np.full((N, 1), c0, np.float32)
    n_acc = np.array([1] * acc + [0] * rej)           # accepted / rejected at position 0
    length = np.ones(N, np.int64)
    for objective in (sts.NLL, sts.ECE):
        r = sts.sts_fit(conf, n_acc, length, grid, bins=15, objective=objective)
        assert r["idx"][0] == 3 and r["T"][0] == pytest.approx(float(T_star))
    assert r["ece_after"][0] < 1e-6 < r["ece_before"][0]


def test_recovers_generating_temperature():
    g = np.random.default_rng(11)
    N, G = 40000, 3
    T_true = np.array([1.6, 2.2, 0.7])
    conf = g.beta(6, 2, size=(N, G)).astype(np.float32)
    # acceptance along each block: position k accepted with probability sigmoid(logit(c)/T_k)
    q = np.stack([sts.scale(conf[:, k], T_true[k]) for k in range(G)], axis=1)
    acc = g.random((N, G)) < q
    n_acc = np.where(acc.all(axis=1), G, np.argmin(acc, axis=1))
    grid = np.arange(0.4, 3.0, 0.05).astype(np.float32)
    r = sts.sts_fit(conf, n_acc, None, grid, bins=15, objective=sts.NLL)
    assert np.all(np.abs(r["T"] - T_true) <= 0.1)
    assert np.all(r["ece_after"] < r["ece_before"])
    assert np.all(r["ece_after"] < 0.02)


def test_unit_temperature_keeps_ece_and_order():
    g = np.random.default_rng(5)
    conf = g.random((200, 2)).astype(np.float32)
    n_acc = g.integers(0, 3, size=200)
    r = sts.sts_fit(conf, n_acc, None, np.array([1.0], np.float32))
    assert np.array_equal(r["ece_before"], r["ece_after"])
    for T in (0.3, 1.7, 4.0):
        cs = sts.scale(conf[:, 0], T)
        assert np.array_equal(np.argsort(cs, kind="stable"), np.argsort(conf[:, 0], kind="stable"))
