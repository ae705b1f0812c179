"""Pins of the oracle's confidence scheduler: brute force, closed forms and invariants."""
import numpy as np
import pytest

import oracle
import synth


def test_temperature_exact_values():
    c = np.array([[0.8, 0.5, 0.2, 0.0, 1.0]], np.float32)
    # T = 1 is the identity on the fp32 inputs
    np.testing.assert_array_equal(oracle.temperature_scale(c, np.ones(5, np.float32)),
                                  c.astype(np.float64))
    # odds 4:1 at T = 2 -> 2:1 -> 2/3; c = 0.5 is a fixed point; 0 and 1 stay put
    out = oracle.temperature_scale(c, np.full(5, 2.0, np.float32))
    c08 = float(np.float32(0.8))
    assert out[0, 0] == pytest.approx(1 / (1 + np.sqrt((1 - c08) / c08)), rel=1e-15)
    assert out[0, 0] == pytest.approx(2 / 3, abs=1e-7)
    assert out[0, 1] == 0.5 and out[0, 3] == 0.0 and out[0, 4] == 1.0
    assert out[0, 2] == pytest.approx(1 / 3, abs=1e-7)
    # order preserving per position
    g = np.random.default_rng(0)
    cc = g.random((50, 1)).astype(np.float32)
    s = oracle.temperature_scale(cc, np.array([1.37], np.float32))[:, 0]
    assert np.array_equal(np.argsort(cc[:, 0], kind="stable"), np.argsort(s, kind="stable"))


def _random_case(g, R, G, kind, Bmax):
    conf = g.random((R, G)).astype(np.float32)
    conf[g.random((R, G)) < 0.1] = 0.0
    temp = (0.6 + g.random(G)).astype(np.float32)
    if kind == "smooth":
        sps = synth.sps_table(Bmax, a=0.02, b=float(g.uniform(1e-3, 5e-2)))
    elif kind == "step":
        sps = synth.sps_table(Bmax, a=0.02, b=float(g.uniform(1e-3, 5e-2)), step=int(g.integers(2, 5)))
    else:
        sps = np.sort(g.random(Bmax + 1))[::-1].astype(np.float32)
    return conf, temp, sps


@pytest.mark.parametrize("kind", ["smooth", "step", "random"])
def test_greedy_equals_brute_force(kind):
    g = np.random.default_rng({"smooth": 1, "step": 2, "random": 3}[kind])
    for _ in range(25):
        R, G = int(g.integers(1, 5)), int(g.integers(1, 5))
        Bmax = int(g.integers(R, R * (G + 1) + 2))
        conf, temp, sps = _random_case(g, R, G, kind, Bmax)
        best, args = oracle.brute_force_schedule(conf, temp, sps, Bmax)
        res = oracle.schedule(conf, temp, sps, Bmax, oracle.GLOBAL)
        assert res["theta"] == pytest.approx(best, rel=1e-12)
        assert tuple(int(v) for v in res["len"]) in [tuple(a) for a in args]


def test_constant_sps_takes_every_positive_candidate():
    g = np.random.default_rng(12)
    R, G = 7, 5
    conf = g.random((R, G)).astype(np.float32)
    conf[2, 3] = 0.0
    conf[5, 0] = 0.0
    pos = int((oracle.prefix_survival(oracle.temperature_scale(conf)) > 0).sum())
    for Bmax in [R, R + 3, R + pos, 200]:
        res = oracle.schedule(conf, None, np.ones(Bmax + 1, np.float32), Bmax)
        assert res["n"] == min(pos, Bmax - R)


def test_zero_speed_above_r_gives_zero_lengths():
    g = np.random.default_rng(13)
    R, G, Bmax = 6, 4, 40
    sps = np.zeros(Bmax + 1, np.float32)
    sps[R] = 3.0
    res = oracle.schedule(g.random((R, G)).astype(np.float32), None, sps, Bmax)
    assert res["n"] == 0 and np.all(res["len"] == 0) and res["K"] == R


def test_early_stop_equals_global_for_smooth_speed():
    g = np.random.default_rng(14)
    for _ in range(10):
        R, G = int(g.integers(1, 40)), int(g.integers(1, 12))
        conf = g.random((R, G)).astype(np.float32)
        Bmax = R * (G + 1)
        sps = synth.sps_table(Bmax, a=0.02, b=float(g.uniform(1e-5, 1e-2)))
        a = oracle.schedule(conf, None, sps, Bmax, oracle.GLOBAL)
        b = oracle.schedule(conf, None, sps, Bmax, oracle.EARLY_STOP)
        assert a["n"] == b["n"]


def test_step_shaped_speed_traps_early_stop():
    # R = 1, certain tokens (c = 1): Theta(0) = 1, Theta(n) = (1 + n) * 0.5 for n >= 1
    sps = np.array([1.0, 1.0, 0.5, 0.5, 0.5, 0.5], np.float32)
    conf = np.ones((1, 4), np.float32)
    es = oracle.schedule(conf, None, sps, 5, oracle.EARLY_STOP)
    gl = oracle.schedule(conf, None, sps, 5, oracle.GLOBAL)
    assert es["n"] == 0 and es["theta"] == 1.0
    assert gl["n"] == 4 and gl["theta"] == 2.5 and list(gl["len"]) == [4]


def test_invariants_on_workload_shape():
    c = synth.custom(915, B=96, V=8, r=1, gamma=16)
    conf = synth.confidences(c)
    temp = synth.temperatures(16)
    for sps in [synth.sps_table(4096), synth.sps_table(4096, step=256)]:
        for mode in (oracle.GLOBAL, oracle.EARLY_STOP):
            res = oracle.schedule(conf, temp, sps, 4096, mode)
            a = res["a"]
            assert np.all(np.diff(a, axis=1) <= 0)
            assert res["K"] == 96 + res["len"].sum()
            assert np.array_equal(res["t_off"], np.concatenate([[0], np.cumsum(res["len"] + 1)]))
            # selected set is the global top-n and is prefix-closed per request
            top = {(r, j) for _, j, r in res["ranked"][: res["n"]]}
            assert top == {(r, j) for r in range(96) for j in range(res["len"][r])}


def test_out_of_range_confidences_are_clamped():
    c = np.array([[1.5, -0.2, np.nan, 0.7]], np.float32)
    out = oracle.temperature_scale(c, np.array([2.0, 2.0, 2.0, -1.0], np.float32))
    assert list(out[0, :3]) == [1.0, 0.0, 0.0]
    assert out[0, 3] == pytest.approx(float(np.float32(0.7)), rel=1e-15)   # T <= 0 counts as 1
    np.testing.assert_array_equal(oracle.temperature_scale(c)[0, :3], [1.0, 0.0, 0.0])


def test_lag_without_history_is_the_speed_curve_alone():
    """Rounds 0 and 1 have no history: all ones, so a = 1 everywhere and
    Theta(n) = (R + n) SPS(R + n). The ranking then takes position 0 of every request, then
    position 1, ..., so len[r] = n* // R + (r < n* % R)."""
    R, G, Bmax = 5, 4, 23
    g = np.random.default_rng(31)
    sps = g.uniform(0.5, 2.0, size=Bmax + 1).astype(np.float32)
    history = [g.uniform(0.05, 0.95, size=(R, G)) for _ in range(2)]
    n = np.arange(min(R * G, Bmax - R) + 1)
    n_star = int(np.argmax((R + n) * sps[R + n].astype(np.float64)))
    want = np.array([n_star // R + (r < n_star % R) for r in range(R)])
    for t in (0, 1):
        got = oracle.lagged_schedule(history, t, None, sps, Bmax)
        assert got["n"] == n_star
        assert np.array_equal(got["len"], want)


def test_lag_reads_round_t_minus_2_only():
    """Round t's schedule ignores what rounds t and t - 1 recorded (no leak of the tokens
    being generated) and follows round t - 2."""
    R, G, Bmax = 6, 5, 40
    g = np.random.default_rng(32)
    sps = (1.0 / (0.02 + 1e-3 * np.arange(Bmax + 1))).astype(np.float32)
    history = [g.uniform(0.05, 0.99, size=(R, G)) for _ in range(6)]
    for t in range(2, 6):
        base = oracle.lagged_schedule(history, t, None, sps, Bmax)
        noisy = [h.copy() for h in history]
        noisy[t] = g.uniform(0.0, 1.0, size=(R, G))
        noisy[t - 1] = g.uniform(0.0, 1.0, size=(R, G))
        same = oracle.lagged_schedule(noisy, t, None, sps, Bmax)
        assert np.array_equal(base["len"], same["len"]) and base["theta"] == same["theta"]
        ref = oracle.schedule(history[t - 2], None, sps, Bmax)
        assert np.array_equal(base["len"], ref["len"]) and base["theta"] == ref["theta"]
        # a round t - 2 with every confidence at zero schedules nothing
        zero = [h.copy() for h in history]
        zero[t - 2] = np.zeros((R, G))
        assert oracle.lagged_schedule(zero, t, None, sps, Bmax)["len"].sum() == 0
