"""GPU parity of dspark_schedule against the fp64 oracle and brute-force enumeration."""
import numpy as np
import pytest
import torch

import oracle
import synth
import draft_sampling_verification_head_amd as dspark
from parity import check_schedule, dev, host

pytestmark = pytest.mark.gpu


def run_schedule(conf, temp, sps, Bmax, mode):
    out = dspark.schedule(dev(conf), dev(sps), Bmax, temp=None if temp is None else dev(temp),
                          mode=mode, want_a=True)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def _check(conf, temp, sps, Bmax, mode):
    g = run_schedule(conf, temp, sps, Bmax, mode)
    ref = check_schedule(conf, temp, sps, Bmax, mode, g["len"], g["K"][0], g["theta"][0], g["a"])
    R = conf.shape[0]
    assert np.array_equal(g["t_off"], np.concatenate([[0], np.cumsum(g["len"] + 1)]))
    return g, ref


@pytest.mark.parametrize("mode", [oracle.GLOBAL, oracle.EARLY_STOP])
@pytest.mark.parametrize("step", [0, 256])
def test_round_workload_full(gpu, mode, step):
    c = synth.config(synth.ROUND)
    conf, temp, sps = synth.confidences(c), synth.temperatures(c.gamma), synth.sps_table(4096, step=step)
    g, ref = _check(conf, temp, sps, 4096, mode)
    assert np.array_equal(g["len"], ref["len"]) and g["K"][0] == ref["K"]


def test_brute_force_tiny(gpu):
    rng = np.random.default_rng(77)
    for it in range(40):
        R, G = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        Bmax = int(rng.integers(R, R * (G + 1) + 2))
        conf = rng.random((R, G)).astype(np.float32)
        conf[rng.random((R, G)) < 0.1] = 0.0
        temp = (0.6 + rng.random(G)).astype(np.float32) if it % 2 else None
        kind = it % 3
        if kind == 0:
            sps = synth.sps_table(Bmax, b=float(rng.uniform(1e-3, 5e-2)))
        elif kind == 1:
            sps = synth.sps_table(Bmax, b=float(rng.uniform(1e-3, 5e-2)), step=int(rng.integers(2, 5)))
        else:
            sps = np.sort(rng.random(Bmax + 1))[::-1].astype(np.float32)
        best, args = oracle.brute_force_schedule(conf, temp, sps, Bmax)
        g = run_schedule(conf, temp, sps, Bmax, oracle.GLOBAL)
        assert float(g["theta"][0]) == pytest.approx(best, rel=1e-6)
        assert tuple(int(v) for v in g["len"]) in [tuple(a) for a in args]


@pytest.mark.parametrize("R,G,Bmax", [
    (1, 1, 1), (1, 1, 2), (3, 5, 3), (1024, 16, 20000), (16384, 1, 20000), (256, 64, 5000),
    (700, 7, 2100), (1, 64, 100),
    (4, 16, 200), (8, 8, 9), (5, 13, 200),   # 64 and 65 candidates: both sides of the one-wave path
])
def test_shapes_and_caps(gpu, R, G, Bmax):
    c = synth.custom(960 + R % 101, B=R, V=8, r=1, gamma=G)
    conf = synth.confidences(c)
    temp = synth.temperatures(G)
    sps = synth.sps_table(Bmax, b=2e-5)
    for mode in (oracle.GLOBAL, oracle.EARLY_STOP):
        _check(conf, temp, sps, Bmax, mode)


def test_closed_forms(gpu):
    rng = np.random.default_rng(12)
    R, G = 7, 5
    conf = rng.random((R, G)).astype(np.float32)
    conf[2, 3] = 0.0
    conf[5, 0] = 0.0
    pos = int((oracle.prefix_survival(oracle.temperature_scale(conf)) > 0).sum())
    for Bmax in [R, R + 3, R + pos, 200]:
        g = run_schedule(conf, None, np.ones(Bmax + 1, np.float32), Bmax, oracle.GLOBAL)
        assert g["K"][0] - R == min(pos, Bmax - R)
    sps = np.zeros(41, np.float32)
    sps[R] = 3.0
    g = run_schedule(conf, None, sps, 40, oracle.GLOBAL)
    assert g["K"][0] == R and np.all(g["len"] == 0)
    # step-shaped speed: early stop is trapped at n = 0, global search reaches n = 4
    sps = np.array([1.0, 1.0, 0.5, 0.5, 0.5, 0.5], np.float32)
    one = np.ones((1, 4), np.float32)
    es = run_schedule(one, None, sps, 5, oracle.EARLY_STOP)
    gl = run_schedule(one, None, sps, 5, oracle.GLOBAL)
    assert es["K"][0] == 1 and es["theta"][0] == 1.0
    assert gl["K"][0] == 5 and gl["theta"][0] == 2.5 and list(gl["len"]) == [4]


def test_out_of_range_inputs(gpu):
    conf = np.array([[1.5, 0.9, np.nan, 0.7], [-0.2, 0.5, 0.5, 0.5]], np.float32)
    temp = np.array([2.0, -1.0, 1.0, 1.0], np.float32)
    _check(conf, temp, synth.sps_table(20, b=1e-3), 20, oracle.GLOBAL)


def test_determinism(gpu):
    c = synth.config(synth.ROUND)
    conf, temp, sps = synth.confidences(c), synth.temperatures(16), synth.sps_table(4096)
    a = run_schedule(conf, temp, sps, 4096, oracle.GLOBAL)
    b = run_schedule(conf, temp, sps, 4096, oracle.GLOBAL)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def _random_shapes(n, seed):
    """Scheduler shapes drawn from a fixed seed within the caps: R * gamma up to 16384,
    Bmax from R to past R * (gamma + 1), temperatures given or not, smooth or step SPS."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        G = int(g.integers(1, 65))
        R = int(g.integers(1, 16384 // G + 1))
        Bmax = int(g.integers(R, R * (G + 1) + 64))
        out.append((R, G, Bmax, bool(g.random() < 0.5), int(g.integers(0, 3))))
    return out


@pytest.mark.parametrize("R,G,Bmax,with_temp,sps_kind", _random_shapes(10, 2029))
def test_random_shapes(gpu, R, G, Bmax, with_temp, sps_kind):
    """Seeded random shapes, confidences with zeros and ones mixed in, against the oracle in
    both modes."""
    g = np.random.default_rng(R * 131 + G)
    conf = g.beta(4.0, 1.5, size=(R, G)).astype(np.float32)
    conf[g.random((R, G)) < 0.05] = 0.0
    conf[g.random((R, G)) < 0.05] = 1.0
    temp = (0.6 + g.random(G)).astype(np.float32) if with_temp else None
    if sps_kind == 0:
        sps = synth.sps_table(Bmax, b=float(g.uniform(1e-6, 1e-4)))
    elif sps_kind == 1:
        sps = synth.sps_table(Bmax, b=float(g.uniform(1e-6, 1e-4)), step=int(g.integers(2, 513)))
    else:
        sps = np.sort(g.random(Bmax + 1))[::-1].astype(np.float32)
    for mode in (oracle.GLOBAL, oracle.EARLY_STOP):
        _check(conf, temp, sps, Bmax, mode)
