"""GPU parity of dspark_sts_fit against the fp64 STS oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import sts
import synth
import draft_sampling_verification_head_amd as dspark
from parity import dev, host


def lib():
    return dspark.binding.load()

pytestmark = pytest.mark.gpu


def validation_set(seed, N, G, T_true, partial=True):
    """Raw scores and verify-style results: position k of a block is accepted with
    probability sigmoid(logit(c) / T_true[k]); verification stops at the first rejection."""
    g = np.random.default_rng(seed)
    conf = g.beta(6, 2, size=(N, G)).astype(np.float32)
    q = np.stack([sts.scale(conf[:, k], T_true[k]) for k in range(G)], axis=1)
    acc = g.random((N, G)) < q
    length = g.integers(1, G + 1, size=N) if partial else np.full(N, G)
    first = np.where(acc.all(axis=1), G, np.argmin(acc, axis=1))
    n_acc = np.minimum(first, length)
    return conf, n_acc.astype(np.int32), length.astype(np.int32)


def run(conf, n_acc, length, grid, bins, objective):
    out = dspark.sts_fit(dev(conf), dev(n_acc), dev(grid), length=None if length is None else dev(length),
                         bins=bins, objective=objective, want_obj=True)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def check(conf, n_acc, length, grid, bins, objective):
    g = run(conf, n_acc, length, grid, bins, objective)
    ref = sts.sts_fit(conf, n_acc, length, grid, bins=bins, objective=objective)
    G = conf.shape[1]
    for k in range(G):
        gi = int(np.argmax(grid == g["T"][k]))
        best = ref["obj"][k].min()
        # the same grid value, or one whose objective ties the minimum within rounding
        assert gi == ref["idx"][k] or ref["obj"][k][gi] <= best * (1 + 1e-9) + 1e-12, k
    tol_obj = np.maximum(1e-6, 1e-6 * np.abs(ref["obj"]))
    assert np.all(np.abs(g["obj"] - ref["obj"]) <= tol_obj)
    assert np.max(np.abs(g["ece_before"] - ref["ece_before"])) < 1e-6
    assert np.max(np.abs(g["ece_after"] - ref["ece_after"])) < 1e-6
    return g, ref


@pytest.mark.parametrize("N,G,nT,bins,objective,partial", [
    (20000, 4, 40, 15, sts.NLL, True),
    (20000, 4, 40, 15, sts.ECE, True),
    (3001, 16, 64, 10, sts.NLL, False),
    (777, 1, 5, 16, sts.ECE, True),
    (65536, 16, 64, 15, sts.NLL, True),
])
def test_matches_oracle(gpu, N, G, nT, bins, objective, partial):
    T_true = np.linspace(0.6, 2.4, G)
    conf, n_acc, length = validation_set(800 + N + G, N, G, T_true, partial)
    grid = np.linspace(0.3, 3.0, nT).astype(np.float32)
    check(conf, n_acc, length if partial else None, grid, bins, objective)


def test_closed_form_single_score(gpu):
    c0, acc, rej = 0.8, 6, 4
    logit = lambda x: np.log(x / (1 - x))
    T_star = np.float32(logit(np.float64(np.float32(c0))) / logit(acc / (acc + rej)))
    grid = np.array([T_star * f for f in (0.8, 0.9, 0.97, 1.0, 1.03, 1.1, 1.25)], np.float32)
    conf = np.full((acc + rej, 1), c0, np.float32)
    n_acc = np.array([1] * acc + [0] * rej, np.int32)
    length = np.ones(acc + rej, np.int32)
    for objective in (sts.NLL, sts.ECE):
        g = run(conf, n_acc, length, grid, 15, objective)
        assert g["T"][0] == grid[3]
        assert g["ece_after"][0] < 1e-6 < g["ece_before"][0]


def test_nothing_observed(gpu):
    conf = np.full((10, 3), 0.7, np.float32)
    n_acc = np.full(10, -1, np.int32)
    g = run(conf, n_acc, None, np.array([0.5, 1.0, 2.0], np.float32), 15, sts.NLL)
    assert np.all(g["T"] == 0.5) and np.all(g["ece_before"] == 0) and np.all(g["ece_after"] == 0)


def test_edge_scores_and_temperatures(gpu):
    """Scores at and past the edges (0, 1, negative, above 1, NaN, the float just below 1) and
    grid values that count as 1 (0, negative, NaN), an infinite temperature (every interior
    score 0.5) and a tiny one (hard 0 / 1 scores), against the oracle with both objectives."""
    g = np.random.default_rng(77)
    N, G = 3000, 3
    conf = g.beta(6, 2, size=(N, G)).astype(np.float32)
    edge = np.array([0.0, 1.0, -0.5, 1.5, np.nan, np.float32(1) - np.float32(2 ** -24), 1e-30, 0.5],
                    np.float32)
    conf[: edge.size * 40] = np.repeat(edge, 40)[:, None]
    n_acc = g.integers(0, G + 1, size=N).astype(np.int32)
    grid = np.array([0.5, 1.0, 2.0, np.inf, 0.0, -1.0, np.nan, 1e-30, 3.0], np.float32)
    with np.errstate(over="ignore"):              # the oracle's power overflows to +inf (score 0)
        for objective in (sts.NLL, sts.ECE):
            check(conf, n_acc, None, grid, 15, objective)


def test_bitwise_reruns_and_poisoned_workspace(gpu):
    """Two calls on workspaces filled with zeros and with random bytes give the same bits
    (every partial is written before it is read, and every sum has a fixed order or is
    exact), with both objectives and with more than one slice of samples per position."""
    g = np.random.default_rng(31)
    N, G = 40000, 5
    conf, n_acc, length = validation_set(31, N, G, np.linspace(0.7, 2.0, G), True)
    grid = np.linspace(0.3, 3.0, 19).astype(np.float32)              # 20 temperatures: groups of 5
    nbytes = lib().dspark_sts_fit_workspace_bytes(N, G, grid.size)
    for objective in (sts.NLL, sts.ECE):
        outs = []
        for fill in ("zeros", "random"):
            ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
            if fill == "random":
                ws.copy_(torch.from_numpy(g.integers(0, 256, nbytes, dtype=np.uint8)))
            out = dspark.sts_fit(dev(conf), dev(n_acc), dev(grid), length=dev(length),
                                 objective=objective, want_obj=True, ws=ws)
            torch.cuda.synchronize()
            outs.append({k: host(v) for k, v in out.items()})
        for k in outs[0]:
            assert outs[0][k].tobytes() == outs[1][k].tobytes(), k
    check(conf, n_acc, length, grid, 15, sts.ECE)


def test_fit_on_verify_results(gpu):
    """Validation pairs taken from dspark_verify's own accept counts and lengths."""
    c = synth.custom(890, B=512, V=640, r=1, gamma=6, w_dtype="f32", tnoise=0.9)
    Ld = synth.draft_logits_all(c)
    Lt = synth.target_padded_all(c).reshape(-1, c.V)
    x = np.empty((c.B, c.gamma), np.int32)
    ux = synth.token_uniforms(c)
    for b in range(c.B):
        for k in range(c.gamma):
            x[b, k] = oracle.inverse_cdf(oracle.softmax_row(Ld[b, k])[0], oracle.clamp_uniform(ux[b, k]))
    u_acc, u_fin = synth.verify_uniforms(c)
    length = np.random.default_rng(5).integers(0, c.gamma + 1, size=c.B).astype(np.int32)
    out = dspark.verify(dev(Ld), dev(Lt), dev(x), dev(u_acc), dev(u_fin), length=dev(length))
    torch.cuda.synchronize()
    n_acc = host(out["n"])
    conf = synth.confidences(synth.custom(891, B=c.B, V=8, r=1, gamma=c.gamma))
    grid = np.linspace(0.25, 4.0, 31).astype(np.float32)
    check(conf, n_acc, length, grid, 15, sts.NLL)


def _random_shapes(n, seed):
    """STS shapes drawn from a fixed seed within the caps: N 1..70000, gamma 1..64 with
    N * gamma kept under 1.2e6 for the oracle, 1..64 grid values, 1..16 bins, either
    objective, full or partial verify lengths."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        G = int(g.integers(1, 65))
        N = int(g.integers(1, min(70000, 1_200_000 // G) + 1))
        out.append((N, G, int(g.integers(1, 65)), int(g.integers(1, 17)),
                    [sts.NLL, sts.ECE][int(g.integers(0, 2))], bool(g.random() < 0.6)))
    return out


@pytest.mark.parametrize("N,G,nT,bins,objective,partial", _random_shapes(8, 2030))
def test_random_shapes(gpu, N, G, nT, bins, objective, partial):
    """Seeded random shapes and grids (sorted or not) against the oracle."""
    g = np.random.default_rng(N + G)
    T_true = g.uniform(0.5, 2.5, G)
    conf, n_acc, length = validation_set(900 + N + G, N, G, T_true, partial)
    grid = g.uniform(0.2, 3.5, nT).astype(np.float32)
    if g.random() < 0.5:
        grid = np.sort(grid)
    check(conf, n_acc, length if partial else None, grid, bins, objective)
