"""GPU tests of the asynchronous round pipeline: the two-step-lag confidence ring
(dspark_conf_ring_*, dspark_schedule_lagged) and a whole round captured as one graph (draft
and lagged schedule on two streams, then verify and the ring push), called through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
import draft_sampling_verification_head_amd as dspark
from parity import check_schedule, dev, host

pytestmark = pytest.mark.gpu


def _history(R, G, rounds, seed):
    g = np.random.default_rng(seed)
    out = []
    for t in range(rounds):
        c = g.beta(8.0, 2.0, size=(R, G)) * 0.97 ** np.arange(1, G + 1)[None, :]
        c[g.random((R, G)) < 0.05] = 0.0
        out.append(c.astype(np.float32))
    return out


@pytest.mark.parametrize("R,G,Bmax", [(12, 4, 40), (512, 16, 4096)])   # one-wave and ranked kernels
def test_lagged_schedule_reads_round_t_minus_2(gpu, R, G, Bmax):
    """At round t the lagged schedule equals dspark_schedule on round t - 2's confidences,
    bit for bit (all ones for t < 2), and matches the oracle's lag rule."""
    hist = _history(R, G, 6, 400 + R)
    temp, sps = dev(synth.temperatures(G)), dev(synth.sps_table(Bmax, step=64))
    ring = dspark.ConfRing(R, G)
    assert ring.rounds() == 0
    for t in range(len(hist)):
        lag = dspark.schedule_lagged(ring, sps, Bmax, temp=temp, want_a=True)
        want_conf = oracle.lagged_confidences(hist, t, R, G).astype(np.float32)
        ref = dspark.schedule(dev(want_conf), sps, Bmax, temp=temp, want_a=True)
        torch.cuda.synchronize()
        for k in ("len", "t_off", "K", "theta", "a"):
            assert np.array_equal(host(lag[k]).view(np.uint8), host(ref[k]).view(np.uint8)), (t, k)
        if t in (1, 4):
            o = oracle.lagged_schedule(hist, t, host(temp), host(sps), Bmax)
            check_schedule(want_conf, host(temp), host(sps), Bmax, oracle.GLOBAL, host(lag["len"]),
                           host(lag["K"])[0], host(lag["theta"])[0], host(lag["a"]))
            assert np.array_equal(host(lag["len"]), o["len"])
        ring.push(dev(hist[t]))
        assert ring.rounds() == t + 1


def test_lag_ring_graph_replays(gpu):
    """[lagged schedule, push] captured once and replayed for six rounds, the round's
    confidences copied into the pushed buffer between replays (eager work in between):
    every replay schedules from round t - 2."""
    R, G, Bmax = 64, 8, 1024
    hist = _history(R, G, 6, 411)
    sps = dev(synth.sps_table(Bmax))
    ring = dspark.ConfRing(R, G)
    conf_buf = torch.empty((R, G), dtype=torch.float32, device="cuda")
    out = dict(len=torch.empty(R, dtype=torch.int32, device="cuda"),
               t_off=torch.empty(R + 1, dtype=torch.int32, device="cuda"),
               K=torch.empty(1, dtype=torch.int32, device="cuda"),
               theta=torch.empty(1, dtype=torch.float32, device="cuda"))
    conf_buf.copy_(dev(hist[0]))
    dspark.schedule_lagged(ring, sps, Bmax, out=out)     # allocates the workspace before capture
    ring.reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dspark.schedule_lagged(ring, sps, Bmax, out=out)
        ring.push(conf_buf)
    torch.cuda.synchronize()
    assert ring.rounds() == 0                            # capture ran nothing
    for t in range(len(hist)):
        conf_buf.copy_(dev(hist[t]))
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.lagged_schedule(hist, t, None, host(sps), Bmax)
        assert np.array_equal(host(out["len"]), ref["len"]), t
        assert int(host(out["K"])[0]) == ref["K"]
        assert ring.rounds() == t + 1


def test_round_graph_matches_eager(gpu):
    """A whole round (resident slab draft on the main stream while the lagged schedule runs on
    a side stream; then the factor-based verify on the schedule's lengths; then the push of
    the round's confidences) captured as one graph: each replay gives the eager round's
    tokens, acceptance and labels bit for bit, for rounds whose schedule differs."""
    B, V, r, G, Bmax = 24, 30000, 256, 4, 256
    c = synth.custom(412, B=B, V=V, r=r, gamma=G, w_dtype="bf16", w_sigma=0.3, tnoise=0.7)
    d = synth.draft_inputs(c)
    t = {k: dev(v) for k, v in d.items()}
    Lt = dev(synth.target_padded_all(c).reshape(-1, V))
    u_acc, u_fin = (dev(x) for x in synth.verify_uniforms(c))
    hist = _history(B, G, 5, 413)
    sps, temp = dev(synth.sps_table(Bmax, b=2e-4)), dev(synth.temperatures(G))
    assert dspark.markov_draft_one_launch(B, t["W1"], t["W2"])
    ring = dspark.ConfRing(B, G)
    conf_buf = torch.empty((B, G), dtype=torch.float32, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    out_d = dict(x=torch.empty((B, G), **i32), q=torch.empty((B, G), **f32),
                 lse=torch.empty((B, G), **f32), L=None)
    out_s = dict(len=torch.empty(B, **i32), t_off=torch.empty(B + 1, **i32), K=torch.empty(1, **i32),
                 theta=torch.empty(1, **f32))
    out_v = dict(n=torch.empty(B, **i32), y=torch.empty((B, G + 1), **i32),
                 lse_t=torch.empty((B, G + 1), **f32), cstar=torch.empty((B, G), **f32))
    side = torch.cuda.Stream()

    def round_fn():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            dspark.schedule_lagged(ring, sps, Bmax, temp=temp, out=out_s)
        dspark.markov_draft(t["U"], t["W1"], t["W2"], t["x0"], t["u"], out=out_d)
        main.wait_stream(side)
        dspark.verify_markov(t["U"], t["W1"], t["W2"], t["x0"], out_d["x"], out_d["lse"], Lt, u_acc,
                             u_fin, t_off=out_s["t_off"], length=out_s["len"], out=out_v)
        ring.push(conf_buf)

    def snapshot():
        return {k: host(v).copy() for k, v in
                [("x", out_d["x"]), ("len", out_s["len"]), ("n", out_v["n"]), ("y", out_v["y"]),
                 ("cstar", out_v["cstar"])]}

    eager = []
    for rnd in range(len(hist)):
        conf_buf.copy_(dev(hist[rnd]))
        round_fn()
        torch.cuda.synchronize()
        eager.append(snapshot())
    assert len({e["len"].tobytes() for e in eager}) > 1          # the lag changes the schedule
    ring.reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        round_fn()
    torch.cuda.synchronize()
    for rnd in range(len(hist)):
        conf_buf.copy_(dev(hist[rnd]))
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k in got:
            assert np.array_equal(got[k].view(np.uint8), eager[rnd][k].view(np.uint8)), (rnd, k)
    assert ring.rounds() == len(hist)
