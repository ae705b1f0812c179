"""Full round on the GPU (draft -> schedule -> flattened verify -> TV labels) against the
oracle's own round on the same seeded inputs. Neither side consumes the other's outputs:
the GPU chain runs on its own results, the oracle chain on its own."""
import numpy as np
import pytest
import torch

import oracle
import synth
import draft_sampling_verification_head_amd as dspark
from parity import (tie_bound, PROB_TOL, Report, check_cstar, check_draft, check_verify, dev,
                    forced_draft_logits, host)

pytestmark = pytest.mark.gpu


def _round_inputs(c):
    base = [synth.base_rows(c, b) for b in range(c.B)]
    U = np.stack([r[: c.gamma] for r in base])
    Lt_pad = np.stack([synth.target_rows(c, b, base[b]) for b in range(c.B)])
    w1, w2 = synth.factors(c)
    u_acc, u_fin = synth.verify_uniforms(c)
    return dict(U=U, W1=w1, W2=w2, x0=synth.x0(c), u=synth.draft_uniforms(c), Lt_pad=Lt_pad,
                conf=synth.confidences(c), temp=synth.temperatures(c.gamma),
                sps=synth.sps_table(4096), u_acc=u_acc, u_fin=u_fin)


def _gpu_round(c, inp, Bmax=4096):
    d = dspark.markov_draft(dev(inp["U"]), dev(inp["W1"]), dev(inp["W2"]), dev(inp["x0"]),
                            dev(inp["u"]), want_logits=True)
    s = dspark.schedule(dev(inp["conf"]), dev(inp["sps"]), Bmax, temp=dev(inp["temp"]))
    # the target rows stand in for the target forward: laid out by the GPU's own offsets
    length = host(s["len"])
    Lt = np.concatenate([inp["Lt_pad"][b, : length[b] + 1] for b in range(c.B)])
    Lt_d = dev(Lt)
    v = dspark.verify(d["L"], Lt_d, d["x"], dev(inp["u_acc"]), dev(inp["u_fin"]),
                      t_off=s["t_off"], length=s["len"], ld_lse=d["lse"], want_lse=True)
    cs = dspark.tv_labels(d["L"], Lt_d, t_off=s["t_off"], length=s["len"], lse_d=v["lse_d"],
                          lse_t=v["lse_t"])
    torch.cuda.synchronize()
    out = {k: host(t) for k, t in d.items()}
    out.update(len=length, t_off=host(s["t_off"]), K=int(host(s["K"])[0]),
               n=host(v["n"]), y=host(v["y"]), cstar=host(cs), Lt=Lt)
    return out


def _oracle_round_check(c, inp, g, requests, rep=None):
    """The schedule exactly; for each listed request the draft on the GPU's own prefix, then
    the verify and labels of the GPU's block on the oracle's fp64 logits (teacher forcing)."""
    sched = oracle.schedule(inp["conf"], inp["temp"], inp["sps"], 4096)
    assert np.array_equal(g["len"], sched["len"]) and g["K"] == sched["K"]
    rep = check_draft(inp["U"], inp["W1"], inp["W2"], inp["x0"], inp["u"], c.w_dtype, g["x"],
                      g["q"], g["lse"], requests, gL=g["L"], rep=Report("round draft"),
                      keep_logits=(kept := {}))
    vrep = Report("round verify")
    Lt = np.concatenate([inp["Lt_pad"][b, : sched["len"][b] + 1] for b in range(c.B)])
    for b in requests:
        Ld = kept.pop(b)
        t_off = sched["t_off"][b:b + 2]
        check_verify(Ld, Lt, g["x"][b:b + 1], inp["u_acc"][b:b + 1], inp["u_fin"][b:b + 1],
                     t_off, sched["len"][b:b + 1], g["n"][b:b + 1], g["y"][b:b + 1], [0],
                     rep=vrep)
        check_cstar(Ld, Lt, t_off, sched["len"][b:b + 1], g["cstar"][b:b + 1], [0], rep=vrep)
    return rep, vrep


def test_tiny_round_exact(gpu):
    c = synth.config(synth.TINY)
    inp = _round_inputs(c)
    inp["sps"] = synth.sps_table(64, b=1e-3)
    g = _gpu_round(c, inp, Bmax=64)
    sched = oracle.schedule(inp["conf"], inp["temp"], inp["sps"], 64)
    assert np.array_equal(g["len"], sched["len"])
    rep = check_draft(inp["U"], inp["W1"], inp["W2"], inp["x0"], inp["u"], c.w_dtype, g["x"],
                      g["q"], g["lse"], range(c.B), gL=g["L"])
    assert rep.ties == 0
    Lt = np.concatenate([inp["Lt_pad"][b, : sched["len"][b] + 1] for b in range(c.B)])
    ref = oracle.markov_draft(inp["U"], inp["W1"], inp["W2"], inp["x0"], inp["u"], c.w_dtype,
                              want_logits=True)
    ov = oracle.verify(ref["L"], Lt, ref["x"], inp["u_acc"], inp["u_fin"], t_off=sched["t_off"],
                       length=sched["len"])
    assert np.array_equal(ov["n"], g["n"]) and np.array_equal(ov["y"], g["y"])
    oc = oracle.tv_labels(ref["L"], Lt, t_off=sched["t_off"], length=sched["len"])
    fin = np.isfinite(oc)
    assert np.array_equal(fin, np.isfinite(g["cstar"]))
    assert np.max(np.abs(g["cstar"][fin] - oc[fin])) < PROB_TOL


def test_round_workload_sampled(gpu):
    c = synth.config(synth.ROUND)
    inp = _round_inputs(c)
    g = _gpu_round(c, inp)
    assert g["K"] == c.B + int(g["len"].sum())
    assert np.all((g["n"] >= 0) & (g["n"] <= g["len"]))
    rep, vrep = _oracle_round_check(c, inp, g, list(range(0, c.B, 8)))
    assert rep.ties <= tie_bound(rep) and vrep.ties <= tie_bound(vrep)
    rep.record()
    vrep.record()
