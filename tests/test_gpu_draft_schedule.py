"""dspark_markov_draft_schedule: the draft and the schedule in one call equal the two calls bit
for bit, with the schedule in the draft's launch (the single-request path, <= 64 candidates)
and without it (larger schedules, batched drafts), with plain and two-step-lag confidences,
and across graph replays."""
import numpy as np
import pytest
import torch

import synth
import draft_sampling_verification_head_amd as dspark
from parity import dev, host

pytestmark = pytest.mark.gpu


def _inputs(seed, B, V, r, G, R):
    c = synth.custom(seed, B=B, V=V, r=r, gamma=G, w_dtype="bf16")
    d = {k: dev(v) for k, v in synth.draft_inputs(c).items()}
    cs = synth.custom(seed + 1, B=R, V=8, r=8, gamma=G)
    d["conf"] = dev(synth.confidences(cs))
    d["temp"] = dev(synth.temperatures(G))
    d["sps"] = dev(synth.sps_table(4096))
    return d


def _separate(d, mode, ring=None, want_logits=True):
    D = dspark.markov_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], want_logits=want_logits)
    if ring is None:
        S = dspark.schedule(d["conf"], d["sps"], 4096, temp=d["temp"], mode=mode, want_a=True)
    else:
        S = dspark.schedule_lagged(ring, d["sps"], 4096, temp=d["temp"], mode=mode, want_a=True)
    return D, S


def _fused(d, mode, ring=None, want_logits=True):
    return dspark.markov_draft_schedule(d["U"], d["W1"], d["W2"], d["x0"], d["u"], d["sps"], 4096,
                                        conf=None if ring is not None else d["conf"], ring=ring,
                                        temp=d["temp"], mode=mode, want_logits=want_logits,
                                        want_a=True)


def _same(a, b):
    for k in a:
        if a[k] is None:
            assert b[k] is None
            continue
        x, y = host(a[k]), host(b[k])
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), k


@pytest.mark.parametrize("B,V,r,G,R,mode,fused", [
    (1, 151936, 256, 7, 1, dspark.GLOBAL, True),       # the single-request workload
    (1, 20000, 64, 16, 4, dspark.EARLY_STOP, True),    # 64 candidates: still one wave
    (1, 20000, 64, 16, 5, dspark.GLOBAL, False),       # 80 candidates: three schedule launches
    (64, 20000, 256, 8, 64, dspark.GLOBAL, False),     # batched draft: the schedule after it
])
def test_draft_schedule_equals_two_calls(gpu, B, V, r, G, R, mode, fused):
    d = _inputs(3100 + B + G, B, V, r, G, R)
    assert dspark.markov_draft_schedule_fused(B, d["W1"], d["W2"], R, G) == fused
    D1, S1 = _separate(d, mode)
    D2, S2 = _fused(d, mode)
    torch.cuda.synchronize()
    _same(D1, D2)
    _same(S1, S2)


def test_draft_schedule_lagged_ring(gpu):
    B, V, r, G, R = 1, 20000, 128, 8, 3
    d = _inputs(3200, B, V, r, G, R)
    ring = dspark.ConfRing(R, G)
    hist = [dev(synth.confidences(synth.custom(3300 + i, B=R, V=8, r=8, gamma=G))) for i in range(3)]
    for i in range(3):
        ring.push(hist[i])
        D1, S1 = _separate(d, dspark.GLOBAL, ring=ring, want_logits=False)
        D2, S2 = _fused(d, dspark.GLOBAL, ring=ring, want_logits=False)
        torch.cuda.synchronize()
        _same(D1, D2)
        _same(S1, S2)
    assert dspark.markov_draft_schedule_fused(B, d["W1"], d["W2"], R, G)


def test_draft_schedule_graph_replays(gpu):
    """A captured fused call replayed with eager fused calls between the replays: every result
    equals the eager one (the draft's slots and the schedule's outputs start over each call)."""
    B, V, r, G, R = 1, 40000, 256, 7, 1
    d = _inputs(3400, B, V, r, G, R)
    ref_d, ref_s = _fused(d, dspark.GLOBAL)
    torch.cuda.synchronize()
    ref_d = {k: v.clone() for k, v in ref_d.items() if v is not None}
    ref_s = {k: v.clone() for k, v in ref_s.items() if v is not None}
    out_d = {k: torch.empty_like(v) for k, v in ref_d.items()}
    out_s = {k: torch.empty_like(v) for k, v in ref_s.items()}

    def call():
        dspark.markov_draft_schedule(d["U"], d["W1"], d["W2"], d["x0"], d["u"], d["sps"], 4096,
                                     conf=d["conf"], temp=d["temp"], want_logits=True, want_a=True,
                                     out=out_d, out_sched=out_s)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        for t in list(out_d.values()) + list(out_s.values()):
            t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        _same(ref_d, out_d)
        _same(ref_s, out_s)
        call()
        torch.cuda.synchronize()
        _same(ref_d, out_d)
