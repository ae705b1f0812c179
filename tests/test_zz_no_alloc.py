"""The allocation-free draft (dspark_markov_draft_noalloc, static device scratch) against the
workspace draft (dspark_markov_draft_ex) through the C ABI: the same tokens, probabilities,
normalisers and logits bit for bit, on two calls in a row with the second input smaller, on
the single-request one-launch path and on the batched slab path; a call whose path needs
more scratch than the array holds is refused and enqueues nothing."""
import numpy as np
import pytest
import torch

import synth
import draft_sampling_verification_head_amd as dspark
from draft_sampling_verification_head_amd import binding
from parity import dev, host

pytestmark = pytest.mark.gpu


def _inputs(seed, B, V, r, G, wdt="bf16"):
    c = synth.custom(seed, B=B, V=V, r=r, gamma=G, w_dtype=wdt, w_sigma=0.3)
    d = synth.draft_inputs(c)
    return {k: dev(v) for k, v in d.items()}


def _outputs(B, G, V, logits):
    return dict(x=torch.full((B, G), -7, dtype=torch.int32, device="cuda"),
                q=torch.full((B, G), -1.0, device="cuda"),
                lse=torch.full((B, G), -1.0, device="cuda"),
                L=torch.full((B, G, V), -1.0, device="cuda") if logits else None)


def _compare(t, logits, per_position=False):
    B, G, V = t["U"].shape
    ref = dspark.markov_draft(t["U"], t["W1"], t["W2"], t["x0"], t["u"], want_logits=logits,
                              per_position=per_position)
    out = dspark.markov_draft_noalloc(t["U"], t["W1"], t["W2"], t["x0"], t["u"],
                                      out=_outputs(B, G, V, logits), per_position=per_position)
    torch.cuda.synchronize()
    keys = ("x", "q", "lse", "L") if logits else ("x", "q", "lse")
    for k in keys:
        assert np.array_equal(host(out[k]).view(np.uint8), host(ref[k]).view(np.uint8)), k
    assert np.all(host(out["x"]) >= 0)


@pytest.mark.parametrize("shapes,logits", [
    ([(1, 151936, 256, 7), (1, 20000, 64, 4)], True),       # single request, one launch
    ([(64, 151936, 256, 16), (12, 9000, 32, 3)], False),    # slab, one launch
    ([(64, 151936, 256, 4), (9, 40000, 128, 2)], True),     # slab with the logits output
])
def test_noalloc_matches_workspace_draft_twice(gpu, shapes, logits):
    for i, (B, V, r, G) in enumerate(shapes):
        t = _inputs(1400 + 10 * i + B, B, V, r, G)
        plan = dspark.markov_draft_plan(t["U"], t["W1"], t["W2"],
                                        torch.empty(1, device="cuda") if logits else None)
        assert plan[2] <= binding.load().dspark_noalloc_scratch_bytes()
        _compare(t, logits)


def test_noalloc_per_position_and_sweep(gpu):
    """Per-position launches (slab) and the vocabulary sweep (fp32 factors, logits to the
    caller) through the static scratch, then a smaller call."""
    t = _inputs(1450, 20, 30000, 64, 3)
    _compare(t, True, per_position=True)
    t = _inputs(1451, 3, 5000, 16, 4, wdt="f32")
    _compare(t, True)
    t = _inputs(1452, 2, 3000, 8, 2, wdt="f32")
    _compare(t, False)


def test_noalloc_refuses_more_than_its_scratch(gpu):
    """The sweep path without the logits output keeps two logits rows per request in scratch:
    8 requests of 600000 logits need 38.4 MB > 32 MiB, so the call is refused with
    DSPARK_ERR_UNSUPPORTED and the outputs stay untouched."""
    lib = binding.load()
    B, V, r, G = 8, 600000, 4, 1
    t = _inputs(1460, B, V, r, G, wdt="f32")
    out = _outputs(B, G, V, False)
    with pytest.raises(binding.DsparkError) as e:
        dspark.markov_draft_noalloc(t["U"], t["W1"], t["W2"], t["x0"], t["u"], out=out)
    assert e.value.status == binding.ERR_UNSUPPORTED
    assert "scratch" in lib.dspark_last_error().decode()
    torch.cuda.synchronize()
    assert bool((out["x"] == -7).all())
