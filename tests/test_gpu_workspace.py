"""Workspaces need no preparation: every entry point gives oracle-matching results when its
workspace holds arbitrary bytes left by earlier calls of other shapes."""
import numpy as np
import pytest
import torch

import oracle
import synth
import draft_sampling_verification_head_amd as dspark
from draft_sampling_verification_head_amd import binding
from parity import tie_bound, check_draft, check_verify, dev, host, PROB_TOL

pytestmark = pytest.mark.gpu


def _poison(tag, nbytes, seed):
    buf = binding.workspace(nbytes, torch.device("cuda:0"), tag)
    g = torch.Generator(device="cuda").manual_seed(seed)
    buf.copy_(torch.randint(0, 256, (buf.numel(),), dtype=torch.uint8, device="cuda", generator=g))
    torch.cuda.synchronize()


def test_poisoned_workspaces(gpu):
    lib = binding.load()
    for seed, (B, V, G) in enumerate([(3, 9000, 3), (6, 20000, 5), (2, 8192, 2)]):
        c = synth.custom(980 + seed, B=B, V=V, r=16, gamma=G, w_dtype="bf16", tnoise=0.7)
        d = synth.draft_inputs(c)
        _poison("draft", lib.dspark_markov_draft_workspace_bytes(B, V, 16, G) + 4096, seed)
        out = dspark.markov_draft(dev(d["U"]), dev(d["W1"]), dev(d["W2"]), dev(d["x0"]),
                                  dev(d["u"]), want_logits=True)
        g = {k: host(v) for k, v in out.items()}
        check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", g["x"], g["q"], g["lse"],
                    range(B), gL=g["L"])

        Ld = synth.draft_logits_all(c)
        Lt_pad = synth.target_padded_all(c)
        lengths = np.array([(b * 7 + seed) % (G + 1) for b in range(B)], np.int32)
        t_off = np.concatenate([[0], np.cumsum(lengths + 1)]).astype(np.int32)
        Lt = np.concatenate([Lt_pad[b, : lengths[b] + 1] for b in range(B)])
        x = np.array([[oracle.inverse_cdf(oracle.softmax_row(Ld[b, k])[0], 0.37) for k in range(G)]
                      for b in range(B)], np.int32)
        u_acc, u_fin = synth.verify_uniforms(c)
        _poison("verify", lib.dspark_verify_workspace_bytes(B, V, G) + 4096, seed + 10)
        v = dspark.verify(dev(Ld), dev(Lt), dev(x), dev(u_acc), dev(u_fin), t_off=dev(t_off),
                          length=dev(lengths))
        check_verify(Ld, Lt, x, u_acc, u_fin, t_off, lengths, host(v["n"]), host(v["y"]), range(B))
        _poison("tv", lib.dspark_tv_labels_workspace_bytes(B, V, G) + 4096, seed + 20)
        cs = host(dspark.tv_labels(dev(Ld), dev(Lt), t_off=dev(t_off), length=dev(lengths)))
        ref = oracle.tv_labels(Ld, Lt, t_off=t_off, length=lengths)
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(cs))
        assert np.max(np.abs(cs[fin] - ref[fin]), initial=0.0) < PROB_TOL

        conf = synth.confidences(c)
        sps = synth.sps_table(64, b=1e-3)
        _poison("schedule", lib.dspark_schedule_workspace_bytes(B, G, 64) + 4096, seed + 30)
        s = dspark.schedule(dev(conf), dev(sps), 64, temp=dev(synth.temperatures(G)))
        ref = oracle.schedule(conf, synth.temperatures(G), sps, 64)
        assert np.array_equal(host(s["len"]), ref["len"])


@pytest.mark.parametrize("fill", ["zeros", "ones", "random"])
@pytest.mark.parametrize("B,V,G,want_logits", [
    (1, 9000, 5, True),       # the register-resident single-request draft
    (1, 20000, 4, False),
    (12, 9000, 3, True),      # the persistent slab draft, with and without the logits
    (24, 20000, 4, False),
])
def test_one_launch_drafts_ignore_stale_slots(gpu, fill, B, V, G, want_logits):
    """The one-launch draft forms meet through position slots in the workspace; a workspace
    of zeros (which reads as published partials and as token 0), of all-one bytes or of
    random bytes must not be taken for this call's slots."""
    lib = binding.load()
    c = synth.custom(990 + B + G, B=B, V=V, r=16, gamma=G, w_dtype="bf16", w_sigma=0.3)
    d = synth.draft_inputs(c)
    W1, W2 = dev(d["W1"]), dev(d["W2"])
    assert dspark.markov_draft_path(B, W1, W2) == ("resident" if B == 1 else "slab")
    assert dspark.markov_draft_one_launch(B, W1, W2, want_logits=want_logits)
    nbytes = lib.dspark_markov_draft_workspace_bytes(B, V, 16, G) + 4096
    if fill in ("zeros", "ones"):
        binding.workspace(nbytes, torch.device("cuda:0"), "draft").fill_(0 if fill == "zeros" else 255)
        torch.cuda.synchronize()
    else:
        _poison("draft", nbytes, 7 * B + G)
    out = dspark.markov_draft(dev(d["U"]), W1, W2, dev(d["x0"]), dev(d["u"]), want_logits=want_logits)
    g = {k: host(v) for k, v in out.items() if v is not None}
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", g["x"], g["q"], g["lse"],
                      range(B), gL=g.get("L"))
    assert rep.ties <= tie_bound(rep)


@pytest.mark.parametrize("B,V,G", [(1, 151936, 4), (24, 20000, 4)])
def test_one_launch_give_up_is_reported(gpu, B, V, G):
    """Failure injection from the host (DSPARK_DRAFT_TEST_SPIN: each wait polls about once):
    the one-launch forms give up, drain, write -1 from the first position they could not draw,
    and count the workgroups that gave up in bytes 0..3 of the workspace. The next ordinary
    call on the same workspace draws every position (count 0) and matches a fresh call."""
    c = synth.custom(1300 + B, B=B, V=V, r=16, gamma=G, w_dtype="bf16", w_sigma=0.3)
    d = synth.draft_inputs(c)
    U, W1, W2, x0, u = dev(d["U"]), dev(d["W1"]), dev(d["W2"]), dev(d["x0"]), dev(d["u"])
    path, one, nbytes = dspark.markov_draft_plan(U, W1, W2)
    assert one and path == ("resident" if B == 1 else "slab")
    ws = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda")
    bad = dspark.markov_draft(U, W1, W2, x0, u, ws=ws, test_spin=True)
    torch.cuda.synchronize()
    gave = binding.draft_gave_up(ws)
    xb = host(bad["x"])
    assert gave >= 1, "a one-poll wait on a multi-workgroup launch should give up"
    assert (xb == -1).any()
    for b in range(B):                          # -1 from some position on, valid before it
        row = xb[b]
        k = int(np.argmax(row == -1)) if (row == -1).any() else G
        assert np.all(row[k:] == -1) and np.all((row[:k] >= 0) & (row[:k] < V))
    good = dspark.markov_draft(U, W1, W2, x0, u, ws=ws)
    torch.cuda.synchronize()
    assert binding.draft_gave_up(ws) == 0
    fresh = dspark.markov_draft(U, W1, W2, x0, u)
    torch.cuda.synchronize()
    for k in ("x", "q", "lse"):
        assert np.array_equal(host(good[k]).view(np.uint8), host(fresh[k]).view(np.uint8)), k


def test_workspace_cache_is_per_stream_and_plan_sized(gpu):
    """The binding keeps one cached workspace per (device, stream, kind); a call on a second
    stream gets its own. The single-request draft's planned workspace holds no logits rows."""
    c = synth.custom(1310, B=1, V=151936, r=256, gamma=7, w_dtype="bf16")
    d = synth.draft_inputs(c)
    U, W1, W2 = dev(d["U"]), dev(d["W1"]), dev(d["W2"])
    path, one, nbytes = dspark.markov_draft_plan(U, W1, W2)
    assert path == "resident" and one
    lib = binding.load()
    # the general workspace also holds two logits rows (2 x V x 4 bytes) and tile partials
    assert nbytes + 2 * c.V * 4 <= lib.dspark_markov_draft_workspace_bytes(1, c.V, c.r, c.gamma)
    s2 = torch.cuda.Stream()
    a = binding.workspace(nbytes, torch.device("cuda:0"), "draft")
    b = binding.workspace(nbytes, torch.device("cuda:0"), "draft", s2)
    assert a.data_ptr() != b.data_ptr()
    x0, u = dev(d["x0"]), dev(d["u"])
    main = torch.cuda.current_stream()
    s2.wait_stream(main)
    with torch.cuda.stream(s2):                 # one-launch drafts must not overlap: in turn
        o2 = dspark.markov_draft(U, W1, W2, x0, u)
    main.wait_stream(s2)
    o1 = dspark.markov_draft(U, W1, W2, x0, u)
    torch.cuda.synchronize()
    assert np.array_equal(host(o1["x"]), host(o2["x"]))
