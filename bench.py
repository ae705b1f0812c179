"""Benchmark of the DSpark hot path on one MI355X.

One step is one pass of the whole path over one batch: Markov-head draft (gamma sequential
vocabulary sweeps) -> prefix-survival scheduler -> rejection-sampling verify of the scheduled
prefixes -> TV labels. Inputs are seeded synthetic tensors resident in HBM before timing;
the target logits stand in for the target model's forward and are generated ahead of time.

Each timed step is launched directly, as a caller of the C ABI launches it: the host enqueues
a step in about 36 us at the single-request workload, well inside the step's GPU time, so
the GPU never waits for it. The same step is also captured once into a HIP graph and
replayed (`ms_per_step_graph`): on this stack a replay adds about 9 us of GPU time per step.
Before every timed step a 512 MB buffer is read so the 256 MB Infinity Cache no longer holds
the Markov factors (the target forward that precedes drafting does the same in serving); the
flush is outside the per-step events, which bracket exactly the step on its stream (the
flush also keeps the GPU busy while the host enqueues the step, so no host gap falls inside
them).

Prints one JSON line. value = (drafted + verified tokens per step) / step time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402  (seeded inputs only)

METRIC = "Markov-head draft tokens/s + verified tokens/s at V=151936; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    "single": synth.SINGLE,   # single-request draft, B=1, V=151936, r=256, gamma=7 (the headline line)
    "batched": synth.BATCHED,  # batched draft, B=64, V=151936, gamma=16
    "verify": synth.VERIFY,   # batched verify + TV labels, B=256, V=151936, gamma=16
    "round": synth.ROUND,    # full round, B=512, V=129280, gamma=16
}
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "draft_sampling_verification_head_amd", "csrc")

# HBM bytes per dispatch of a dominant kernel, from two rocprofv3 --pmc runs (FETCH_SIZE,
# WRITE_SIZE) of this benchmark, each scaled by the same counter on a kernel of known size
# in the same run (the 512 MB flush read: fetch scale 1.9996; its fill: write scale 1.0).
# A figure holds only for the kernel sources it was measured with.
MEASURED_TRAFFIC = {
    ("single", "draft_resident"): dict(
        bytes=86696716.7,
        profile="profiles/draft_resident_single_request_B1_V151936.md",
        sources={"draft_resident.hip": "3b10cd99634f60bcf455ad08b5b56544542e0f32a11f7d72e767f4bb9f507202",
                 "draw.h": "f0ce56704c0ecddfcb12c94b365cb76428c1d65276c0e1114289aa0f5b04a122",
                 "common.h": "97b949bdb612b911538ef35847a6ba82a3dffe9004498e237d6935e1c1330f84"}),
    # the per-position sweep of one request (bench.py --per-position)
    ("single", "draft_step_gemv"): dict(
        bytes=79190153.7,
        profile="profiles/draft_step_gemv_single_request_B1_V151936.md",
        sources={"draft.hip": "48a48f93317cfc1a63460cbe3d00ebf91bb049d6b29ba4e96aeab52653667d8d",
                 "draw.h": "f0ce56704c0ecddfcb12c94b365cb76428c1d65276c0e1114289aa0f5b04a122",
                 "common.h": "97b949bdb612b911538ef35847a6ba82a3dffe9004498e237d6935e1c1330f84"}),
    ("batched", "draft_slab_resident"): dict(
        bytes=1446072095.4,
        profile="profiles/draft_slab_resident_batched_B64_V151936.md",
        sources={"draft_slab.hip": "21b13026391fbfdf5bd1eb540df939c58901b0a9cb5ba32671181343b05300f5",
                 "slab.h": "30a5c0d57967acb7597dbfd00d25a931686c28c32d439bbb8511f3ca1f0fa765",
                 "draw.h": "f0ce56704c0ecddfcb12c94b365cb76428c1d65276c0e1114289aa0f5b04a122",
                 "common.h": "97b949bdb612b911538ef35847a6ba82a3dffe9004498e237d6935e1c1330f84"}),
    # the two kernels of one dspark_verify_tv call on the sweep path (vt_sweep, vt_select)
    ("verify", "dspark_verify_tv"): dict(
        bytes=5221276587.5,
        profile="profiles/verify_tv_verify_B256_V151936.md",
        sources={"verify.hip": "efe611bd18c839ca90d544abe373e633178acc100ea6dd2072766ba3e22300bd",
                 "rows.h": "034bd45b0d847736581802a52cbc1a69584399aadbae0696fe836fb20b4fd3e8",
                 "common.h": "97b949bdb612b911538ef35847a6ba82a3dffe9004498e237d6935e1c1330f84"}),
    # one RNN-head draft call (bench.py --workload rnn): the one-launch form, and the
    # per-position form summed over its launches (rnn_state once, then per position
    # draft_step_mfma<true> and rnn_select_kernel)
    ("rnn_single", "draft_resident<true>"): dict(
        bytes=85624927.6,
        profile="profiles/rnn_draft_B1_B64_V151936.md",
        sources={"draft_resident.hip": "3b10cd99634f60bcf455ad08b5b56544542e0f32a11f7d72e767f4bb9f507202",
                 "draw.h": "f0ce56704c0ecddfcb12c94b365cb76428c1d65276c0e1114289aa0f5b04a122",
                 "common.h": "97b949bdb612b911538ef35847a6ba82a3dffe9004498e237d6935e1c1330f84"}),
    ("rnn_batched", "rnn_mfma"): dict(
        bytes=2559845665.8,
        profile="profiles/rnn_draft_B1_B64_V151936.md",
        sources={"draft_mfma.hip": "574c0084782453dbb56f6417a98d3ebace902c5086dd80af19406b4574a5982e",
                 "draw.h": "f0ce56704c0ecddfcb12c94b365cb76428c1d65276c0e1114289aa0f5b04a122",
                 "common.h": "97b949bdb612b911538ef35847a6ba82a3dffe9004498e237d6935e1c1330f84"}),
    ("round", "draft_slab_resident"): dict(
        bytes=4835505781.0,
        profile="profiles/draft_slab_resident_round_B512_V129280.md",
        sources={"draft_slab.hip": "21b13026391fbfdf5bd1eb540df939c58901b0a9cb5ba32671181343b05300f5",
                 "slab.h": "30a5c0d57967acb7597dbfd00d25a931686c28c32d439bbb8511f3ca1f0fa765",
                 "draw.h": "f0ce56704c0ecddfcb12c94b365cb76428c1d65276c0e1114289aa0f5b04a122",
                 "common.h": "97b949bdb612b911538ef35847a6ba82a3dffe9004498e237d6935e1c1330f84"}),
}


# VALU instructions of one STS fit (sts_prep + sts_stats + sts_pick; SQ_INSTS_VALU summed over
# the dispatches of one call on the STS workload), kept while the sources are unchanged.
MEASURED_VALU = {
    ("sts", "sts_fit"): dict(
        instructions=47677714,
        profile="profiles/sts_fit_N65536_G16.md",
        sources={"sts.hip": "071d3440ddd427b45792a33fe2c331c76fdf1be42a193ee2da7f1df25c289e5d",
                 "common.h": "97b949bdb612b911538ef35847a6ba82a3dffe9004498e237d6935e1c1330f84"}),
}
# VALU issue peak of the chip: 256 CUs x 4 SIMDs, one wave64 instruction per SIMD every 4
# cycles (16 lanes; fp32 and fp64 adds, multiplies and FMAs alike), at 2.4 GHz.
VALU_PEAK_GINSTR = 256 * 4 * 2.4 / 4


def sources_unchanged(sources: dict) -> bool:
    """Whether every kernel source still has the sha256 a counter figure was taken with."""
    import hashlib
    for name, digest in sources.items():
        with open(os.path.join(CSRC, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return False
    return True


def measured_traffic(workload: str, kernel: str):
    """Counter-measured bytes per dispatch, or None if absent or the sources have changed."""
    rec = MEASURED_TRAFFIC.get((workload, kernel))
    if rec is None or not sources_unchanged(rec["sources"]):
        return None
    return rec["bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS) + ["sts", "pipeline", "mfma", "rnn"],
                    default="single")
    ap.add_argument("--no-flush", action="store_true", help="keep the Infinity Cache warm")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--materialised-logits", action="store_true",
                    help="draft writes its logits and verify reads them, also where the verify "
                         "could rebuild them from the Markov factors")
    ap.add_argument("--rebuilt-logits", action="store_true",
                    help="verify rebuilds the draft logits from the Markov factors wherever the "
                         "draft takes the slab path, also past V = 131072")
    ap.add_argument("--per-position", action="store_true",
                    help="draft with DSPARK_DRAFT_PER_POSITION: launches per position instead of the "
                         "one-launch forms (one request then takes the vocabulary sweep)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="extra eager steps with no timing (for rocprofv3 runs)")
    ap.add_argument("--sub-steps", type=int, default=10,
                    help="timed steps of each sub-record of the default run (batched draft, "
                         "batched verify); 0 leaves them out")
    ap.add_argument("--sub-cpu-seconds", type=float, default=3.0,
                    help="CPU time of each sub-record's oracle baseline sample")
    return ap.parse_args()


def build_inputs(seed: int):
    import synth
    c = synth.config(seed)
    base = [synth.base_rows(c, b) for b in range(c.B)]
    U = np.stack([r[: c.gamma] for r in base])
    Lt = np.stack([synth.target_rows(c, b, base[b]) for b in range(c.B)]).reshape(-1, c.V)
    del base
    w1, w2 = synth.factors(c)
    u_acc, u_fin = synth.verify_uniforms(c)
    return c, dict(U=U, W1=w1, W2=w2, x0=synth.x0(c), u=synth.draft_uniforms(c), Lt=Lt,
                   conf=synth.confidences(c), temp=synth.temperatures(c.gamma),
                   sps=synth.sps_table(4096), u_acc=u_acc, u_fin=u_fin)


def to_dev(a, torch, device):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def draft_bytes_per_position(c, logits_written: bool = True) -> float:
    """Algorithmic HBM bytes of one draft position: W2 read, U_k read, W1 rows, L_d write (when
    the logits are written), outputs."""
    sw = 2 if c.w_dtype == "bf16" else 4
    return (c.r * c.V * sw + c.B * c.V * 4 + c.B * c.r * sw + c.B * 12 +
            (c.B * c.V * 4 if logits_written else 0))


def draft_bytes_one_launch(c, logits_written: bool = True) -> float:
    """Algorithmic HBM bytes of a draft call that draws every position in one launch with W2
    held on chip: W2 read once, then per position U_k, the W1 rows (or nothing more for the
    state), the outputs and the logits row when written."""
    sw = 2 if c.w_dtype == "bf16" else 4
    per_pos = c.B * c.V * 4 + c.B * c.r * sw + c.B * 12 + (c.B * c.V * 4 if logits_written else 0)
    return c.r * c.V * sw + c.gamma * per_pos


def verify_bytes_read_once(c) -> float:
    """Algorithmic HBM bytes of a verify + TV call: every verified draft and target row read
    once (gamma draft rows, gamma + 1 target rows per request), plus the outputs."""
    return c.B * (2 * c.gamma + 1) * c.V * 4 + c.B * (3 * c.gamma + 2) * 4


def measured_peaks(torch, device) -> dict:
    """What this GPU reaches on plain library work, beside the published peaks: a 1 GiB fp32
    device-to-device copy (bytes read + written over its time) and a bf16 8192^3 matmul
    (torch / hipBLASLt), each timed with HIP events over 10 calls after 3 warm-up calls."""
    def timed(fn, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / n

    src = torch.ones(1 << 28, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    copy_gbs = 2 * src.numel() * 4 / timed(lambda: dst.copy_(src)) / 1e9
    del src, dst
    n = 8192
    x = torch.ones((n, n), dtype=torch.bfloat16, device=device)
    y = torch.ones((n, n), dtype=torch.bfloat16, device=device)
    mm_tflops = 2.0 * n ** 3 / timed(lambda: torch.matmul(x, y)) / 1e12
    del x, y
    torch.cuda.empty_cache()
    return dict(hbm_copy_gbs=copy_gbs, bf16_matmul_tflops=mm_tflops,
                how="1 GiB fp32 copy_ (read + write bytes); bf16 8192^3 torch.matmul")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def all_core_threads() -> int:
    """Threads for the all-cores oracle leg: the cores this process may run on, capped by
    OMP_NUM_THREADS where that is set (the CPU share of the machine)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(cap))) if cap and cap.isdigit() else n


def cpu_baseline(c, inp, seconds: float, verify_only: bool = False, threads: int = 1) -> dict:
    """The fp64 oracle on the same step, with `threads` BLAS / OpenMP threads, repeated for
    about `seconds`."""
    from threadpoolctl import threadpool_limits
    import oracle

    reqs = list(range(min(c.B, 2)))       # a bounded sample of requests
    G, V = c.gamma, c.V
    tokens = 0
    t0 = time.perf_counter()
    steps = 0
    with threadpool_limits(limits=threads):
        while True:
            Lt = inp["Lt"].reshape(c.B, G + 1, V)[reqs].reshape(-1, V)
            if verify_only:
                Ld = inp["U"][reqs]
                x = np.array([[oracle.inverse_cdf(oracle.softmax_row(Ld[i, k])[0], 0.5)
                               for k in range(G)] for i in range(len(reqs))])
                oracle.verify(Ld, Lt, x, inp["u_acc"][reqs], inp["u_fin"][reqs])
                oracle.tv_labels(Ld, Lt)
                tokens += len(reqs) * G
            else:
                d = oracle.markov_draft(inp["U"][reqs], inp["W1"], inp["W2"], inp["x0"][reqs],
                                        inp["u"][reqs], c.w_dtype, want_logits=True)
                s = oracle.schedule(inp["conf"][reqs], inp["temp"], inp["sps"], 4096)
                oracle.verify(d["L"], Lt, d["x"], inp["u_acc"][reqs], inp["u_fin"][reqs],
                              length=s["len"])
                oracle.tv_labels(d["L"], Lt, length=s["len"])
                tokens += len(reqs) * G + int(s["len"].sum())
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds or el * (steps + 1) / steps > 30.0:
                break
    return dict(value=tokens / el, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{steps} oracle steps over requests {reqs} of the same workload "
                       f"({'verify + TV' if verify_only else 'draft + schedule + verify + TV'}, "
                       f"fp64, {threads} thread{'s' if threads > 1 else ''}), {el:.1f} s",
                cpu=cpu_model())


def bench_sts(args, torch, dspark, device):
    """Timing of the per-position temperature fit (STS) on synthetic validation pairs:
    N = 65536 requests, gamma = 16, 64 grid temperatures, 15 bins, NLL objective. Scores
    are Beta(6, 2); verification of a block stops at its first rejection, position k being
    accepted with probability sigmoid(logit(c) / T_k), T_k from 0.6 to 2.4."""
    from oracle import sts as oracle_sts
    g = np.random.default_rng(2024)
    N, G, nT, bins = 65536, 16, 64, 15
    conf = g.beta(6, 2, size=(N, G)).astype(np.float32)
    T_true = np.linspace(0.6, 2.4, G)
    q = np.stack([1.0 / (1.0 + ((1.0 - conf[:, k].astype(np.float64)) / conf[:, k]) ** (1.0 / T_true[k]))
                  for k in range(G)], axis=1)
    acc = g.random((N, G)) < q
    n_acc = np.where(acc.all(axis=1), G, np.argmin(acc, axis=1)).astype(np.int32)
    grid = np.linspace(0.3, 3.0, nT).astype(np.float32)
    tc, tn, tg = (torch.from_numpy(a).to(device) for a in (conf, n_acc, grid))
    for _ in range(max(1, args.warmup)):
        dspark.sts_fit(tc, tn, tg, bins=bins)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        a.record()
        out = dspark.sts_fit(tc, tn, tg, bins=bins)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # the method's work: every observed pair at every grid temperature and at T = 1
    obs = 0
    for k in range(G):
        obs += int(np.sum((k < n_acc) | ((k == n_acc) & (n_acc < G))))
    evals = obs * (nT + 1)
    rec = MEASURED_VALU[("sts", "sts_fit")]
    instr = rec["instructions"] if rec["instructions"] and sources_unchanged(rec["sources"]) else None
    achieved = None if instr is None else instr / (ms * 1e-3) / 1e9
    roofline = dict(bound="alu", kernel="sts_fit (sts_prep + sts_stats + sts_pick)",
                    achieved=achieved, peak=VALU_PEAK_GINSTR, unit="G VALU instr/s",
                    frac=None if achieved is None else achieved / VALU_PEAK_GINSTR, traffic=None,
                    evaluations_per_call=evals,
                    lane_instr_per_evaluation=None if instr is None else instr * 64 / evals,
                    evaluations_per_s=evals / (ms * 1e-3),
                    timing="HIP events around each call (three launches)",
                    instructions=f"SQ_INSTS_VALU of one call, {rec['profile']}")
    res = dict(metric="STS per-position temperature fit: validation pairs per second",
               value=N * G / (ms * 1e-3), unit="pairs/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=ms, higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="f64", data="synthetic",
               config=dict(workload="STS fit", N=N, gamma=G, grid=nT, bins=bins, objective="nll"),
               T=[round(float(v), 4) for v in out["T"].cpu()],
               ece_before=float(out["ece_before"].mean()), ece_after=float(out["ece_after"].mean()),
               roofline=roofline)
    if args.cpu_seconds > 0:
        import time
        from threadpoolctl import threadpool_limits
        fits, t0 = 0, time.perf_counter()
        with threadpool_limits(limits=1):
            while True:
                oracle_sts.sts_fit(conf, n_acc, None, grid, bins=bins)
                fits += 1
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds:
                    break
        res["cpu_baseline"] = dict(value=fits * N * G / el, unit="pairs/s", cores=1, kind="oracle",
                                   sample=f"{fits} fp64 oracle fits of the same {N} x {G} pairs "
                                          f"and {nT} temperatures, one thread, {el:.1f} s")
    print(json.dumps(res), flush=True)


def bench_rnn(args, torch, dspark, device):
    """The RNN head's draft (h_1 = W1[x_0], h_k = A h_{k-1} + W1[x_{k-1}], B_k = h_k W2) on
    the single-request shapes (B = 1, V = 151936, r = 256, gamma = 7: one launch with W2 in
    registers and A in LDS) and the batched shapes (B = 64, gamma = 16: per position an MFMA
    projection launch, whose extra workgroups form A h_k meanwhile, and a draw launch that
    adds the drawn token's W1 row to finish h_{k+1}). Factors, base logits, context tokens and
    uniforms are those of the Markov workloads, A ~ N(0, (0.5 / sqrt(r))^2). Each call is
    launched directly and timed with HIP events, the Infinity Cache flushed before it.
    Algorithmic bytes per call: the one-launch form reads W2 and A once, then per position
    U_k and the W1 rows; the per-position form reads W2 at every position and writes the
    logits rows the draw reads, plus the state rows (hi and lo bf16) and A."""
    import synth
    from oracle import rnn as oracle_rnn
    flush = torch.ones(128 << 20, dtype=torch.float32, device=device)
    recs = {}
    for name, preset in (("single", synth.SINGLE), ("batched", synth.BATCHED)):
        c = synth.config(preset)
        B, V, r, G = c.B, c.V, c.r, c.gamma
        w1, w2 = synth.factors(c)
        a = synth.rnn_factor(c)
        U_h = np.stack([synth.base_rows(c, b)[:G] for b in range(B)])
        x0_h, u_h = synth.x0(c), synth.draft_uniforms(c)
        W1, W2, A, U, x0, u = (to_dev(x, torch, device) for x in (w1, w2, a, U_h, x0_h, u_h))
        path = dspark.rnn_draft_path(B, W1, W2, A)

        def call():
            return dspark.rnn_draft(U, W1, W2, A, x0, u)

        for _ in range(max(1, args.warmup)):
            out = call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for e0, e1 in ev:
            flush.sum()
            e0.record()
            out = call()
            e1.record()
        torch.cuda.synchronize()
        us = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3
        x = out["x"].cpu().numpy()
        assert ((x >= 0) & (x < V)).all()
        if path == "resident":
            moved = r * V * 2 + r * r * 2 + G * (B * V * 4 + B * r * 2 + B * 12)
            limiter = ("latency: W2 and A loaded once, then per position three cross-CU "
                       "hand-overs (as the Markov head's one-launch draft)")
        else:
            moved = G * (draft_bytes_per_position(c, True) + B * r * 2 * 2 + r * r * 2)
            limiter = "HBM: W2, U_k and the logits rows per position"
        achieved = moved / (us * 1e-6) / 1e9
        key = ("rnn_single", "draft_resident<true>") if path == "resident" else ("rnn_batched", "rnn_mfma")
        traffic = measured_traffic(*key)
        recs[name] = dict(B=B, V=V, r=r, gamma=G, path=path, draft_us=us,
                          draft_tok_s=B * G / (us * 1e-6),
                          roofline=dict(bound="hbm", kernel=("draft_resident<true>" if path == "resident" else
                                                              "draft_step_mfma<true> + rnn_select per position"),
                                        achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                                        frac=achieved / HBM_PEAK_GBS, traffic=traffic,
                                        physical_gbs=None if traffic is None else traffic / (us * 1e-6) / 1e9,
                                        bytes_per_call=moved, limiter=limiter,
                                        timing="HIP events around each call, median"))
        if name == "single" and args.cpu_seconds > 0:
            import time
            from threadpoolctl import threadpool_limits
            n, t0 = 0, time.perf_counter()
            with threadpool_limits(limits=1):
                while True:
                    oracle_rnn.rnn_draft(U_h, w1, w2, a, x0_h, u_h, w_dtype="bf16")
                    n += 1
                    el = time.perf_counter() - t0
                    if el >= args.cpu_seconds:
                        break
            recs[name]["cpu_baseline"] = dict(
                value=n * B * G / el, unit="draft tokens/s", cores=1, kind="oracle",
                sample=f"{n} fp64 oracle drafts of the single-request workload "
                       f"({B} x {G} tokens at V = {V}), one thread, {el:.1f} s")
        del U, W1, W2, A, x0, u, out
        torch.cuda.empty_cache()
    one = recs["single"]
    res = dict(metric="RNN-head draft tokens/s at V=151936", value=one["draft_tok_s"],
               unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
               ms_per_step=one["draft_us"] / 1e3, higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16", data="synthetic",
               config=dict(workload="RNN-head draft, single request", B=1, V=one["V"], r=one["r"],
                           gamma=one["gamma"], factors="bf16", mall_flush=True, launch="direct"),
               roofline=one["roofline"], path=one["path"],
               sub_workloads=dict(batched=recs["batched"]))
    if "cpu_baseline" in one:
        res["cpu_baseline"] = one["cpu_baseline"]
    print(json.dumps(res), flush=True)


def bench_pipeline(args, torch, dspark, device):
    """The asynchronous round on the round workload's shapes (B=512, V=129280, gamma=16):
    [P1] "硬件感知与置信度自适应调度机制" (the asynchronous adaptation) and [P3]
    "Confidence-Scheduled Verification". Step t is scheduled from the confidences of step
    t - 2 (dspark_schedule_lagged over a dspark_conf_ring), so the schedule depends on
    nothing this round produces and no host round trip is needed: the whole round (lagged
    schedule, draft, verify + TV on the rebuilt draft logits, push of this round's
    confidences) is one captured graph. Variants, each run as `steps` rounds back to back
    with no host synchronisation between rounds (the Infinity Cache flushed before each
    round, outside the round's events); the variants take turns over three passes and each
    reports the median of its three per-pass means:
      graph              the captured round, schedule before the draft (the `value`);
      graph_overlapped   the captured round with the schedule on a second stream beside the
                         draft;
      eager              the same launches issued from the host each round;
      eager_sync         the synchronous scheduler the pages contrast it with: the schedule
                         uses this round's confidences, so it runs after the draft, and the
                         host reads the verify batch size before it launches verify.
    bubble_us = eager_sync - graph per round: the host handshake that the lag removes. The
    same four variants also run on the first 32 requests (`small_batch`), where a round is
    short and fixed per-round costs weigh more."""
    c, inp = build_inputs(WORKLOADS["round"])
    full = {k: to_dev(v, torch, device) for k, v in inp.items()}
    G, V = c.gamma, c.V
    Bmax = 4096
    flush = torch.ones(128 << 20, dtype=torch.float32, device=device)

    def sequence(fn, n):
        """n rounds back to back; each round's GPU span from events recorded after its flush
        and after its last launch (no host synchronisation between rounds)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in ev:
            if not args.no_flush:
                flush.sum()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def measure(B):
        """The four variants on the first B requests of the workload."""
        t = dict(full)
        for k in ("U", "x0", "u", "conf", "u_acc", "u_fin"):
            t[k] = full[k][:B].contiguous()
        t["Lt"] = full["Lt"][: B * (G + 1)]
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        out_d = dict(x=torch.empty((B, G), **i32), q=torch.empty((B, G), **f32),
                     lse=torch.empty((B, G), **f32), L=None)
        out_s = dict(len=torch.empty(B, **i32), t_off=torch.empty(B + 1, **i32),
                     K=torch.empty(1, **i32), theta=torch.empty(1, **f32))
        out_v = dict(n=torch.empty(B, **i32), y=torch.empty((B, G + 1), **i32),
                     lse_t=torch.empty((B, G + 1), **f32), cstar=torch.empty((B, G), **f32))
        ring = dspark.ConfRing(B, G, device=device)
        side = torch.cuda.Stream(device=device)

        def draft():
            dspark.markov_draft(t["U"], t["W1"], t["W2"], t["x0"], t["u"], out=out_d)

        def verify():
            dspark.verify_markov(t["U"], t["W1"], t["W2"], t["x0"], out_d["x"], out_d["lse"],
                                 t["Lt"], t["u_acc"], t["u_fin"], t_off=out_s["t_off"],
                                 length=out_s["len"], out=out_v)

        def round_async(overlap: bool):
            main = torch.cuda.current_stream()
            if overlap:
                side.wait_stream(main)
                with torch.cuda.stream(side):
                    dspark.schedule_lagged(ring, t["sps"], Bmax, temp=t["temp"], out=out_s)
                draft()
                main.wait_stream(side)
            else:
                dspark.schedule_lagged(ring, t["sps"], Bmax, temp=t["temp"], out=out_s)
                draft()
            verify()
            ring.push(t["conf"])

        def round_sync():
            draft()
            dspark.schedule(t["conf"], t["sps"], Bmax, temp=t["temp"], out=out_s)
            int(out_s["K"].item())                    # the host handshake
            verify()

        for _ in range(max(2, args.warmup)):
            round_async(True)
            round_async(False)
            round_sync()
        torch.cuda.synchronize()
        graphs = {}
        for name, overlap in (("graph", False), ("graph_overlapped", True)):
            graphs[name] = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graphs[name]):
                round_async(overlap)
        torch.cuda.synchronize()
        for _ in range(args.profile_steps):
            graphs["graph"].replay()
        for _ in range(args.warmup):
            graphs["graph"].replay()
        variants = dict(graph=graphs["graph"].replay,
                        graph_overlapped=graphs["graph_overlapped"].replay,
                        eager=lambda: round_async(False), eager_sync=round_sync)
        runs = {name: [] for name in variants}
        means = {name: [] for name in variants}
        for _ in range(3):                            # variants interleaved, three passes
            for name, fn in variants.items():
                r = sequence(fn, args.steps)
                runs[name] += r
                means[name].append(float(np.mean(r)))
        per_round = {k: float(np.median(v)) for k, v in means.items()}
        pct = {k: [float(np.percentile(v, 10)), float(np.percentile(v, 90))] for k, v in runs.items()}
        graphs["graph"].replay()
        torch.cuda.synchronize()
        verified = int(out_s["len"].sum().item())
        return t, draft, per_round, pct, verified

    B = c.B
    small_B = 32
    _, _, small_round, _, small_verified = measure(small_B)
    t, draft, per_round, pct, verified = measure(B)
    n = args.steps
    # the draft alone (the dominant kernel): launch-stream events around eager calls, a cache
    # flush before each (the flush keeps the GPU busy while the host enqueues the call)
    draft_ms = float(np.mean(sequence(draft, n)))
    drafted = B * G
    ms_round = per_round["graph"]
    per_pos = draft_bytes_per_position(c, False)
    one = dspark.markov_draft_one_launch(B, t["W1"], t["W2"])
    kernel = "draft_slab_resident" if one else "draft_slab_step + draft_slab_select"
    units = G if one else 1
    launch_us = draft_ms * 1e3 / (1 if one else G)
    bytes_launch = draft_bytes_one_launch(c, False) if one else per_pos
    achieved = bytes_launch / (launch_us * 1e-6) / 1e9
    # the same kernel on the same shapes as the round workload: its counter record applies
    roof = dict(bound="hbm", kernel=kernel, achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=achieved / HBM_PEAK_GBS, traffic=measured_traffic("round", kernel),
                bytes_per_launch=bytes_launch, positions_per_launch=units, launch_us=launch_us,
                effective_gbs=per_pos * units / (launch_us * 1e-6) / 1e9)
    mp = measured_peaks(torch, device)
    roof["measured_peak"] = dict(mp, frac_of_copy=achieved / mp["hbm_copy_gbs"])
    res = dict(
        metric=METRIC, value=(drafted + verified) / (ms_round * 1e-3), unit="tokens/s", n_gpus=1,
        steps=n, warmup=args.warmup, ms_per_step=ms_round, higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload=f"{c.name}: asynchronous rounds (two-step-lag schedule, one captured "
                             "graph per round, rounds back to back)", B=B, V=V, r=c.r, gamma=G,
                    factors=c.w_dtype, sps="1/(0.02+1e-5 B)", Bmax=Bmax,
                    mall_flush=not args.no_flush, graph_replay=True,
                    draft_logits="rebuilt by verify from the factors"),
        drafted_per_step=drafted, verified_per_step=verified,
        pipeline_ms_per_round=per_round,
        pipeline_p10_p90=pct,
        bubble_us=(per_round["eager_sync"] - ms_round) * 1e3,
        small_batch=dict(B=small_B, ms_per_round=small_round,
                         bubble_us=(small_round["eager_sync"] - small_round["graph"]) * 1e3,
                         tokens_per_s=(small_B * G + small_verified) / (small_round["graph"] * 1e-3)),
        draft_us=draft_ms * 1e3,
        roofline=roof,
    )
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(c, inp, args.cpu_seconds, False)
        res["cpu_baseline_all_cores"] = cpu_baseline(c, inp, args.cpu_seconds, False,
                                                     threads=all_core_threads())
    print(json.dumps(res), flush=True)


# MFMA busy share of the persistent slab draft per batch size, from one rocprofv3 --pmc run of
# `--workload mfma` (SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs / (GRBM_GUI_ACTIVE x
# 1024 SIMDs), the MfmaUtil expression of rocprofiler's counter definitions). A figure holds
# only for the kernel sources it was measured with.
MEASURED_MFMA_BUSY = dict(
    util={64: 7.58, 256: 13.78, 512: 15.87, 1024: 17.26},
    profile="profiles/draft_slab_resident_mfma_sweep_V151936.md",
    sources={"draft_slab.hip": "19be639ac5edace8d1f3be5b5077b08e21960b1cead6f4683dc6d9ecc1157cee",
             "slab.h": "30a5c0d57967acb7597dbfd00d25a931686c28c32d439bbb8511f3ca1f0fa765",
             "draw.h": "43a8e1c1813a52d9afa9b7e05469d4ab43e1fc94f9fc81e6a04f463aa99ef44e",
             "common.h": "97b949bdb612b911538ef35847a6ba82a3dffe9004498e237d6935e1c1330f84"})


def bench_mfma(args, torch, dspark, device):
    """Where the MFMA rate of the batched draft rises with the batch: the persistent slab
    draft (W2 held in registers, no logits output) at V = 151936, r = 256, gamma = 16 for
    B = 64, 256, 512, 1024, the Infinity Cache flushed before each call. Per call the draft
    moves W2 once and gamma base-logit rows per request, so its arithmetic intensity is about
    2 r / 4 = 128 flop per byte however large B is, and the attainable rate is
    min(bf16 peak, intensity x 8 TB/s). Factors as the batched workload; U ~ N(0, 3^2),
    tokens and uniforms drawn on the device from a fixed seed."""
    import synth
    c = synth.config(synth.BATCHED)
    w1, w2 = synth.factors(c)
    W1, W2 = to_dev(w1, torch, device), to_dev(w2, torch, device)
    V, r, G = c.V, c.r, c.gamma
    flush = torch.ones(128 << 20, dtype=torch.float32, device=device)
    rows = []
    for B in (64, 256, 512, 1024):
        gen = torch.Generator(device=device).manual_seed(1000 + B)
        U = torch.randn((B, G, V), generator=gen, device=device) * 3.0
        x0 = torch.randint(0, V, (B,), generator=gen, device=device, dtype=torch.int32)
        u = torch.rand((B, G), generator=gen, device=device).clamp_(max=1 - 2 ** -24)
        out = dict(x=torch.empty((B, G), dtype=torch.int32, device=device),
                   q=torch.empty((B, G), dtype=torch.float32, device=device),
                   lse=torch.empty((B, G), dtype=torch.float32, device=device))
        one = dspark.markov_draft_one_launch(B, W1, W2)

        def call():
            dspark.markov_draft(U, W1, W2, x0, u, out=out)

        for _ in range(max(1, args.warmup)):
            call()
        torch.cuda.synchronize()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            flush.sum()
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
        assert bool(((out["x"] >= 0) & (out["x"] < V)).all())
        flops = 2.0 * B * r * V * G
        moved = r * V * 2 + G * (B * V * 4 + B * r * 2 + B * 12)     # W2 once, then per position
        tf = flops / (us * 1e-6) / 1e12
        attain = min(MFMA_BF16_PEAK_TFLOPS, flops / moved * HBM_PEAK_GBS / 1e3)
        row = dict(B=B, one_launch=bool(one), draft_us=us, draft_tok_s=B * G / (us * 1e-6),
                   tflops=tf, frac_peak=tf / MFMA_BF16_PEAK_TFLOPS, flop_per_byte=flops / moved,
                   attainable_tflops=attain, frac_attainable=tf / attain,
                   hbm_gbs=moved / (us * 1e-6) / 1e9)
        if MEASURED_MFMA_BUSY and sources_unchanged(MEASURED_MFMA_BUSY["sources"]):
            row["mfma_busy_pct_counters"] = MEASURED_MFMA_BUSY["util"].get(B)
        rows.append(row)
        del U, x0, u, out, g
        torch.cuda.empty_cache()
    mp = measured_peaks(torch, device)
    for row in rows:
        row["frac_of_matmul"] = row["tflops"] / mp["bf16_matmul_tflops"]
    big = rows[-1]
    res = dict(metric="batched Markov draft MFMA rate vs batch size (bf16 TFLOP/s)",
               value=big["tflops"], unit="TFLOP/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=big["draft_us"] / 1e3, higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
               config=dict(workload="MFMA sweep: persistent slab draft, no logits output",
                           V=V, r=r, gamma=G, B=[x["B"] for x in rows], mall_flush=True,
                           graph_replay=True),
               sweep=rows, measured_peak=mp)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps(dict(error="this benchmark runs on exactly one GPU; "
                                    "multi-GPU figures are not produced", n_gpus=args.gpus)))
        sys.exit(2)
    import torch
    import draft_sampling_verification_head_amd as dspark

    device = torch.device("cuda:0")
    if args.workload == "sts":
        return bench_sts(args, torch, dspark, device)
    if args.workload == "pipeline":
        return bench_pipeline(args, torch, dspark, device)
    if args.workload == "mfma":
        return bench_mfma(args, torch, dspark, device)
    if args.workload == "rnn":
        return bench_rnn(args, torch, dspark, device)
    mp = measured_peaks(torch, device)
    res = run_workload(args, args.workload, torch, dspark, device, args.steps, args.cpu_seconds, mp)
    if args.workload == "single" and args.sub_steps > 0 and not args.per_position:
        # the same protocol on the batched shapes at V = 151936 (the draft on the slab MFMA
        # path, and the verify + TV call), each its own record beside the headline
        subs = {}
        for name in ("batched", "verify"):
            sub = run_workload(args, name, torch, dspark, device, args.sub_steps,
                               args.sub_cpu_seconds, mp)
            for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data"):
                sub.pop(k, None)
            subs[name] = sub
            torch.cuda.empty_cache()
        res["sub_workloads"] = subs
    print(json.dumps(res), flush=True)


def run_workload(args, workload, torch, dspark, device, steps, cpu_seconds, mp):
    """One workload under the step protocol; returns its record (the JSON line's fields)."""
    seed = WORKLOADS[workload]
    verify_only = workload == "verify"
    c, inp = build_inputs(seed)
    t = {k: to_dev(v, torch, device) for k, v in inp.items()}
    B, G, V = c.B, c.gamma, c.V
    Bmax = 4096

    # where the draft takes the slab path, verify rebuilds the draft logits from the Markov
    # factors (dspark_verify_markov) and the draft does not write them
    # (at V > 131072 the rebuilding pass holds five 16-column tiles of W2 per wave, which
    # does not fit its registers without spills, and writing the logits is faster there)
    rebuild = (not verify_only and not args.materialised_logits and
               (V <= 131072 or args.rebuilt_logits) and
               dspark.markov_draft_path(B, t["W1"], t["W2"]) == "slab")
    out_d = dict(x=torch.empty((B, G), dtype=torch.int32, device=device),
                 q=torch.empty((B, G), dtype=torch.float32, device=device),
                 lse=torch.empty((B, G), dtype=torch.float32, device=device),
                 L=None if rebuild else torch.empty((B, G, V), dtype=torch.float32, device=device))
    out_s = dict(len=torch.empty(B, dtype=torch.int32, device=device),
                 t_off=torch.empty(B + 1, dtype=torch.int32, device=device),
                 K=torch.empty(1, dtype=torch.int32, device=device),
                 theta=torch.empty(1, dtype=torch.float32, device=device))
    out_v = dict(n=torch.empty(B, dtype=torch.int32, device=device),
                 y=torch.empty((B, G + 1), dtype=torch.int32, device=device),
                 lse_d=torch.empty((B, G), dtype=torch.float32, device=device),
                 lse_t=torch.empty((B, G + 1), dtype=torch.float32, device=device))
    out_v["cstar"] = torch.empty((B, G), dtype=torch.float32, device=device)

    if verify_only:
        # draft logits are the inputs; draft tokens x ~ p_d are drawn once, before timing, with
        # the library's own sampler (a zero Markov bias leaves softmax(L_d) unchanged)
        out_d["L"].copy_(t["U"])
        zw1 = torch.zeros((V, 1), dtype=torch.float32, device=device)
        zw2 = torch.zeros((1, V), dtype=torch.float32, device=device)
        dspark.markov_draft(t["U"], zw1, zw2, t["x0"], t["u"], out=dict(x=out_d["x"]))
        torch.cuda.synchronize()

    def draft():
        dspark.markov_draft(t["U"], t["W1"], t["W2"], t["x0"], t["u"], out=out_d,
                            per_position=args.per_position)

    def schedule():
        dspark.schedule(t["conf"], t["sps"], Bmax, temp=t["temp"], out=out_s)

    def verify():
        # verify and TV labels in one call (dspark_verify_markov or dspark_verify_tv)
        if rebuild:
            dspark.verify_markov(t["U"], t["W1"], t["W2"], t["x0"], out_d["x"], out_d["lse"],
                                 t["Lt"], t["u_acc"], t["u_fin"], t_off=out_s["t_off"],
                                 length=out_s["len"], out=out_v)
        elif verify_only:
            dspark.verify(out_d["L"], t["Lt"], out_d["x"], t["u_acc"], t["u_fin"], out=out_v,
                          with_tv=True)
        else:
            dspark.verify(out_d["L"], t["Lt"], out_d["x"], t["u_acc"], t["u_fin"],
                          length=out_s["len"], ld_lse=out_d["lse"], out=out_v, with_tv=True)

    parts = dict(verify_tv=verify) if verify_only else dict(draft=draft, schedule=schedule,
                                                           verify_tv=verify)
    # the schedule does not read this step's draft: where the draft takes the single-request
    # launch and the schedule fits one wave, the step runs both in that launch
    fused = (not verify_only and not args.per_position and
             dspark.markov_draft_schedule_fused(B, t["W1"], t["W2"], B, G))

    def draft_schedule():
        dspark.markov_draft_schedule(t["U"], t["W1"], t["W2"], t["x0"], t["u"], t["sps"], Bmax,
                                     conf=t["conf"], temp=t["temp"], out=out_d, out_sched=out_s)

    step_fns = [draft_schedule, verify] if fused else list(parts.values())
    # otherwise the schedule runs on a second stream beside the draft: the persistent draft
    # holds one compute unit per vocabulary slab, and the schedule's few workgroups take
    # compute units it leaves free (18 of 256 at V = 151936)
    overlap = not fused and not verify_only
    side = torch.cuda.Stream(device=device) if overlap else None

    def step():
        if overlap:
            main = torch.cuda.current_stream()
            side.wait_stream(main)
            with torch.cuda.stream(side):
                schedule()
            draft()
            main.wait_stream(side)
            verify()
            return
        for fn in step_fns:
            fn()

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    for _ in range(args.profile_steps):
        step()
    torch.cuda.synchronize()

    # capture one step, and each part on its own
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        step()
    g_parts = {}
    for name, fn in parts.items():
        g_parts[name] = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_parts[name]):
            fn()
    torch.cuda.synchronize()

    # reading 512 MB evicts the factors from the 256 MB Infinity Cache without leaving dirty
    # lines behind (a write-based flush would make the first draft step pay the write-back)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=device)
    verified = B * G if verify_only else int(out_s["len"].sum().item())
    drafted = 0 if verify_only else B * G

    def timed(graph, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            if not args.no_flush:
                flush.sum()
            ev[i][0].record()
            graph.replay()
            ev[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def timed_eager(fn, n):
        """Launch-stream HIP events around eager calls: the GPU time of the call's kernels
        without the graph launch (the cache flush before each call keeps the GPU busy while
        the host enqueues the events and the call, so no host gap falls inside them)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            if not args.no_flush:
                flush.sum()
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()
    ms_graph = timed(g_step, steps)
    ms = timed_eager(step, steps)
    ms_parts = {name: float(np.mean(timed(g, steps))) for name, g in g_parts.items()}
    # the dominant call on its own, for the roofline: draft (or verify + TV)
    dominant = "verify_tv" if verify_only else "draft"
    ms_kernel = float(np.mean(timed_eager(parts[dominant], steps)))
    torch.cuda.synchronize()

    ms_step = float(np.mean(ms))
    value = (drafted + verified) / (ms_step * 1e-3)
    if verify_only:
        # the method's own work: every draft and target row read once (the one-sweep form
        # reads nothing else but one chunk of the final row pair per request)
        bytes_call = verify_bytes_read_once(c)
        launch_us = ms_kernel * 1e3
        roof = dict(bound="hbm", kernel="dspark_verify_tv (vt_sweep + vt_select)",
                    achieved=bytes_call / (launch_us * 1e-6) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
        roof.update(frac=roof["achieved"] / HBM_PEAK_GBS,
                    traffic=measured_traffic("verify", "dspark_verify_tv"), bytes_per_launch=bytes_call,
                    launch_us=launch_us, call_us_graph=ms_parts[dominant] * 1e3,
                    timing="HIP events on the launch stream around eager calls",
                    limiter="HBM: one pass over the rows; per-chunk waits for the row's normalisers")
        if roof["traffic"] is not None:
            roof["physical_gbs"] = roof["traffic"] / (launch_us * 1e-6) / 1e9
    else:
        path = dspark.markov_draft_path(B, t["W1"], t["W2"])
        if args.per_position and path == "resident":
            path = "sweep"                    # one request drafted per position: the sweep
        per_pos = draft_bytes_per_position(c, not rebuild)   # algorithmic bytes of one position
        one_launch = (not args.per_position and
                      dspark.markov_draft_one_launch(B, t["W1"], t["W2"], want_logits=not rebuild))
        if one_launch:
            # one launch draws all gamma positions: W2 read once and held in registers, then
            # per position U_k (and the logits row when written)
            kernel = "draft_resident" if path == "resident" else "draft_slab_resident"
            units, launch_us = G, ms_kernel * 1e3
            bytes_launch = draft_bytes_one_launch(c, not rebuild)
            limiter = ("latency: per position three cross-CU hand-overs (tile partials to one "
                       "poller, the pick to the tile's owner, the token to all) after a GEMV "
                       "from registers" if path == "resident" else
                       "HBM stream of U_k and three flag barriers per position")
        else:
            # one step kernel per position; the per-position time also carries the draws
            kernel = {"mfma": "draft_step_mfma + draft_select",
                      "slab": "draft_slab_step + draft_slab_select"}.get(path, "draft_step_gemv")
            units, launch_us = 1, ms_kernel * 1e3 / G
            bytes_launch = per_pos
            limiter = "HBM: W2 and U_k per position"
        roof = dict(bound="hbm", kernel=kernel, achieved=bytes_launch / (launch_us * 1e-6) / 1e9,
                    peak=HBM_PEAK_GBS, unit="GB/s")
        traffic = measured_traffic(workload, kernel)
        roof.update(frac=roof["achieved"] / HBM_PEAK_GBS,
                    traffic=traffic,
                    bytes_per_launch=bytes_launch, positions_per_launch=units,
                    launch_us=launch_us, draft_path=path, call_us_graph=ms_parts[dominant] * 1e3,
                    timing="HIP events on the launch stream around eager calls",
                    limiter=limiter,
                    # the per-position sweep's bytes (W2 read at every position) over the same
                    # time: what a draft without W2 on chip would have to move
                    effective_gbs=per_pos * units / (launch_us * 1e-6) / 1e9)
        if traffic is not None:
            roof["physical_gbs"] = traffic / (launch_us * 1e-6) / 1e9
        if path in ("mfma", "slab"):
            tflops = 2.0 * B * c.r * V * units / (launch_us * 1e-6) / 1e12
            roof["mfma"] = dict(achieved=tflops, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                                frac=tflops / MFMA_BF16_PEAK_TFLOPS)
    roof["measured_peak"] = dict(mp, frac_of_copy=roof["achieved"] / mp["hbm_copy_gbs"])
    if "mfma" in roof:
        roof["mfma"]["frac_of_matmul"] = roof["mfma"]["achieved"] / mp["bf16_matmul_tflops"]
    what = "verify + TV labels" if verify_only else "draft + schedule + verify + TV labels"
    res = dict(
        metric=METRIC, value=value, unit="tokens/s", n_gpus=1, steps=steps,
        warmup=args.warmup, ms_per_step=ms_step, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload=f"{c.name}: {what} per step", B=B, V=V, r=c.r, gamma=G,
                    factors=c.w_dtype, sps="1/(0.02+1e-5 B)", Bmax=Bmax,
                    mall_flush=not args.no_flush,
                    launch="direct (the graph-replayed step: ms_per_step_graph)",
                    draft_logits=("input" if verify_only else
                                  "rebuilt by verify from the factors" if rebuild else
                                  "written by the draft"),
                    draft_launches="per position" if args.per_position else "default",
                    schedule=("none" if verify_only else
                              "in the draft's launch" if fused else
                              "its own launches, on a second stream beside the draft")),
        drafted_per_step=drafted, verified_per_step=verified,
        breakdown_us={k: v * 1e3 for k, v in ms_parts.items()},
        ms_per_step_p10_p90=[float(np.percentile(ms, 10)), float(np.percentile(ms, 90))],
        ms_per_step_graph=float(np.mean(ms_graph)),
        roofline=roof,
    )
    if not verify_only:
        res["draft_tok_s"] = drafted / (ms_parts["draft"] * 1e-3)
    res["verified_tok_s"] = verified / (ms_parts["verify_tv"] * 1e-3)
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(c, inp, cpu_seconds, verify_only)
        res["cpu_baseline_all_cores"] = cpu_baseline(c, inp, cpu_seconds, verify_only,
                                                     threads=all_core_threads())
    del t, g_step, g_parts, out_d, out_v, flush
    return res


if __name__ == "__main__":
    main()
