#!/usr/bin/env python3
"""Throughput of the jagged HSTU attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload windowed]

A step is one pass of the whole hot path (scheduler kernel + attention kernel)
over one batch of seeded synthetic inputs already resident in HBM.  Before
every timed step a 1 GiB buffer is rewritten (outside the timed events) so
that the 256 MB last-level cache holds none of the inputs.  Prints one JSON
line with valid-pair TFLOP/s, tokens/s, the attention kernel's roofline
position and the fp64 CPU oracle timed on this host as a baseline.

The default workload is the largest one that fits one GPU, the windowed
batch (16 sequences of 2048-8192 tokens, window 1024, 50 candidates each),
whose attention is bound by the bf16 matrix cores; the line also carries a
`secondary` record for the short ranking batch, bound by HBM bandwidth,
measured the same way in the same run (skip it with --no-secondary).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "jagged HSTU attn fwd TFLOP/s (valid pairs) + % bf16 MFMA peak; tokens/s"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}      # dense MFMA peaks, MI355X (256 CU x 2.4 GHz)
PEAK_HBM_GBS = 8000.0
_CSRC = "jagged_hstu_attention_attn_amd/csrc/"
# The sources each forward kernel is built from: a counter summary is valid
# for the kernel and source hash it records.
KERNEL_SOURCES = {   # the kernel and the scheduler whose work order sets its traffic
    "hstu_attn_fwd_kernel": ["attn_fwd.hip", "attn_common.hpp", "hstu_device.hpp", "plan.hip"],
    "hstu_attn_fwd_w16_kernel": ["attn_fwd_w16.hip", "attn_common.hpp", "hstu_device.hpp",
                                 "plan.hip"],
    "hstu_attn_fwd_pp_kernel": ["attn_fwd_pp.hip", "attn_common.hpp", "hstu_device.hpp",
                                "plan.hip"],
    "hstu_attn_fwd_w32_kernel": ["attn_fwd_w32.hip", "attn_common.hpp", "hstu_device.hpp",
                                 "plan.hip"],
}
KERNEL_OF_CHOICE = {"four_wave": "hstu_attn_fwd_kernel", "sixteen_row": "hstu_attn_fwd_w16_kernel",
                    "eight_wave": "hstu_attn_fwd_pp_kernel",
                    "thirtytwo_row": "hstu_attn_fwd_w32_kernel"}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def settle(step, flush, seconds: float) -> dict:
    """Untimed steps of the workload itself (cache flush included) for
    `seconds` of wall time, before the warm-up steps.  From a fresh start the
    first few dozen steps run up to ~15% slower however the warm-up count is
    set (measured on the windowed batch: steps 1-20 at 364 us, 41-60 at 310
    us; a one-off fill of the flush buffer does not remove it), so the timed
    steps start from steady state.  Reported in the JSON line as `settle`."""
    import torch
    if seconds <= 0:
        return {"steps": 0, "seconds": 0.0}
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(10):
            if flush is not None:
                flush.fill_(n & 0xFF)
            step()
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    return {"steps": n, "seconds": round(time.perf_counter() - t0, 3)}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, _CSRC + rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(inp, valid_pairs: int):
    """Algorithmic flops and HBM bytes of one forward: 2*(d_qk+d_v) flops per
    valid pair and head (the two products Q K^T and A V; masked pairs inside a
    computed tile are not counted); q, k, v, u read once, out written once,
    plus timestamps, offsets and candidate counts, and the bias tables."""
    H, dqk, dv, N, B = inp.num_heads, inp.d_qk, inp.d_v, inp.total_tokens, inp.num_seqs
    es = 2 if inp.dtype == "bf16" else 4
    flops = 2.0 * (dqk + dv) * H * valid_pairs
    byts = N * H * (2 * dqk + 3 * dv) * es
    if inp.timestamps is not None:
        byts += 8 * N
    byts += 4 * (B + 1) + (4 * B if inp.num_targets is not None else 0)
    byts += 4 * (0 if inp.pos_table is None else inp.pos_table.shape[0])
    byts += 4 * (0 if inp.time_table is None else inp.time_table.shape[0])
    return flops, byts


def candidate_rows_work(inp):
    """Valid pairs per head, flops and HBM bytes of the candidate rows alone:
    candidate i of a sequence with n_h history tokens sees the history keys
    [max(0, n_h - W), n_h) (all of them when W = 0) and itself; it reads its
    q and u, those keys' k and v, and writes its output row."""
    H, dqk, dv = inp.num_heads, inp.d_qk, inp.d_v
    es = 2 if inp.dtype == "bf16" else 4
    pairs = keys = rows = 0
    for b in range(inp.num_seqs):
        L = int(inp.offsets[b + 1] - inp.offsets[b])
        T = 0 if inp.num_targets is None else min(max(int(inp.num_targets[b]), 0), L)
        n_h = L - T
        seen = min(n_h, inp.max_attn_len) if inp.max_attn_len > 0 else n_h
        pairs += T * (seen + 1)
        keys += seen + T
        rows += T
    flops = 2.0 * (dqk + dv) * H * pairs
    byts = H * es * (rows * (dqk + 2 * dv) + keys * (dqk + dv))
    if inp.timestamps is not None:
        byts += 8 * (keys + rows)
    return pairs, flops, byts


def bench_layer(args, inp) -> int:
    """Whole-layer timing: one step = LayerNorm + projection GEMM + scheduler +
    attention + output GEMM on one batch already in HBM."""
    import torch
    from jagged_hstu_attention_attn_amd.api import HstuLayer, valid_pairs
    from jagged_hstu_attention_attn_amd.device_inputs import call_kwargs, to_device
    from jagged_hstu_attention_attn_amd.inputs import WORKLOADS
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(
        torch.bfloat16)
    L = inp.layer
    dev = to_device(inp, "cuda")
    kw = call_kwargs(inp, dev)
    lay = HstuLayer(t(L["x"]), t(L["w_uvqk"]), t(L["b_uvqk"]), t(L["w_o"]), dev["offsets"],
                    num_heads=inp.num_heads, d_qk=inp.d_qk, d_v=inp.d_v, **kw)
    N, D = L["x"].shape
    H, dqk, dv = inp.num_heads, inp.d_qk, inp.d_v
    W = H * (2 * dv + 2 * dqk)
    pairs = valid_pairs(inp.offsets, inp.num_targets, inp.contextual_len, inp.max_attn_len)
    f_proj, f_out = 2.0 * N * D * W, 2.0 * N * H * dv * D
    f_attn = 2.0 * (dqk + dv) * H * pairs
    flops = f_proj + f_attn + f_out
    flush = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    settled = settle(lay, flush, args.settle_s)
    for s in range(args.warmup):   # warm-up steps are the timed steps, flush included
        if flush is not None:
            flush.fill_(s & 0xFF)
        lay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for s, (e0, e1) in enumerate(evs):
        if flush is not None:
            flush.fill_(s & 0xFF)
        e0.record(stream)
        lay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    tflops = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "HSTU layer forward TFLOP/s (projections + valid-pair attention)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": settled, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "layer (full HSTU layer)", "num_seqs": inp.num_seqs,
                   "total_tokens": N, "hidden": D, "num_heads": H, "d_qk": dqk, "d_v": dv,
                   "valid_pairs_per_head": pairs,
                   "seed": args.seed if args.seed is not None else WORKLOADS["layer"].seed,
                   "cache_flushed": flush is not None, "parallelism": "single GPU"},
        "flops": {"projection": f_proj, "attention": f_attn, "output": f_out},
        "tokens_per_s": N / (ms * 1e-3),
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_TFLOPS["bf16"],
        "wall_s": wall,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_backward(args, inp) -> int:
    """Backward timing: one step = the whole backward call (o recomputed by
    the forward kernel when the epilogue needs it, gate backward, scheduler,
    dQ pass, dK/dV pass, table reduction) on one batch already in HBM, with
    dout given.  Flops counted: 2 (3 d_qk + 2 d_v) per valid pair and head
    (S, dA, dV, dK, dQ contractions; the recomputation is not counted)."""
    import torch
    from jagged_hstu_attention_attn_amd.api import JaggedAttnBwdCall, valid_pairs
    from jagged_hstu_attention_attn_amd.device_inputs import call_kwargs, to_device
    from jagged_hstu_attention_attn_amd.inputs import WORKLOADS
    dev = to_device(inp, "cuda")
    call = JaggedAttnBwdCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                             epilogue=args.epilogue, **call_kwargs(inp, dev))
    dt = dev["q"].dtype
    g = torch.Generator(device="cuda").manual_seed(0)
    dout = torch.randn(dev["v"].shape, generator=g, device="cuda", dtype=torch.float32).to(dt)
    o_saved = None
    if args.saved_o:
        # the training forward keeps o / n_scale; the backward then skips its recompute
        from jagged_hstu_attention_attn_amd.api import JaggedAttnCall
        fwd = JaggedAttnCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                             epilogue=args.epilogue, save_o=True, **call_kwargs(inp, dev))
        fwd()
        o_saved = fwd.o_raw
    pairs = valid_pairs(inp.offsets, inp.num_targets, inp.contextual_len, inp.max_attn_len)
    H, dqk, dv = inp.num_heads, inp.d_qk, inp.d_v
    fpp = 2.0 * (3 * dqk + 2 * dv)
    flops = fpp * H * pairs
    flush = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    log(f"backward: {inp.num_seqs} sequences, {inp.total_tokens} tokens, {pairs} valid "
        f"pairs/head; warmup {args.warmup}")
    settled = settle(lambda: call(dout, o_saved), flush, args.settle_s)
    for s in range(args.warmup):   # warm-up steps are the timed steps, flush included
        if flush is not None:
            flush.fill_(s & 0xFF)
        call(dout, o_saved)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for s, (e0, e1) in enumerate(evs):
        if flush is not None:
            flush.fill_(s & 0xFF)
        e0.record(stream)
        call(dout, o_saved)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"backward step {ms * 1e3:.1f} us, {tflops:.1f} TFLOP/s")
    result = {
        "metric": "jagged HSTU attn bwd TFLOP/s (valid pairs, 5 contractions)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": settled, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None, "dtype": inp.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "pass": "backward", "epilogue": args.epilogue,
                   "o": "saved by the training forward" if args.saved_o else "recomputed",
                   "num_seqs": inp.num_seqs, "total_tokens": inp.total_tokens,
                   "num_heads": H, "d_qk": dqk, "d_v": dv, "valid_pairs_per_head": pairs,
                   "seed": args.seed if args.seed is not None else WORKLOADS[args.workload].seed,
                   "cache_flushed": flush is not None, "parallelism": "single GPU"},
        "tokens_per_s": inp.total_tokens / (ms * 1e-3),
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_TFLOPS["bf16"],
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle backward")
        result["cpu_baseline"] = cpu_baseline(inp, fpp, args.cpu_budget, backward=True)
    print(json.dumps(result), flush=True)
    return 0


def traffic_from_profile(workload: str, kernel: str):
    """HBM bytes per attention launch from the committed counter summary, if
    it was taken on `kernel` as its source stands; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_kern = re.search(r"^kernel:\s*(\S+)", text, re.M)
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_kern or not m_sha or not m_bytes or m_kern.group(1) != kernel:
        return None
    if m_sha.group(1) != kernel_source_hash(kernel):
        return None
    return float(m_bytes.group(1))


def cpu_baseline(inp, flops_per_pair_head: float, budget_s: float, backward: bool = False):
    """The fp64 oracle, as it stands, on this host's cores over a bounded
    prefix of the batch (whole sequences), in the metric's unit."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    from jagged_hstu_attention_attn_amd.inputs import make_inputs
    nthreads = oracle.default_threads()

    def timed(x):
        if not backward:
            return oracle.timed_forward(x, nthreads=nthreads)[1]
        dout = np.random.default_rng(0).standard_normal(
            (x.total_tokens, x.num_heads, x.d_v))
        t0 = time.perf_counter()
        oracle.backward(x, dout, nthreads=nthreads)
        return time.perf_counter() - t0

    # estimate from a small prefix, then take the largest prefix within budget
    B = inp.num_seqs
    probe = make_inputs(inp.workload, num_seqs=max(1, min(B, 4)), dtype=inp.dtype)
    t_probe = timed(probe)
    pairs_probe = oracle.count_allowed(probe.offsets, probe.num_targets, probe.contextual_len,
                                       probe.max_attn_len)
    rate = pairs_probe / max(t_probe, 1e-6)
    lens = inp.lengths
    nb = B
    total_pairs = oracle.count_allowed(inp.offsets, inp.num_targets, inp.contextual_len,
                                       inp.max_attn_len)
    if total_pairs / rate > budget_s:
        lo, hi = 1, B
        while lo < hi:
            mid = (lo + hi + 1) // 2
            off = np.concatenate([[0], np.cumsum(lens[:mid])]).astype(np.int32)
            nt = None if inp.num_targets is None else inp.num_targets[:mid]
            p = oracle.count_allowed(off, nt, inp.contextual_len, inp.max_attn_len)
            if p / rate <= budget_s:
                lo = mid
            else:
                hi = mid - 1
        nb = lo
    sample = make_inputs(inp.workload, num_seqs=nb, dtype=inp.dtype) if nb < B else inp
    pairs = oracle.count_allowed(sample.offsets, sample.num_targets, sample.contextual_len,
                                 sample.max_attn_len)
    # a sample that finishes quickly is run again until about half the budget
    # has passed, so that the rate is not one short measurement
    runs, secs = 0, 0.0
    while runs == 0 or (secs < 0.5 * budget_s and runs < 1000):
        secs += timed(sample)
        runs += 1
    used = nthreads
    per_run = secs / runs
    tflops = flops_per_pair_head * sample.num_heads * pairs / per_run / 1e12
    return {
        "value": tflops, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
        "sample": (f"{nb} of {B} sequences of the {inp.workload} batch "
                   f"({sample.total_tokens} tokens, {sample.num_heads} heads, "
                   f"{'backward, ' if backward else ''}fp64 C loop, "
                   f"OpenMP over (sequence, head)), {runs} run(s), {secs:.2f} s in all"),
        "seconds": secs, "runs": runs, "tokens_per_s": sample.total_tokens / per_run,
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up (0: none)")
    ap.add_argument("--workload", default="windowed",
                    choices=["tiny", "ranking", "longtail", "windowed", "layer"])
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-flush", action="store_true", help="keep inputs cache-resident")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary (ranking, HBM-bound) record")
    ap.add_argument("--secondary-steps", type=int, default=50)
    ap.add_argument("--epilogue", default="ln_u", choices=["ln_u", "none", "ln_all_u"],
                    help="per-head LayerNorm * U (default), none, or one LayerNorm over all heads")
    ap.add_argument("--full-layer", action="store_true",
                    help="layer workload only: time the whole HSTU layer (LayerNorm, "
                         "projection GEMM, attention, output GEMM)")
    ap.add_argument("--candidates-only", action="store_true",
                    help="compute only the candidate rows (history reused; no CPU baseline)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (gradients of q, k, v, u and the bias tables)")
    ap.add_argument("--saved-o", action="store_true",
                    help="with --backward: take o / n_scale kept by the training forward")
    ap.add_argument("--fwd-kernel", default="auto",
                    choices=["auto", "four_wave", "eight_wave", "sixteen_row", "thirtytwo_row"],
                    help="forward kernel: chosen by batch shape (auto), or forced")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards by sequence with no exchange, so each GPU would run this "
              "same measurement on its own batch)",
              file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes 5 times")
        return 0

    from jagged_hstu_attention_attn_amd.api import set_fwd_kernel
    from jagged_hstu_attention_attn_amd.inputs import make_inputs

    set_fwd_kernel(args.fwd_kernel)
    log(f"workload {args.workload}: generating inputs")
    inp = make_inputs(args.workload, seed=args.seed)
    if args.full_layer:
        if inp.layer is None:
            print("--full-layer needs the layer workload", file=sys.stderr)
            return 2
        return bench_layer(args, inp)
    if args.backward:
        return bench_backward(args, inp)
    result = measure_forward(args, inp, args.workload, args.steps, args.warmup)
    if not args.no_cpu_baseline and not args.candidates_only:
        log("timing the fp64 CPU oracle")
        result["cpu_baseline"] = cpu_baseline(inp, 2.0 * (inp.d_qk + inp.d_v), args.cpu_budget)
    if (not args.no_secondary and args.workload != "ranking" and args.seed is None
            and not args.candidates_only and args.epilogue == "ln_u"):
        del inp
        log("secondary record: ranking batch")
        sec_inp = make_inputs("ranking")
        sec = measure_forward(args, sec_inp, "ranking", args.secondary_steps, args.warmup)
        keep = ("value", "unit", "ms_per_step", "steps", "warmup", "settle", "config",
                "tokens_per_s",
                "pct_bf16_mfma_peak", "pct_hbm_peak", "plan_us", "roofline")
        result["secondary"] = {k: sec[k] for k in keep}
        result["secondary"]["why"] = ("the short ranking batch, whose attention is bound by HBM "
                                      "bandwidth (arithmetic intensity 31 flop/B)")
    print(json.dumps(result), flush=True)
    return 0


def measure_forward(args, inp, workload: str, steps: int, warmup: int) -> dict:
    """Times `steps` forward steps (scheduler + attention) of one batch after
    `warmup` untimed ones, then the same steps again with the attention
    kernel's own start/end events; returns the result record."""
    import torch
    from jagged_hstu_attention_attn_amd.api import JaggedAttnCall, valid_pairs
    from jagged_hstu_attention_attn_amd.device_inputs import call_kwargs, to_device
    from jagged_hstu_attention_attn_amd.inputs import WORKLOADS

    dev = to_device(inp, "cuda")
    call = JaggedAttnCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                          candidates_only=args.candidates_only, epilogue=args.epilogue,
                          **call_kwargs(inp, dev))
    if args.candidates_only:
        pairs, flops, byts = candidate_rows_work(inp)
    else:
        pairs = valid_pairs(inp.offsets, inp.num_targets, inp.contextual_len, inp.max_attn_len)
        flops, byts = algorithmic(inp, pairs)
    flush = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    log(f"{workload}: {inp.num_seqs} sequences, {inp.total_tokens} tokens, {pairs} valid "
        f"pairs/head; warmup {warmup}")
    def fwd_step():
        call.plan()
        call.run()
    settled = settle(fwd_step, flush, args.settle_s)
    log(f"{workload}: settled over {settled['steps']} untimed steps ({settled['seconds']} s)")
    # Warm-up steps are the timed steps (flush, scheduler, attention).
    for s in range(warmup):
        if flush is not None:
            flush.fill_(s & 0xFF)
        call.plan()
        call.run()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    steps_ev = [(ev(), ev()) for _ in range(steps)]        # around each step
    parts_ev = [(ev(), ev(), ev()) for _ in range(steps)]  # around scheduler / launch
    # the attention kernel's own start / end times (hipExtLaunchKernelGGL);
    # an event exists once recorded
    kev = [(ev(), ev()) for _ in range(steps)]
    for k0, k1 in kev:
        k0.record(stream)
        k1.record(stream)
    log(f"{workload}: timing {steps} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for s in range(steps):
        if flush is not None:
            flush.fill_(s & 0xFF)
        e0, e1 = steps_ev[s]
        e0.record(stream)
        call.plan()
        call.run()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # The same steps again for the parts: markers around the scheduler and the
    # attention launch, the attention launched with events at its own start
    # and end (markers inside a step and a launch that records events both
    # lengthen it, so the step times above come from plain steps).
    log(f"{workload}: timing the scheduler and the attention kernel over {steps} more steps")
    for s in range(steps):
        if flush is not None:
            flush.fill_(s & 0xFF)
        m0, m1, m2 = parts_ev[s]
        m0.record(stream)
        call.plan()
        m1.record(stream)
        call.run_timed(*kev[s])
        m2.record(stream)
    torch.cuda.synchronize()
    step_ms = [e0.elapsed_time(e1) for e0, e1 in steps_ev]
    plan_ms = [m0.elapsed_time(m1) for m0, m1, _ in parts_ev]
    launch_ms = [m1.elapsed_time(m2) for _, m1, m2 in parts_ev]
    attn_ms = [k0.elapsed_time(k1) for k0, k1 in kev]
    ms = sum(step_ms) / len(step_ms)
    attn = sum(attn_ms) / len(attn_ms)
    launch = sum(launch_ms) / len(launch_ms)
    plan = sum(plan_ms) / len(plan_ms)
    log(f"{workload}: step {ms * 1e3:.1f} us (plan {plan * 1e3:.1f} us, attention kernel "
        f"{attn * 1e3:.1f} us, {launch * 1e3:.1f} us between markers around its launch), "
        f"wall {wall:.3f} s")

    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[inp.dtype]
    ai = flops / byts
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if ai >= ridge else "hbm"
    if bound == "hbm":
        achieved = byts / (attn * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = flops / (attn * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    kernel = KERNEL_OF_CHOICE.get(call.kernel_name(), "hstu_attn_fwd_kernel")
    traffic = (None if args.candidates_only or args.epilogue != "ln_u"
               else traffic_from_profile(workload, kernel))
    roof["traffic"] = traffic
    roof["traffic_source"] = (
        f"profiles/attn_fwd_{workload}_traffic.md: rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE "
        "runs of bench.py, scaled by the copy calibration, taken on this kernel's current source"
        if traffic is not None else
        "null: no counter summary taken on this kernel's current source")
    roof["kernel"] = kernel
    roof["kernel_us"] = attn * 1e3
    roof["kernel_timing"] = ("HIP events taken at the kernel's own start and end, over a "
                             "second pass of the same steps")
    roof["launch_us"] = launch * 1e3
    roof["algorithmic_bytes"] = byts
    roof["algorithmic_flops"] = flops

    return {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "settle": settled,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic",
        "config": {
            "workload": workload,
            "rows": "candidates" if args.candidates_only else "all",
            "epilogue": args.epilogue,
            "num_seqs": inp.num_seqs,
            "total_tokens": inp.total_tokens,
            "num_heads": inp.num_heads,
            "d_qk": inp.d_qk,
            "d_v": inp.d_v,
            "valid_pairs_per_head": pairs,
            "seed": args.seed if args.seed is not None else WORKLOADS[workload].seed,
            "cache_flushed": flush is not None,
            "parallelism": "single GPU",
        },
        "tokens_per_s": inp.total_tokens / (ms * 1e-3),
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_TFLOPS["bf16"],
        "pct_hbm_peak": 100.0 * byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "plan_us": plan * 1e3,
        "wall_s": wall,
        "roofline": roof,
    }


if __name__ == "__main__":
    sys.exit(main())
