"""HIP path against the fp64 oracle, element by element, on seeded inputs.

Tolerances: max|gpu - oracle| <= 1e-5 * max|oracle| for fp32 and
<= 1e-2 * max|oracle| for bf16, over the whole output (or over the sampled
rows for full-size long workloads, which the oracle evaluates row by row).
Masked / padded positions must match exactly (zero-pattern test).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from jagged_hstu_attention_attn_amd.api import HstuLayer, JaggedAttnCall, jagged_attn_fwd
from jagged_hstu_attention_attn_amd.device_inputs import call_kwargs, to_device
from jagged_hstu_attention_attn_amd.inputs import JaggedInputs, make_custom, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}
DEV = "cuda:0"


def gpu_forward(inp, epilogue="ln_u", ld=None, out=None, pos_clamp=False):
    dev = to_device(inp, DEV, ld=ld)
    o = jagged_attn_fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                        epilogue=epilogue, out=out, pos_clamp=pos_clamp,
                        **call_kwargs(inp, dev))
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


def assert_close(gpu, ref, dtype, rows=None):
    if rows is not None:
        gpu, ref = gpu[rows], ref[rows]
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    scale = np.abs(ref).max()
    err = np.abs(gpu - ref).max()
    assert err <= TOL[dtype] * scale, f"max err {err:.3e} vs bound {TOL[dtype] * scale:.3e}"
    return err / max(scale, 1e-300)


def ora(inp, epilogue="ln_u", rows=None, pos_clamp=False):
    ep = {"ln_u": oracle.EPILOGUE_LN_U, "none": oracle.EPILOGUE_NONE,
          "ln_all_u": oracle.EPILOGUE_LN_ALL_U}[epilogue]
    return oracle.forward(inp, epilogue=ep, rows=rows, pos_clamp=pos_clamp)


# ---------------------------------------------------------------------------
# Worked example of "HSTU tensor by tensor", section "SiLU aggregation
# coefficients are not probabilities", on the device.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d", [("f32", 8), ("bf16", 128), ("f32", 128), ("bf16", 256)])
def test_worked_example(dtype, d):
    inp = make_custom([2], d_qk=d, d_v=d, dtype=dtype, alpha=1.0, n_scale=1.0)
    inp.q[:] = 0; inp.k[:] = 0; inp.v[:] = 0; inp.u[:] = 1
    inp.q[1, 0, 0] = 1.0
    inp.k[0, 0, 0] = -1.0; inp.k[1, 0, 0] = 1.0
    inp.v[0, 0, 0] = 1.0; inp.v[1, 0, 1] = 1.0
    out = gpu_forward(inp, epilogue="none")
    tol = 1e-6 if dtype == "f32" else 4e-3
    assert abs(out[1, 0, 0] - (-0.2689414214)) < tol
    assert abs(out[1, 0, 1] - 0.7310585786) < tol
    assert np.all(out[1, 0, 2:] == 0) and np.all(out[0] == 0)


# ---------------------------------------------------------------------------
# Named workloads.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("epilogue", ["ln_u", "none"])
def test_tiny_workload(epilogue):
    inp = make_inputs("tiny")
    assert_close(gpu_forward(inp, epilogue), ora(inp, epilogue), "f32")


@pytest.mark.parametrize("seed", [1234, 1, 2, 3, 4])
def test_ranking_workload_full(seed):
    inp = make_inputs("ranking", seed=seed)
    assert_close(gpu_forward(inp), ora(inp), "bf16")


def test_ranking_workload_epilogue_none():
    inp = make_inputs("ranking", seed=7)
    assert_close(gpu_forward(inp, "none"), ora(inp, "none"), "bf16")


@pytest.mark.parametrize("name", ["ranking", "longtail", "windowed"])
def test_fp32_shadow(name):
    """Same geometry in fp32 separates logic errors from bf16 rounding."""
    inp = make_inputs(name, num_seqs={"ranking": 16, "longtail": 6, "windowed": 1}[name],
                      dtype="f32")
    assert_close(gpu_forward(inp), ora(inp), "f32")


@pytest.mark.parametrize("seed", [1234, 2])
def test_longtail_reduced_full(seed):
    inp = make_inputs("longtail", seed=seed, num_seqs=8)
    assert_close(gpu_forward(inp), ora(inp), "bf16")


def _sample_rows(inp, n, seed):
    rng = np.random.default_rng(seed)
    N = inp.total_tokens
    rows = set(rng.choice(N, size=min(n, N), replace=False).tolist())
    # plus the last rows of the longest sequence and the first/last token of each sequence
    b = int(np.argmax(inp.lengths))
    rows |= set(range(int(inp.offsets[b + 1]) - 64, int(inp.offsets[b + 1])))
    rows |= set(int(x) for x in inp.offsets[:-1]) | set(int(x) - 1 for x in inp.offsets[1:])
    return np.array(sorted(r for r in rows if 0 <= r < N))


@pytest.mark.parametrize("name", ["longtail", "windowed"])
def test_full_size_sampled_rows(name):
    inp = make_inputs(name)
    rows = _sample_rows(inp, 400, 5)
    assert_close(gpu_forward(inp), ora(inp, rows=rows), "bf16", rows=rows)


@pytest.mark.parametrize("seed", [1234, 1, 2, 3, 4])
@pytest.mark.parametrize("name", ["longtail", "windowed"])
def test_long_workloads_whole_output(name, seed):
    """The whole output of the full-size long-tail and windowed batches (the
    configuration the benchmark times) against the whole fp64 oracle."""
    print(f"case whole {name} seed {seed}", flush=True)
    inp = make_inputs(name, seed=seed)
    assert_close(gpu_forward(inp), ora(inp), "bf16")


def _zero_pattern_windows(inp, epilogue_rows=128):
    """Zero pattern of every allowed / masked pair of a one-sequence batch:
    for each window of 128 keys [j0, j0 + 128), V is one-hot over the window
    (key j0 + e sets column e), so with epilogue NONE out[i, e] = a_{i, j0+e},
    nonzero exactly where the pair is allowed (scores stay away from 0)."""
    assert inp.num_seqs == 1 and inp.num_heads == 1 and inp.d_v == 128
    L = int(inp.lengths[0])
    T = 0 if inp.num_targets is None else int(inp.num_targets[0])
    mask = oracle._dense_mask(L, T, inp.contextual_len, inp.max_attn_len, L)
    for j0 in range(0, L, epilogue_rows):
        inp.v[:] = 0
        for e in range(min(epilogue_rows, L - j0)):
            inp.v[j0 + e, 0, e] = 1.0
        out = gpu_forward(inp, "none")[:, 0, :]
        w = min(epilogue_rows, L - j0)
        got = out[:, :w] != 0
        bad = np.argwhere(got != mask[:, j0:j0 + w])
        assert bad.size == 0, f"window {j0}: {len(bad)} pairs differ, first (i, j) = " \
                              f"{(int(bad[0][0]), j0 + int(bad[0][1]))}"
        assert np.all(out[:, w:] == 0)


def test_zero_pattern_windowed_sequence():
    """A windowed sequence of 2600 tokens (window 1024, 50 candidates whose
    window is clamped at the history end): every query tile, both window
    edges, the candidate block and the split items of the static plan."""
    print("case zero pattern windowed", flush=True)
    inp = make_custom([2600], num_heads=1, d_qk=128, d_v=128, dtype="bf16", seed=41,
                      num_targets=[50], max_attn_len=1024, pos_len=4096, pos_std=0.2,
                      time_len=64, alpha=0.05)
    _zero_pattern_windows(inp)


def test_zero_pattern_longtail_sequence():
    """A long causal sequence with a 6-token bidirectional prefix, long enough
    that its last query tiles are split along the keys."""
    print("case zero pattern longtail", flush=True)
    inp = make_custom([3000], num_heads=1, d_qk=128, d_v=128, dtype="bf16", seed=42,
                      contextual_len=6, pos_len=4096, pos_std=0.2, time_len=64, alpha=0.05)
    _zero_pattern_windows(inp)


def test_windowed_one_sequence_full():
    inp = make_inputs("windowed", num_seqs=1)
    assert_close(gpu_forward(inp), ora(inp), "bf16")


def test_layer_strided_views():
    """Views with token stride 2048 (slices of a fused U|V|Q|K projection)."""
    inp = make_inputs("layer", num_seqs=6)
    a = gpu_forward(inp, ld=2048)
    b = gpu_forward(inp)
    assert np.array_equal(a, b)
    assert_close(a, ora(inp), "bf16")


# ---------------------------------------------------------------------------
# Edge cases: ragged tails around the 32-key / 128-row tiles, empty
# sequences, all-candidate sequences, prefix longer than the history, windows
# at the tile size, large absolute timestamps and spans beyond 2^30 s.
# ---------------------------------------------------------------------------
EDGE_LENGTHS = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257, 300]


@pytest.mark.parametrize("dtype,d", [("f32", 8), ("bf16", 128), ("bf16", 64), ("f32", 64),
                                     ("bf16", 256)])
@pytest.mark.parametrize("rules", ["causal", "targets", "prefix", "window", "all"])
def test_edges(dtype, d, rules):
    rng = np.random.default_rng(hash(rules) % 1000)
    lengths = list(EDGE_LENGTHS)
    B = len(lengths)
    nt = None
    c = W = 0
    if rules in ("targets", "all"):
        nt = [int(x) for x in rng.integers(0, 40, size=B)]
        nt[1] = 1; nt[3] = 31; nt[7] = 64       # all-candidate / exact-tile cases
    if rules in ("prefix", "all"):
        c = 6 if rules == "all" else 40
    if rules in ("window", "all"):
        W = {"window": 32, "all": 33}[rules]
    inp = make_custom(lengths, num_heads=2, d_qk=d, d_v=d, dtype=dtype, seed=11,
                      num_targets=nt, contextual_len=c, max_attn_len=W, pos_len=300,
                      pos_std=0.3, time_len=64, time_std=0.3, alpha=1.0 / math.sqrt(d),
                      t0=(1 << 33) + 17)
    for ep in ("ln_u", "none"):
        assert_close(gpu_forward(inp, ep), ora(inp, ep), dtype)


@pytest.mark.parametrize("W", [1, 31, 32, 33, 127, 128, 129])
def test_window_sizes(W):
    inp = make_custom([700, 129], num_heads=1, d_qk=128, d_v=128, dtype="bf16", seed=W,
                      num_targets=[25, 3], max_attn_len=W, pos_len=1024, time_len=64,
                      alpha=1 / math.sqrt(128))
    assert_close(gpu_forward(inp), ora(inp), "bf16")


def test_no_bias_tables():
    inp = make_custom([5, 300, 77], num_heads=3, d_qk=128, d_v=128, dtype="bf16", seed=2,
                      alpha=0.2)
    assert_close(gpu_forward(inp), ora(inp), "bf16")


@pytest.mark.parametrize("dtype,d", [("f32", 8), ("bf16", 128), ("bf16", 256)])
def test_wide_timestamp_span_uses_exact_buckets(dtype, d):
    """Gaps of ~2^27 s push spans past 2^30, the 64-bit bucket path."""
    inp = make_custom([150, 40], num_heads=2, d_qk=d, d_v=d, dtype=dtype, seed=9,
                      time_len=64, time_std=0.5, pos_len=64, alpha=0.3)
    rng = np.random.default_rng(1)
    gaps = rng.integers(0, 1 << 28, size=inp.total_tokens)
    ts = []
    for b in range(inp.num_seqs):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        g = gaps[s:e].copy(); g[0] = 0
        ts.append((1 << 40) + np.cumsum(g))
    inp.timestamps = np.concatenate(ts).astype(np.int64)
    assert_close(gpu_forward(inp), ora(inp), dtype)


def test_unsorted_timestamps():
    inp = make_custom([90, 33], num_heads=1, d_qk=8, d_v=8, dtype="f32", seed=4, time_len=40,
                      time_std=0.5, alpha=0.5)
    rng = np.random.default_rng(3)
    inp.timestamps = (1_600_000_000 + rng.integers(0, 10**7, size=inp.total_tokens)).astype(np.int64)
    assert_close(gpu_forward(inp), ora(inp), "f32")


# ---------------------------------------------------------------------------
# Zero pattern: with V = one-hot rows and no epilogue, out[i, j] = a_ij, so the
# zeros of the output are exactly the masked pairs and the padding columns.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rules", [dict(), dict(num_targets=[9, 0, 30]), dict(contextual_len=5),
                                   dict(max_attn_len=17, num_targets=[4, 7, 2])])
def test_zero_pattern_exact(rules):
    lengths = [100, 57, 128]
    inp = make_custom(lengths, num_heads=2, d_qk=128, d_v=128, dtype="bf16", seed=3,
                      pos_len=256, pos_std=0.2, time_len=64, alpha=0.05, **rules)
    inp.v[:] = 0
    for b in range(inp.num_seqs):
        s = int(inp.offsets[b])
        for j in range(int(inp.lengths[b])):
            inp.v[s + j, :, j] = 1.0
    out = gpu_forward(inp, "none")
    ref = ora(inp, "none")
    T = rules.get("num_targets")
    for b in range(inp.num_seqs):
        s, L = int(inp.offsets[b]), int(inp.lengths[b])
        t = 0 if T is None else T[b]
        mask = np.array([[oracle.allowed(L, t, rules.get("contextual_len", 0),
                                         rules.get("max_attn_len", 0), i, j)
                          for j in range(L)] for i in range(L)])
        for h in range(2):
            blk = out[s:s + L, h, :L]
            assert np.array_equal(blk != 0, mask)
            assert np.all(out[s:s + L, h, L:] == 0)
            assert np.array_equal(ref[s:s + L, h, :L] != 0, mask)
    assert_close(out, ref, "bf16")


# ---------------------------------------------------------------------------
# Every row written exactly once, nothing outside `out` touched.
# ---------------------------------------------------------------------------
def test_write_coverage_and_guards():
    inp = make_inputs("ranking", num_seqs=20)
    dev = to_device(inp, DEV)
    N, H, dv = inp.total_tokens, inp.num_heads, inp.d_v
    big = torch.full((N + 64, H, dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    big[:32] = 7.0
    big[32 + N:] = -3.0
    out = big[32:32 + N]
    jagged_attn_fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"], out=out,
                    **call_kwargs(inp, dev))
    torch.cuda.synchronize()
    assert torch.all(big[:32] == 7.0) and torch.all(big[32 + N:] == -3.0)
    assert not torch.isnan(out.float()).any()
    assert_close(out.float().cpu().numpy().astype(np.float64), ora(inp), "bf16")


def test_determinism_bitwise():
    inp = make_inputs("longtail", num_seqs=10)
    a = gpu_forward(inp)
    b = gpu_forward(inp)
    assert np.array_equal(a, b)


def test_plan_reuse_across_runs():
    inp = make_inputs("ranking", num_seqs=24)
    dev = to_device(inp, DEV)
    call = JaggedAttnCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                          **call_kwargs(inp, dev))
    call.plan()
    o1 = call.run().float().cpu().numpy().astype(np.float64)
    inp2 = JaggedInputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    inp2.q = inp.q[::-1].copy()
    call.q.copy_(to_device(inp2, DEV)["q"])
    o2 = call.run().float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    assert_close(o1, ora(inp), "bf16")
    assert_close(o2, ora(inp2), "bf16")


def test_run_timed_matches_run():
    """The timed launch does the same work (bitwise the same output) and its
    events bracket the attention kernel itself: a positive duration no longer
    than that between markers recorded around the launch."""
    inp = make_inputs("ranking", num_seqs=24)
    dev = to_device(inp, DEV)
    call = JaggedAttnCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                          **call_kwargs(inp, dev))
    call.plan()
    ref = call.run().clone()
    stream = torch.cuda.current_stream()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    k1.record(stream)
    call.out.zero_()
    m0.record(stream)
    got = call.run_timed(k0, k1)
    m1.record(stream)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    kernel_ms, marker_ms = k0.elapsed_time(k1), m0.elapsed_time(m1)
    assert 0.0 < kernel_ms <= marker_ms, (kernel_ms, marker_ms)


def test_split_items_plan_reuse():
    """One long causal sequence: its last query tiles reach far more key tiles
    than a workgroup's share, so the scheduler splits them along the keys and
    the chunks' partial outputs are summed by the chunk that finishes last.
    Two runs of one plan (the arrival counters must rearm) and a third call
    with a fresh plan all match the oracle and each other bitwise."""
    inp = make_custom([4096, 700, 33], num_heads=2, d_qk=128, d_v=128, dtype="bf16", seed=8,
                      contextual_len=6, pos_len=4096, time_len=64, alpha=0.0884)
    dev = to_device(inp, DEV)
    call = JaggedAttnCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                          **call_kwargs(inp, dev))
    call.plan()
    o1 = call.run().float().cpu().numpy().astype(np.float64)
    o2 = call.run().float().cpu().numpy().astype(np.float64)
    o3 = gpu_forward(inp)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(3968, 4096), np.arange(0, 4096, 97),
                                     np.arange(4096, 4829, 41)]))
    assert_close(o1, ora(inp, rows=rows), "bf16", rows=rows)
    assert np.array_equal(o1, o2) and np.array_equal(o1, o3)


def test_d256_split_items_candidates_and_clamp():
    """bf16 with d_qk = d_v = 256 (one workgroup per CU): a 2200-token
    sequence whose last query tiles are split along the keys, candidates,
    a contextual prefix and both position-bias readings, on sampled rows of
    the long sequence and all rows of the short ones."""
    print("case d256 split/candidates/clamp", flush=True)
    inp = make_custom([2200, 700, 33], num_heads=2, d_qk=256, d_v=256, dtype="bf16", seed=12,
                      num_targets=[40, 5, 3], contextual_len=6, pos_len=4096, time_len=64,
                      alpha=1.0 / 16)
    rows = np.unique(np.concatenate([np.arange(2048, 2200), np.arange(0, 2200, 61),
                                     np.arange(2200, inp.total_tokens)]))
    for clamp in (False, True):
        assert_close(gpu_forward(inp, pos_clamp=clamp), ora(inp, rows=rows, pos_clamp=clamp),
                     "bf16", rows=rows)


@pytest.mark.parametrize("lengths,targets,window", [
    ([256, 1, 0, 130, 129], [20, 0, 0, 5, 129], 0),   # every sequence within two query tiles
    ([256, 257, 40], [0, 30, 3], 100),                 # one sequence of three tiles
    ([5, 17, 3], [2, 17, 0], 4),                       # fewer units than workgroups
])
def test_queue_boundaries_plan_reuse(lengths, targets, window):
    """Batches at the edge of the work-queue mode (sequences of at most 256
    rows take units from a counter in decreasing cost; a longer one switches
    the batch to the static plan).  Three runs of one plan -- the counter must
    rewind after the last fetch, also when workgroups stay idle -- match the
    oracle and each other bitwise."""
    inp = make_custom(lengths, num_heads=3, d_qk=64, d_v=64, dtype="bf16", seed=21,
                      num_targets=targets, contextual_len=3, max_attn_len=window,
                      pos_len=512, time_len=64, alpha=0.125)
    dev = to_device(inp, DEV)
    call = JaggedAttnCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                          **call_kwargs(inp, dev))
    call.plan()
    outs = []
    for _ in range(3):
        call.out.zero_()
        outs.append(call.run().float().cpu().numpy().astype(np.float64))
    torch.cuda.synchronize()
    assert_close(outs[0], ora(inp), "bf16")
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("dtype,d", [("f32", 8), ("bf16", 64)])
def test_large_batch_plan(dtype, d):
    """More sequences than the scheduler keeps in LDS (2048) and more items
    than its compact variant takes (4096): the workspace-backed path."""
    rng = np.random.default_rng(17)
    lengths = rng.integers(0, 160, size=3000)
    lengths[::7] = 0
    inp = make_custom(lengths.tolist(), num_heads=2, d_qk=d, d_v=d, dtype=dtype, seed=3,
                      num_targets=rng.integers(0, 12, size=3000).tolist(), pos_len=512,
                      time_len=64, alpha=0.3)
    assert_close(gpu_forward(inp), ora(inp), dtype)


# ---------------------------------------------------------------------------
# Candidate rows only ("Scaling HSTU", section "Many candidates make reuse
# valuable"): the candidates of a sequence see its history and themselves, so
# their outputs can be computed apart from the history rows and in micro-batches.
# ---------------------------------------------------------------------------
def _candidates_forward(inp, sentinel=-5.0):
    dev = to_device(inp, DEV)
    N, H, dv = inp.total_tokens, inp.num_heads, inp.d_v
    out = torch.full((N, H, dv), sentinel, dtype=dev["q"].dtype, device=DEV)
    jagged_attn_fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"], out=out,
                    candidates_only=True, **call_kwargs(inp, dev))
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _candidate_rows(inp):
    rows = []
    for b in range(inp.num_seqs):
        s0, s1 = int(inp.offsets[b]), int(inp.offsets[b + 1])
        nt = 0 if inp.num_targets is None else int(inp.num_targets[b])
        rows.extend(range(s1 - min(max(nt, 0), s1 - s0), s1))
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("name,kw", [("ranking", dict(num_seqs=24)),
                                     ("windowed", dict(num_seqs=2))])
def test_candidates_only(name, kw):
    inp = make_inputs(name, **kw)
    got = _candidates_forward(inp)
    rows = _candidate_rows(inp)
    hist = np.setdiff1d(np.arange(inp.total_tokens), rows)
    assert np.all(got[hist] == -5.0), "history rows were written"
    assert_close(got, ora(inp, rows=rows), "bf16", rows=rows)


def _subset(inp, keep_rows, offsets, num_targets):
    out = JaggedInputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    for name in ("q", "k", "v", "u"):
        setattr(out, name, getattr(inp, name)[keep_rows].copy())
    if inp.timestamps is not None:
        out.timestamps = inp.timestamps[keep_rows].copy()
    out.offsets = np.asarray(offsets, dtype=np.int32)
    out.num_targets = np.asarray(num_targets, dtype=np.int32)
    return out


def test_candidate_independence_bitwise():
    """A candidate's output does not depend on the other candidates: changing
    their q, k, v, u and timestamps leaves its row bitwise unchanged."""
    inp = make_custom([300, 45, 129], num_heads=2, d_qk=128, d_v=128, dtype="bf16", seed=33,
                      num_targets=[60, 60, 60], contextual_len=4, pos_len=512, time_len=64,
                      alpha=0.2, n_scale=400.0)
    keep = []   # candidates 20..39 of each sequence stay, the others change
    others = []
    for b in range(3):
        s1 = int(inp.offsets[b + 1])
        keep.extend(range(s1 - 40, s1 - 20))
        others.extend(list(range(s1 - 60, s1 - 40)) + list(range(s1 - 20, s1)))
    a = _candidates_forward(inp)
    b = _candidates_forward(_perturb(inp, np.array(others)))
    assert np.array_equal(a[keep], b[keep])


@pytest.mark.parametrize("dtype,d,tol", [("f32", 64, 1e-6), ("bf16", 128, 1e-2)])
def test_candidate_microbatches(dtype, d, tol):
    """Three users, each with a history and 60 candidates.  Computing the
    candidates in micro-batches of 20 (each laid out after its user's
    history) gives the rows of the all-at-once computation.  The position
    bias uses the raw i - j, and a micro-batch moves its candidates to other
    positions, so this holds exactly with the time bias alone (timestamps
    travel with their tokens)."""
    hist = [300, 45, 129]
    lengths = [h + 60 for h in hist]
    inp = make_custom(lengths, num_heads=2, d_qk=d, d_v=d, dtype=dtype, seed=31,
                      num_targets=[60, 60, 60], contextual_len=4, time_len=64,
                      alpha=0.2, n_scale=400.0)
    full = _candidates_forward(inp)
    for m in range(3):
        keep, offs, nts = [], [0], []
        for b, h in enumerate(hist):
            s0 = int(inp.offsets[b])
            keep.extend(range(s0, s0 + h))
            keep.extend(range(s0 + h + 20 * m, s0 + h + 20 * m + 20))
            offs.append(offs[-1] + h + 20)
            nts.append(20)
        mb = _subset(inp, np.array(keep), offs, nts)
        got = _candidates_forward(mb)
        for b, h in enumerate(hist):
            g = got[offs[b] + h: offs[b] + h + 20]
            f = full[int(inp.offsets[b]) + h + 20 * m: int(inp.offsets[b]) + h + 20 * m + 20]
            scale = np.abs(f).max()
            assert np.abs(g - f).max() <= tol * scale
        rows = _candidate_rows(mb)
        assert_close(got, ora(mb, rows=rows), dtype, rows=rows)


# ---------------------------------------------------------------------------
# Epilogue variant: LayerNorm over all heads of a token.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,kw,dtype", [("ranking", dict(num_seqs=24), "bf16"),
                                           ("longtail", dict(num_seqs=6), "f32"),
                                           ("tiny", dict(), "f32")])
def test_ln_all_heads(name, kw, dtype):
    inp = make_inputs(name, dtype=dtype, **kw)
    assert_close(gpu_forward(inp, epilogue="ln_all_u"), ora(inp, "ln_all_u"), dtype)


@pytest.mark.parametrize("heads,d,dtype", [(16, 128, "bf16"), (32, 128, "bf16"),
                                           (16, 128, "f32"), (3, 64, "bf16")])
def test_ln_all_heads_widths(heads, d, dtype):
    """Token widths H * d_v that take 4 and 8 16-byte chunks per lane in the
    all-heads LayerNorm pass (1 and 2 come from the workloads above), and a
    width of 24 chunks that leaves most lanes idle."""
    inp = make_custom([37, 130, 5], num_heads=heads, d_qk=d, d_v=d, dtype=dtype, seed=5,
                      num_targets=[4, 20, 0], contextual_len=2, pos_len=256, time_len=64,
                      alpha=1.0 / math.sqrt(d))
    assert_close(gpu_forward(inp, epilogue="ln_all_u"), ora(inp, "ln_all_u"), dtype)


def test_ln_all_heads_strided_and_candidates():
    inp = make_inputs("layer", num_seqs=5)
    assert_close(gpu_forward(inp, epilogue="ln_all_u", ld=2048), ora(inp, "ln_all_u"), "bf16")
    inp = make_inputs("ranking", num_seqs=12)
    dev = to_device(inp, DEV)
    out = torch.full((inp.total_tokens, inp.num_heads, inp.d_v), -5.0, dtype=torch.bfloat16,
                     device=DEV)
    jagged_attn_fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"], out=out,
                    epilogue="ln_all_u", candidates_only=True, **call_kwargs(inp, dev))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    rows = _candidate_rows(inp)
    hist = np.setdiff1d(np.arange(inp.total_tokens), rows)
    assert np.all(got[hist] == -5.0)
    assert_close(got, ora(inp, "ln_all_u", rows=rows), "bf16", rows=rows)


# ---------------------------------------------------------------------------
# Full HSTU layer: LayerNorm, fused U/V/Q/K projection + SiLU (MFMA GEMM),
# attention on the strided branches, output projection + residual.
# ---------------------------------------------------------------------------
def gpu_layer(inp):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
        DEV).to(torch.bfloat16)
    L = inp.layer
    dev = to_device(inp, DEV)
    kw = call_kwargs(inp, dev)
    lay = HstuLayer(t(L["x"]), t(L["w_uvqk"]), t(L["b_uvqk"]), t(L["w_o"]), dev["offsets"],
                    num_heads=inp.num_heads, d_qk=inp.d_qk, d_v=inp.d_v,
                    timestamps=kw["timestamps"], num_targets=kw["num_targets"],
                    contextual_len=kw["contextual_len"], max_attn_len=kw["max_attn_len"],
                    alpha=kw["alpha"], n_scale=kw["n_scale"], pos_table=kw["pos_table"],
                    time_table=kw["time_table"], eps=kw["eps"])
    y = lay()
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("num_seqs,seed", [(8, 1234), (3, 7)])
def test_layer_forward(num_seqs, seed):
    inp = make_inputs("layer", num_seqs=num_seqs, seed=seed)
    assert_close(gpu_layer(inp), oracle.layer_forward(inp), "bf16")


def test_layer_forward_full_size_sampled_rows():
    inp = make_inputs("layer")
    rows = _sample_rows(inp, 300, 9)
    assert_close(gpu_layer(inp), oracle.layer_forward(inp, rows=rows), "bf16", rows=rows)


def test_layer_forward_full_size_whole_output():
    """The full layer batch (64 sequences, hidden 512): every output row."""
    print("case whole layer", flush=True)
    inp = make_inputs("layer")
    assert_close(gpu_layer(inp), oracle.layer_forward(inp), "bf16")


# ---------------------------------------------------------------------------
# Information flow on the device, bitwise ("Do not copy softmax masking
# mechanically": change future inputs, earlier outputs must not move).
# ---------------------------------------------------------------------------
def _perturb(inp, rows, seed=5):
    rng = np.random.default_rng(seed)
    out = JaggedInputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    for name in ("q", "k", "v", "u"):
        arr = getattr(inp, name).copy()
        vals = rng.standard_normal(arr[rows].shape).astype(np.float32)
        if inp.dtype == "bf16":
            from jagged_hstu_attention_attn_amd.inputs import bf16_round
            vals = bf16_round(vals)
        arr[rows] = vals
        setattr(out, name, arr)
    if inp.timestamps is not None:
        ts = inp.timestamps.copy()
        ts[rows] += rng.integers(1, 10**6, size=len(rows))
        out.timestamps = ts
    return out


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 8), ("bf16", 256)])
def test_future_perturbation_bitwise(dtype, d):
    inp = make_custom([300, 90], num_heads=2, d_qk=d, d_v=d, dtype=dtype, seed=21,
                      num_targets=[12, 5], pos_len=512, time_len=64, alpha=0.2)
    a = gpu_forward(inp)
    for p in (1, 31, 32, 100, 200, 287):
        b = gpu_forward(_perturb(inp, list(range(p, 300))))
        assert np.array_equal(a[:p], b[:p]), p
        assert np.array_equal(a[300:], b[300:])          # other sequence untouched
    # candidates do not see each other
    for cand in (288, 295, 299):
        b = gpu_forward(_perturb(inp, [cand]))
        others = [r for r in range(288, 300) if r != cand]
        assert np.array_equal(a[:288], b[:288]) and np.array_equal(a[others], b[others])


def test_window_reach_bitwise():
    W = 40
    inp = make_custom([400], num_heads=1, d_qk=128, d_v=128, dtype="bf16", seed=8,
                      max_attn_len=W, pos_len=512, alpha=0.1)
    a = gpu_forward(inp)
    p = 150
    b = gpu_forward(_perturb(inp, [p]))
    changed = [i for i in range(400) if not np.array_equal(a[i], b[i])]
    assert changed == list(range(p, p + W + 1))


def test_batch_independence_bitwise():
    inp = make_custom([40, 300, 0, 129], num_heads=2, d_qk=128, d_v=128, dtype="bf16", seed=2,
                      num_targets=[3, 20, 0, 9], pos_len=512, time_len=64, alpha=0.1)
    full = gpu_forward(inp)
    for b in range(inp.num_seqs):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        if e == s:
            continue
        one = JaggedInputs(
            workload="one", dtype="bf16", offsets=np.array([0, e - s], np.int32),
            num_targets=inp.num_targets[b:b + 1], timestamps=inp.timestamps[s:e],
            q=inp.q[s:e], k=inp.k[s:e], v=inp.v[s:e], u=inp.u[s:e], pos_table=inp.pos_table,
            time_table=inp.time_table, contextual_len=0, max_attn_len=0, alpha=inp.alpha,
            n_scale=inp.n_scale)
        assert np.array_equal(gpu_forward(one), full[s:e])


def test_overflowing_masked_scores_fp32():
    inp = make_custom([60], num_heads=1, d_qk=8, d_v=8, dtype="f32", seed=8, alpha=1.0)
    a = gpu_forward(inp)
    bad = JaggedInputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    bad.k = inp.k.copy(); bad.q = inp.q.copy()
    bad.k[40:] = 3e38
    bad.q[40:] = -3e38
    b = gpu_forward(bad)
    assert np.all(np.isfinite(b[:40]))
    assert np.array_equal(a[:40], b[:40])


def test_empty_batch():
    inp = make_custom([0, 0], num_heads=1, d_qk=8, d_v=8)
    dev = to_device(inp, DEV)
    out = jagged_attn_fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                          **call_kwargs(inp, dev))
    torch.cuda.synchronize()
    assert out.shape == (0, 1, 8)


# ---------------------------------------------------------------------------
# d_qk != d_v ("HSTU tensor by tensor", section "Trace four projections":
# the Q/K and U/V branches have their own widths).  One side of the staging
# then goes directly between HBM and registers.
# ---------------------------------------------------------------------------
def _unequal(dqk, dv, W=0, seed=61, H=2):
    return make_custom([1, 37, 129, 300, 260, 5], num_heads=H, d_qk=dqk, d_v=dv, dtype="bf16",
                       seed=seed, num_targets=[0, 5, 20, 50, 3, 5], contextual_len=3,
                       max_attn_len=W, pos_len=64, pos_std=0.3, time_len=16, time_std=0.3,
                       alpha=1.0 / math.sqrt(dqk))


@pytest.mark.parametrize("dqk,dv", [(64, 128), (128, 64)])
@pytest.mark.parametrize("epilogue", ["ln_u", "none", "ln_all_u"])
@pytest.mark.parametrize("W", [0, 100])
def test_unequal_head_dims(dqk, dv, epilogue, W):
    inp = _unequal(dqk, dv, W=W)
    assert_close(gpu_forward(inp, epilogue), ora(inp, epilogue), "bf16")


@pytest.mark.parametrize("dqk,dv", [(64, 128), (128, 64)])
def test_unequal_head_dims_ranking_shape(dqk, dv):
    """Ranking-like batch (128 users, histories U[20, 200] + 20 candidates, 4 heads)."""
    rng = np.random.default_rng(77)
    hist = rng.integers(20, 201, size=128)
    inp = make_custom((hist + 20).tolist(), num_heads=4, d_qk=dqk, d_v=dv, dtype="bf16",
                      seed=78, num_targets=[20] * 128, pos_len=4096, time_len=64,
                      alpha=1.0 / math.sqrt(dqk))
    assert_close(gpu_forward(inp), ora(inp), "bf16")


@pytest.mark.parametrize("dqk,dv", [(64, 128), (128, 64)])
def test_unequal_head_dims_candidates_only(dqk, dv):
    inp = _unequal(dqk, dv, W=40)
    got = _candidates_forward(inp)
    rows = _candidate_rows(inp)
    assert_close(got, ora(inp, rows=rows), "bf16", rows=rows)


# ---------------------------------------------------------------------------
# Position bias at clamped positions (the alternative reading of the
# candidate clamp of "HSTU-MUSA", section "Mathematical Equivalence").
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 8), ("f32", 64)])
@pytest.mark.parametrize("epilogue", ["ln_u", "none"])
def test_pos_clamp(dtype, d, epilogue):
    inp = make_custom([1, 37, 129, 300, 260, 5], num_heads=2, d_qk=d, d_v=d, dtype=dtype,
                      seed=91, num_targets=[0, 5, 20, 50, 3, 5], contextual_len=3,
                      max_attn_len=100, pos_len=512, pos_std=0.3, time_len=16, time_std=0.3,
                      alpha=1.0 / math.sqrt(d))
    got = gpu_forward(inp, epilogue, pos_clamp=True)
    assert_close(got, ora(inp, epilogue, pos_clamp=True), dtype)
    # history rows are those of the raw reading
    raw = gpu_forward(inp, epilogue)
    rows = _candidate_rows(inp)
    hist = np.setdiff1d(np.arange(inp.total_tokens), rows)
    assert np.array_equal(got[hist], raw[hist])


def test_pos_clamp_ranking_workload():
    inp = make_inputs("ranking")
    assert_close(gpu_forward(inp, pos_clamp=True), ora(inp, pos_clamp=True), "bf16")


def test_pos_clamp_candidates_only():
    inp = make_inputs("windowed", num_seqs=2)
    dev = to_device(inp, DEV)
    out = torch.full((inp.total_tokens, inp.num_heads, inp.d_v), -5.0, dtype=torch.bfloat16,
                     device=DEV)
    jagged_attn_fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"], out=out,
                    candidates_only=True, pos_clamp=True, **call_kwargs(inp, dev))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    rows = _candidate_rows(inp)
    assert_close(got, ora(inp, rows=rows, pos_clamp=True), "bf16", rows=rows)


def test_one_shot_calls_share_a_stream_workspace():
    """jagged_attn_fwd keeps one workspace per (device, stream): calls of
    different sizes in a row (the workspace grows, then is reused) and a call
    on a second stream give the same output as a call with its own
    workspace; a too-small caller workspace is refused."""
    from jagged_hstu_attention_attn_amd import api
    print("case one-shot workspace reuse", flush=True)
    small = make_custom([40, 130], num_heads=2, d_qk=128, d_v=128, dtype="bf16", seed=3,
                        pos_len=256, time_len=64, alpha=0.1)
    big = make_inputs("longtail", num_seqs=6, seed=5)   # items long enough to split
    outs = []
    for inp in (small, big, small, big):
        outs.append(gpu_forward(inp))
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        o2 = gpu_forward(small)
    torch.cuda.synchronize()
    for inp, o in ((small, outs[0]), (big, outs[1])):
        dev = to_device(inp, DEV)
        own = JaggedAttnCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                             **call_kwargs(inp, dev))()
        torch.cuda.synchronize()
        assert np.array_equal(o, own.float().cpu().numpy().astype(np.float64))
    assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3])
    assert np.array_equal(outs[0], o2)
    assert_close(outs[1], ora(big), "bf16")
    dev = to_device(small, DEV)
    with pytest.raises(ValueError):
        JaggedAttnCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                       workspace=torch.empty(16, dtype=torch.uint8, device=DEV),
                       **call_kwargs(small, dev))
    assert len(api._ws_cache) >= 2


def test_d256_candidates_only_and_ln_all_heads():
    """bf16 d = 256 through the candidates-only call (history rows untouched)
    and the LayerNorm-over-all-heads epilogue (H * d_v = 1024)."""
    print("case d256 candidates-only / ln_all_u", flush=True)
    inp = make_custom([300, 140, 33], num_heads=4, d_qk=256, d_v=256, dtype="bf16", seed=44,
                      num_targets=[60, 20, 5], contextual_len=2, pos_len=512, time_len=64,
                      alpha=1.0 / 16)
    got = _candidates_forward(inp)
    rows = _candidate_rows(inp)
    hist = np.setdiff1d(np.arange(inp.total_tokens), rows)
    assert np.all(got[hist] == -5.0), "history rows were written"
    assert_close(got, ora(inp, rows=rows), "bf16", rows=rows)
    assert_close(gpu_forward(inp, epilogue="ln_all_u"), ora(inp, "ln_all_u"), "bf16")
