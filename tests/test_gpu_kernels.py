"""Each bf16 d = 128 forward kernel (four-wave, eight-wave, sixteen-row,
thirty-two-row)
against the fp64 oracle.

The library picks a forward kernel by shape (see the header: the sixteen-row
one for bf16 with d = 128); every test here forces each kernel in turn on the
small ragged batches of every mask rule, the tile-edge lengths, windows, split
items, candidate rows, the clamped-position bias and the exact zero pattern,
so that every kernel's geometry is checked, not only the automatic choice's.
Tolerance: max|gpu - oracle| <= 1e-2 * max|oracle| (bf16).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from jagged_hstu_attention_attn_amd.api import JaggedAttnCall, fwd_kernel, jagged_attn_fwd
from jagged_hstu_attention_attn_amd.device_inputs import call_kwargs, to_device
from jagged_hstu_attention_attn_amd.inputs import make_custom, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["four_wave", "eight_wave", "sixteen_row", "thirtytwo_row"], autouse=True)
def kernel(request):
    """The forward kernel every call of the test is forced to."""
    global _KERNEL
    _KERNEL = request.param
    yield request.param
    _KERNEL = None


_KERNEL = None

DEV = "cuda:0"
EDGE_LENGTHS = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257, 300]


def _fwd(inp, epilogue="ln_u", kernel=None, ld=None, pos_clamp=False, out=None,
         candidates_only=False):
    with fwd_kernel(kernel or _KERNEL):
        dev = to_device(inp, DEV, ld=ld)
        o = jagged_attn_fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                            epilogue=epilogue, pos_clamp=pos_clamp, out=out,
                            candidates_only=candidates_only, **call_kwargs(inp, dev))
        torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


def _ora(inp, epilogue="ln_u", rows=None, pos_clamp=False):
    ep = {"ln_u": oracle.EPILOGUE_LN_U, "none": oracle.EPILOGUE_NONE}[epilogue]
    return oracle.forward(inp, epilogue=ep, rows=rows, pos_clamp=pos_clamp)


def _close(gpu, ref, rows=None, tol=1e-2):
    if rows is not None:
        gpu, ref = gpu[rows], ref[rows]
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    scale = np.abs(ref).max()
    err = np.abs(gpu - ref).max()
    assert err <= tol * scale, f"max err {err:.3e} vs bound {tol * scale:.3e}"


@pytest.mark.parametrize("rules", ["causal", "targets", "prefix", "window", "all"])
def test_pp_edges(rules):
    print(f"case {_KERNEL} edges {rules}", flush=True)
    rng = np.random.default_rng(hash(rules) % 1000)
    lengths = list(EDGE_LENGTHS)
    B = len(lengths)
    nt = None
    c = W = 0
    if rules in ("targets", "all"):
        nt = [int(x) for x in rng.integers(0, 40, size=B)]
        nt[1] = 1; nt[3] = 31; nt[7] = 64
    if rules in ("prefix", "all"):
        c = 6 if rules == "all" else 40
    if rules in ("window", "all"):
        W = {"window": 32, "all": 33}[rules]
    inp = make_custom(lengths, num_heads=2, d_qk=128, d_v=128, dtype="bf16", seed=11,
                      num_targets=nt, contextual_len=c, max_attn_len=W, pos_len=300,
                      pos_std=0.3, time_len=64, time_std=0.3, alpha=1.0 / math.sqrt(128),
                      t0=(1 << 33) + 17)
    for ep in ("ln_u", "none"):
        _close(_fwd(inp, ep), _ora(inp, ep))


@pytest.mark.parametrize("W", [1, 31, 32, 33, 127, 128, 129, 1024])
def test_pp_window_sizes(W):
    print(f"case {_KERNEL} window {W}", flush=True)
    inp = make_custom([1500, 129, 700], num_heads=1, d_qk=128, d_v=128, dtype="bf16", seed=W,
                      num_targets=[25, 3, 50], max_attn_len=W, pos_len=4096, time_len=64,
                      alpha=1 / math.sqrt(128))
    _close(_fwd(inp), _ora(inp))


def test_pp_no_bias_tables_and_alpha_zero():
    print(f"case {_KERNEL} no_bias", flush=True)
    inp = make_custom([5, 300, 77, 640], num_heads=3, d_qk=128, d_v=128, dtype="bf16", seed=2,
                      alpha=0.2)
    _close(_fwd(inp), _ora(inp))
    inp0 = make_custom([300, 77], num_heads=2, d_qk=128, d_v=128, dtype="bf16", seed=3,
                       alpha=0.0, pos_len=64, time_len=16)
    _close(_fwd(inp0), _ora(inp0))


def test_pp_wide_timestamp_span():
    """Spans past 2^30 s: the 64-bit time-bucket path."""
    print(f"case {_KERNEL} wide_ts", flush=True)
    inp = make_custom([450, 40], num_heads=2, d_qk=128, d_v=128, dtype="bf16", seed=9,
                      time_len=64, time_std=0.5, pos_len=64, alpha=0.3)
    rng = np.random.default_rng(1)
    gaps = rng.integers(0, 1 << 28, size=inp.total_tokens)
    ts = []
    for b in range(inp.num_seqs):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        g = gaps[s:e].copy(); g[0] = 0
        ts.append((1 << 40) + np.cumsum(g))
    inp.timestamps = np.concatenate(ts).astype(np.int64)
    _close(_fwd(inp), _ora(inp))


def test_pp_unsorted_timestamps():
    print(f"case {_KERNEL} unsorted_ts", flush=True)
    inp = make_custom([390, 33], num_heads=1, d_qk=128, d_v=128, dtype="bf16", seed=4,
                      time_len=40, time_std=0.5, alpha=0.5 / math.sqrt(128))
    rng = np.random.default_rng(3)
    inp.timestamps = (1_600_000_000 + rng.integers(0, 10**7, size=inp.total_tokens)).astype(
        np.int64)
    _close(_fwd(inp), _ora(inp))


@pytest.mark.parametrize("name,n", [("ranking", 40), ("longtail", 8), ("windowed", 1)])
def test_pp_workloads(name, n):
    print(f"case {_KERNEL} workload {name} {n}", flush=True)
    inp = make_inputs(name, num_seqs=n)
    _close(_fwd(inp), _ora(inp))


def test_pp_strided_views():
    print(f"case {_KERNEL} strided", flush=True)
    inp = make_inputs("layer", num_seqs=4)
    a = _fwd(inp, ld=2048)
    b = _fwd(inp)
    assert np.array_equal(a, b)
    _close(a, _ora(inp))


def test_pp_split_items_plan_reuse():
    """Long causal sequence: its last tiles are split along the keys; two runs
    of one plan and a fresh plan agree bitwise and with the oracle."""
    print(f"case {_KERNEL} split", flush=True)
    inp = make_custom([4096, 700, 33], num_heads=2, d_qk=128, d_v=128, dtype="bf16", seed=8,
                      contextual_len=6, pos_len=4096, time_len=64, alpha=0.0884)
    with fwd_kernel(_KERNEL):
        dev = to_device(inp, DEV)
        call = JaggedAttnCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                              **call_kwargs(inp, dev))
        call.plan()
        o1 = call.run().float().cpu().numpy().astype(np.float64)
        o2 = call.run().float().cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
    o3 = _fwd(inp)
    rows = np.unique(np.concatenate([np.arange(3968, 4096), np.arange(0, 4096, 97),
                                     np.arange(4096, 4829, 41)]))
    _close(o1, _ora(inp, rows=rows), rows=rows)
    assert np.array_equal(o1, o2) and np.array_equal(o1, o3)


def test_pp_candidates_only():
    print(f"case {_KERNEL} candidates", flush=True)
    inp = make_inputs("windowed", num_seqs=2)
    N, H, dv = inp.total_tokens, inp.num_heads, inp.d_v
    out = torch.full((N, H, dv), -5.0, dtype=torch.bfloat16, device=DEV)
    got = _fwd(inp, out=out, candidates_only=True)
    rows = []
    for b in range(inp.num_seqs):
        s1 = int(inp.offsets[b + 1])
        rows.extend(range(s1 - int(inp.num_targets[b]), s1))
    rows = np.array(rows)
    hist = np.setdiff1d(np.arange(N), rows)
    assert np.all(got[hist] == -5.0), "history rows were written"
    _close(got, _ora(inp, rows=rows), rows=rows)


@pytest.mark.parametrize("epilogue", ["ln_u", "none"])
def test_pp_pos_clamp(epilogue):
    print(f"case {_KERNEL} pos_clamp {epilogue}", flush=True)
    inp = make_custom([1, 37, 129, 300, 260, 700], num_heads=2, d_qk=128, d_v=128,
                      dtype="bf16", seed=91, num_targets=[0, 5, 20, 50, 3, 40],
                      contextual_len=3, max_attn_len=100, pos_len=512, pos_std=0.3,
                      time_len=16, time_std=0.3, alpha=1.0 / math.sqrt(128))
    _close(_fwd(inp, epilogue, pos_clamp=True), _ora(inp, epilogue, pos_clamp=True))


def test_pp_zero_pattern_exact():
    """One-hot V over keys [0, 128) and no epilogue: out[i, j] = a_ij, so the
    zeros of those columns are exactly the masked pairs, for rows spread over
    several query tiles and both key halves of the workgroup."""
    print(f"case {_KERNEL} zero_pattern", flush=True)
    lengths, nt, W = [700, 300], [40, 10], 90
    inp = make_custom(lengths, num_heads=1, d_qk=128, d_v=128, dtype="bf16", seed=5,
                      num_targets=nt, contextual_len=3, max_attn_len=W, pos_len=1024,
                      pos_std=0.2, time_len=64, alpha=0.05)
    inp.v[:] = 0
    for b in range(inp.num_seqs):
        s = int(inp.offsets[b])
        for j in range(min(128, int(inp.lengths[b]))):
            inp.v[s + j, :, j] = 1.0
    out = _fwd(inp, "none")
    for b in range(inp.num_seqs):
        s, L = int(inp.offsets[b]), int(inp.lengths[b])
        for i in range(L):
            want = np.array([oracle.allowed(L, nt[b], 3, W, i, j) for j in range(min(128, L))])
            assert np.array_equal(out[s + i, 0, :len(want)] != 0, want), (b, i)


def test_pp_matches_other_kernel():
    """The forced kernel and another kernel on one long-tail batch: each
    within tolerance of the oracle, and of each other."""
    other = "sixteen_row" if _KERNEL == "four_wave" else "four_wave"
    print(f"case {_KERNEL} vs_{other}", flush=True)
    inp = make_inputs("longtail", num_seqs=6, seed=3)
    a = _fwd(inp)
    b = _fwd(inp, kernel=other)
    ref = _ora(inp)
    _close(a, ref)
    _close(b, ref)
    _close(a, b)


_XCD_CASE = {}


def _xcd_case():
    """Many windowed sequences of four query tiles: every item reaches at most
    five key tiles, small against a workgroup's share of the batch, so the
    scheduler plans one work queue per XCD.  The oracle runs once for all
    kernels."""
    if not _XCD_CASE:
        rng = np.random.default_rng(41)
        B = 200   # the work list's item bound stays within the scheduler's LDS lists
        lengths = [int(x) for x in rng.integers(400, 513, size=B)]
        nt = [int(x) for x in rng.integers(0, 30, size=B)]
        inp = make_custom(lengths, num_heads=4, d_qk=128, d_v=128, dtype="bf16", seed=41,
                          num_targets=nt, contextual_len=2, max_attn_len=32, pos_len=1024,
                          pos_std=0.2, time_len=64, time_std=0.2, alpha=1.0 / math.sqrt(128))
        _XCD_CASE["inp"] = inp
        _XCD_CASE["ref"] = _ora(inp)
    return _XCD_CASE["inp"], _XCD_CASE["ref"]


def test_pp_xcd_queues_plan_reuse():
    """Per-XCD work queues: the plan header names the mode (word 2 == 2) and
    eight unit ranges that tile the units in order; three runs of one plan --
    every XCD's counter must rewind after its last fetch -- match the oracle
    and each other bitwise."""
    print(f"case {_KERNEL} xcd_queues", flush=True)
    inp, ref = _xcd_case()
    with fwd_kernel(_KERNEL):
        dev = to_device(inp, DEV)
        call = JaggedAttnCall(dev["q"], dev["k"], dev["v"], dev["u"], dev["offsets"],
                              **call_kwargs(inp, dev))
        call.plan()
        hdr = call.workspace[:256].view(torch.int32).cpu().numpy()
        outs = []
        for _ in range(3):
            call.out.zero_()
            outs.append(call.run().float().cpu().numpy().astype(np.float64))
        torch.cuda.synchronize()
        hdr_after = call.workspace[:256].view(torch.int32).cpu().numpy()
    assert hdr[2] == 2, f"plan mode {hdr[2]}"
    n_units = int(hdr[4])
    bounds = hdr[16:25]
    assert bounds[0] == 0 and bounds[8] == n_units and np.all(np.diff(bounds) >= 0), bounds
    assert np.all(hdr_after[8:16] == 0), "an XCD counter was not rewound"
    _close(outs[0], ref)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
