"""Pins the CPU oracle to facts fixed by the pages and by mathematics.

Each test names the passage it follows.  None of these retypes the oracle's
formula: they use printed values, hand-worked masks, closed forms written as
prefix sums, library routines (scipy, torch, Python integers) and invariants.
"""
import dataclasses
import math

import numpy as np
import pytest

from jagged_hstu_attention_attn_amd.inputs import make_custom, make_inputs, JaggedInputs


def _inputs(offsets, q, k, v, u=None, **kw):
    offsets = np.asarray(offsets, dtype=np.int32)
    if u is None:
        u = np.ones_like(v)
    base = dict(workload="t", dtype="f32", offsets=offsets, num_targets=None, timestamps=None,
                q=q, k=k, v=v, u=u, pos_table=None, time_table=None, contextual_len=0,
                max_attn_len=0, alpha=1.0, n_scale=1.0)
    base.update(kw)
    return JaggedInputs(**base)


# ---------------------------------------------------------------------------
# "HSTU tensor by tensor", section "SiLU aggregation coefficients are not
# probabilities": SiLU(-1) ~ -0.269, SiLU(0) = 0, SiLU(1) ~ 0.731.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("x,printed", [(-1.0, -0.269), (0.0, 0.0), (1.0, 0.731)])
def test_silu_printed_values(oracle_mod, x, printed):
    from scipy.special import expit
    d = 8
    q = np.zeros((1, 1, d)); q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, d)); k[0, 0, 0] = x
    v = np.zeros((1, 1, d)); v[0, 0, 0] = 1.0
    out = oracle_mod.forward(_inputs([0, 1], q, k, v), epilogue=oracle_mod.EPILOGUE_NONE)
    got = out[0, 0, 0]
    assert abs(got - printed) <= 5e-4           # printed to three decimals
    assert got == pytest.approx(x * expit(x), abs=1e-15)
    assert oracle_mod.silu(x) == pytest.approx(x * expit(x), abs=1e-15)


def test_silu_extremes_no_nan(oracle_mod):
    # Large negative scores must give -0 (not NaN); large positive give x.
    assert oracle_mod.silu(-800.0) == 0.0
    assert oracle_mod.silu(800.0) == 800.0
    assert not math.isnan(oracle_mod.silu(-1e308))


# Same section: values [1,0] and [0,1] with coefficients [-0.269, 0.731]
# aggregate to [-0.269, 0.731], outside the segment between them.
def test_worked_example_signed_aggregation(oracle_mod):
    d = 8
    q = np.zeros((2, 1, d)); q[1, 0, 0] = 1.0            # q_1 = e0, q_0 = 0
    k = np.zeros((2, 1, d)); k[0, 0, 0] = -1.0; k[1, 0, 0] = 1.0
    v = np.zeros((2, 1, d)); v[0, 0, 0] = 1.0; v[1, 0, 1] = 1.0
    out = oracle_mod.forward(_inputs([0, 2], q, k, v), epilogue=oracle_mod.EPILOGUE_NONE)
    o1 = out[1, 0]
    assert abs(o1[0] - (-0.269)) <= 5e-4 and abs(o1[1] - 0.731) <= 5e-4
    assert np.all(o1[2:] == 0.0)
    assert np.all(out[0, 0] == 0.0)                       # SiLU(0) = 0
    assert o1[0] + o1[1] != pytest.approx(1.0)             # not a convex combination


# "Trace four projections": a.sum(-1) is not required to equal one.  With V = 1
# every output column equals the row sum of the coefficient matrix.
def test_row_sums_not_normalised(oracle_mod):
    inp = make_custom([12], d_qk=8, d_v=8, seed=3, alpha=1.0, n_scale=1.0)
    inp.v[:] = 1.0
    out = oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_NONE)[:, 0, :]
    assert np.allclose(out, out[:, :1])
    sums = out[:, 0]
    assert np.any(np.abs(sums - 1.0) > 1e-3)
    assert np.any(sums < 0.0)


# ---------------------------------------------------------------------------
# Mask rules ("HSTU-MUSA", "Mathematical Equivalence"): hand-worked patterns.
# ---------------------------------------------------------------------------
def _golden_masks():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "masks.txt")
    cases, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("case "):
            parts = line.split()
            kv = dict(p.split("=") for p in parts[2:])
            cur = dict(name=parts[1], L=int(kv["L"]), T=int(kv["T"]), c=int(kv["c"]),
                       W=int(kv["W"]), rows=[])
            cases.append(cur)
        else:
            cur["rows"].append([int(ch) for ch in line])
    for c in cases:
        assert len(c["rows"]) == c["L"] and all(len(r) == c["L"] for r in c["rows"])
    return cases


GOLDEN = _golden_masks()


@pytest.mark.parametrize("case", GOLDEN, ids=[c["name"] for c in GOLDEN])
def test_golden_mask_through_forward(oracle_mod, case):
    """Q = K = 0 and a one-entry position table of 1 give s_ij = 1 everywhere;
    V = identity makes out[i, j] = SiLU(1) * allowed(i, j)."""
    L = case["L"]
    want = np.array(case["rows"], dtype=bool)
    q = np.zeros((L, 1, 8)); k = np.zeros((L, 1, 8))
    v = np.eye(L).reshape(L, 1, L)
    inp = _inputs([0, L], q, k, v, pos_table=np.array([1.0], np.float32),
                  num_targets=np.array([case["T"]], np.int32),
                  contextual_len=case["c"], max_attn_len=case["W"])
    out = oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_NONE)[:, 0, :]
    silu1 = 1.0 / (1.0 + math.exp(-1.0))
    assert np.array_equal(out != 0.0, want)
    assert np.allclose(out[want], silu1, rtol=0, atol=1e-15)
    got = np.array([[oracle_mod.allowed(L, case["T"], case["c"], case["W"], i, j)
                     for j in range(L)] for i in range(L)])
    assert np.array_equal(got, want)
    assert oracle_mod.count_allowed([0, L], [case["T"]], case["c"], case["W"]) == want.sum()


def test_golden_masks_match_dense_builder(oracle_mod):
    for case in GOLDEN:
        m = oracle_mod._dense_mask(case["L"], case["T"], case["c"], case["W"], case["L"])
        assert np.array_equal(m, np.array(case["rows"], dtype=bool)), case["name"]


# ---------------------------------------------------------------------------
# Dense padded brute force (the form of the teaching snippet in "Trace four
# projections": SiLU over everything, masked_fill(~mask, 0), then A @ V).
# ---------------------------------------------------------------------------
def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 5))
    lengths = rng.integers(0, 41, size=B)
    lengths[0] = max(lengths[0], 1)
    H = int(rng.integers(1, 3))
    dqk = int(rng.choice([4, 8, 16]))
    dv = int(rng.choice([4, 8, 16]))
    T = rng.integers(0, 8, size=B) if rng.random() < 0.6 else None
    c = int(rng.integers(0, 8)) if rng.random() < 0.5 else 0
    W = int(rng.integers(1, 12)) if rng.random() < 0.5 else 0
    pos = int(rng.choice([0, 1, 5, 64]))
    tim = int(rng.choice([0, 1, 7, 64]))
    return make_custom(lengths, num_heads=H, d_qk=dqk, d_v=dv, seed=seed, num_targets=T,
                       contextual_len=c, max_attn_len=W, pos_len=pos, pos_std=0.5,
                       time_len=tim, time_std=0.5, alpha=float(rng.uniform(0.1, 1.0)),
                       n_scale=float(rng.uniform(1.0, 50.0)))


@pytest.mark.parametrize("seed", range(40))
def test_oracle_equals_dense_bruteforce(oracle_mod, seed):
    inp = _random_case(seed)
    for ep in (oracle_mod.EPILOGUE_NONE, oracle_mod.EPILOGUE_LN_U, oracle_mod.EPILOGUE_LN_ALL_U):
        a = oracle_mod.forward(inp, epilogue=ep)
        b = oracle_mod.dense_forward(inp, epilogue=ep)
        scale = max(1.0, np.abs(b).max())
        assert np.abs(a - b).max() <= 1e-12 * scale


# ---------------------------------------------------------------------------
# Closed form: Q = 0 and a constant position bias beta make every score beta,
# so o_i = SiLU(beta)/n * sum over allowed j of v_j -- a prefix-sum expression
# per rule, evaluated here with numpy.cumsum.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("L,T,c,W", [(50, 0, 0, 0), (50, 7, 0, 0), (50, 0, 6, 0),
                                     (50, 0, 0, 9), (50, 7, 0, 9), (60, 10, 5, 0),
                                     (33, 33, 0, 0), (40, 5, 3, 4)])
def test_closed_form_prefix_sums(oracle_mod, L, T, c, W):
    from scipy.special import expit
    beta = 0.37
    n = 11.0
    rng = np.random.default_rng(L * 100 + T * 10 + c + W)
    v = rng.standard_normal((L, 1, 8))
    q = np.zeros((L, 1, 8)); k = rng.standard_normal((L, 1, 8))
    inp = _inputs([0, L], q, k, v, pos_table=np.array([beta], np.float32), n_scale=n,
                  num_targets=np.array([T], np.int32), contextual_len=c, max_attn_len=W)
    out = oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_NONE)[:, 0, :]
    cs = np.concatenate([np.zeros((1, 8)), np.cumsum(v[:, 0, :], axis=0)])  # cs[m] = sum_{j<m}
    n_h = L - T
    cc = min(c, n_h)
    a = float(np.float32(beta)) * expit(float(np.float32(beta))) / n
    for i in range(L):
        if i < cc:
            lo, hi = 0, cc
        elif i < n_h:
            lo, hi = 0, i + 1
        else:
            lo, hi = 0, n_h
        p = min(i, n_h)
        if W > 0:
            lo = max(lo, p - W)
        want = cs[hi] - cs[min(lo, hi)]
        if i >= n_h:
            want = want + v[i, 0]
        assert np.allclose(out[i], a * want, rtol=1e-12, atol=1e-13), i


# ---------------------------------------------------------------------------
# Time bucket floor(log2(1 + |dt|)) in exact integers, against Python's
# int.bit_length (units: seconds; "Relative time adds information content
# similarity lacks").
# ---------------------------------------------------------------------------
def test_time_bucket_exact(oracle_mod):
    rng = np.random.default_rng(7)
    deltas = set(range(0, 4200)) | set(int(x) for x in rng.integers(0, 1 << 20, 3000))
    for kk in range(1, 63):
        deltas |= {(1 << kk) - 2, (1 << kk) - 1, 1 << kk}
    deltas |= {(1 << 62) + 12345, (1 << 63) - 2}
    for d in sorted(x for x in deltas if x >= 0):
        want = (d + 1).bit_length() - 1
        t0 = 5_000_000_000
        if d < (1 << 62):
            assert oracle_mod.time_bucket(t0 + d, t0) == want, d
            assert oracle_mod.time_bucket(t0, t0 + d) == want, d
        assert oracle_mod.time_bucket(d, 0) == want, d


# ---------------------------------------------------------------------------
# Information flow ("Do not copy softmax masking mechanically": change future
# inputs and verify that earlier outputs remain unchanged; distinguish history,
# padding, prediction and candidate positions).  Exact equality in fp64.
# ---------------------------------------------------------------------------
def _base_flow_inputs(L=40, T=6, c=0, W=0, seed=11):
    return make_custom([L], num_heads=2, d_qk=8, d_v=8, seed=seed, num_targets=[T],
                       contextual_len=c, max_attn_len=W, pos_len=64, pos_std=0.3,
                       time_len=64, time_std=0.3, alpha=0.4)


def _perturb(inp, rows, seed=99):
    rng = np.random.default_rng(seed)
    out = JaggedInputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    for name in ("q", "k", "v", "u"):
        arr = getattr(inp, name).copy()
        arr[rows] = rng.standard_normal(arr[rows].shape)
        setattr(out, name, arr)
    ts = inp.timestamps.copy()
    ts[rows] = ts[rows] + rng.integers(1, 10**6, size=len(rows))
    out.timestamps = ts
    return out


@pytest.mark.parametrize("p", [1, 7, 20, 33])
def test_future_perturbation_leaves_past_unchanged(oracle_mod, p):
    inp = _base_flow_inputs(L=40, T=6, c=0)
    a = oracle_mod.forward(inp)
    b = oracle_mod.forward(_perturb(inp, list(range(p, 40))))
    assert np.array_equal(a[:p], b[:p])
    assert not np.array_equal(a[p:], b[p:])


def test_candidates_do_not_see_each_other(oracle_mod):
    inp = _base_flow_inputs(L=40, T=6)
    a = oracle_mod.forward(inp)
    for cand in range(34, 40):
        b = oracle_mod.forward(_perturb(inp, [cand]))
        others = [r for r in range(34, 40) if r != cand]
        assert np.array_equal(a[:34], b[:34])
        assert np.array_equal(a[others], b[others])
        assert not np.array_equal(a[cand], b[cand])


def test_window_limits_reach(oracle_mod):
    W = 5
    inp = _base_flow_inputs(L=40, T=0, W=W)
    a = oracle_mod.forward(inp)
    p = 10
    b = oracle_mod.forward(_perturb(inp, [p]))
    changed = [i for i in range(40) if not np.array_equal(a[i], b[i])]
    assert changed == list(range(p, p + W + 1))


def test_prefix_rows_ignore_history(oracle_mod):
    c = 6
    inp = _base_flow_inputs(L=40, T=4, c=c)
    a = oracle_mod.forward(inp)
    b = oracle_mod.forward(_perturb(inp, list(range(c, 40))))
    assert np.array_equal(a[:c], b[:c])
    # ... while a prefix token reaches every row (bidirectional inside the prefix)
    b2 = oracle_mod.forward(_perturb(inp, [c - 1]))
    assert all(not np.array_equal(a[i], b2[i]) for i in range(40))


# ---------------------------------------------------------------------------
# Jagged layout ("Scaling HSTU", "Variable length is a central systems
# issue"): sequences are independent; permuting them permutes the output.
# ---------------------------------------------------------------------------
def _split(inp, b):
    s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
    return JaggedInputs(
        workload="one", dtype=inp.dtype, offsets=np.array([0, e - s], np.int32),
        num_targets=None if inp.num_targets is None else inp.num_targets[b:b + 1],
        timestamps=None if inp.timestamps is None else inp.timestamps[s:e],
        q=inp.q[s:e], k=inp.k[s:e], v=inp.v[s:e], u=inp.u[s:e], pos_table=inp.pos_table,
        time_table=inp.time_table, contextual_len=inp.contextual_len,
        max_attn_len=inp.max_attn_len, alpha=inp.alpha, n_scale=inp.n_scale)


def test_batch_independence_and_permutation(oracle_mod):
    inp = make_custom([13, 0, 29, 5, 1], num_heads=2, d_qk=8, d_v=8, seed=4,
                      num_targets=[3, 0, 4, 5, 0], contextual_len=2, max_attn_len=6,
                      pos_len=32, time_len=16, alpha=0.5)
    full = oracle_mod.forward(inp)
    for b in range(inp.num_seqs):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        assert np.array_equal(full[s:e], oracle_mod.forward(_split(inp, b)))
    perm = [3, 0, 4, 2, 1]
    parts = [_split(inp, b) for b in perm]
    lens = [p.total_tokens for p in parts]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cat = lambda f: np.concatenate([getattr(p, f) for p in parts])
    pinp = JaggedInputs(workload="perm", dtype="f32", offsets=offs,
                        num_targets=cat("num_targets"), timestamps=cat("timestamps"),
                        q=cat("q"), k=cat("k"), v=cat("v"), u=cat("u"),
                        pos_table=inp.pos_table, time_table=inp.time_table,
                        contextual_len=2, max_attn_len=6, alpha=0.5, n_scale=inp.n_scale)
    pout = oracle_mod.forward(pinp)
    for new_b, b in enumerate(perm):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        assert np.array_equal(pout[offs[new_b]:offs[new_b + 1]], full[s:e])


# ---------------------------------------------------------------------------
# Masking after the nonlinearity must not produce NaN ("Do not copy softmax
# masking mechanically": SiLU of -inf can meet inf * 0).
# ---------------------------------------------------------------------------
def test_overflowing_future_scores_stay_harmless(oracle_mod):
    inp = make_custom([20], d_qk=8, d_v=8, seed=8, alpha=1.0)
    a = oracle_mod.forward(inp)
    bad = JaggedInputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    bad.k = inp.k.copy()
    bad.q = inp.q.copy()
    bad.k[12:] = 3e38           # q_i . k_j far beyond the fp32 range for j >= 12
    bad.q[12:] = -3e38
    b = oracle_mod.forward(bad)
    assert np.all(np.isfinite(b[:12]))
    assert np.array_equal(a[:12], b[:12])


# LayerNorm(o) * u against torch's layer_norm in fp64 (no affine, biased var).
def test_layernorm_gate_matches_torch(oracle_mod):
    import torch
    inp = make_custom([17, 30], num_heads=3, d_qk=16, d_v=16, seed=5, num_targets=[2, 5],
                      pos_len=40, time_len=20, alpha=0.3)
    o = oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_NONE)
    y = oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_LN_U)
    eps = float(np.float32(inp.eps))
    ln = torch.nn.functional.layer_norm(torch.from_numpy(o), (inp.d_v,), eps=eps).numpy()
    assert np.allclose(y, ln * inp.u.astype(np.float64), rtol=1e-12, atol=1e-12)


def test_degenerate_zero_scores(oracle_mod):
    inp = make_custom([9, 4], d_qk=8, d_v=8, seed=6, alpha=0.0)
    assert np.all(oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_NONE) == 0.0)
    assert np.all(oracle_mod.forward(inp) == 0.0)       # LayerNorm of zeros is zero


# ---------------------------------------------------------------------------
# Padding arithmetic of "Scaling HSTU", "Variable length is a central systems
# issue": lengths [10,100,1000] give 3000 padded vs 1110 ragged token
# positions, pair-work ratio 3*1000^2/(10^2+100^2+1000^2) = 2.970; the causal
# pair count is 55 + 5050 + 500500 = 505605.
# ---------------------------------------------------------------------------
def test_padding_arithmetic_tiny_workload(oracle_mod):
    inp = make_inputs("tiny")
    L = inp.lengths
    assert L.tolist() == [10, 100, 1000]
    assert inp.offsets.tolist() == [0, 10, 110, 1110]
    assert len(L) * L.max() == 3000 and L.sum() == 1110
    assert round(len(L) * L.max() ** 2 / float((L ** 2).sum()), 3) == 2.970
    assert oracle_mod.count_allowed(inp.offsets) == 505605
    assert inp.n_scale == 1000.0


# ---------------------------------------------------------------------------
# LayerNorm over all heads of a token (the variant that normalises the
# concatenated H * d_v outputs instead of each head's d_v; "HSTU tensor by
# tensor", section "Similar shape, different aggregation", norm then U gate).
# ---------------------------------------------------------------------------
def test_ln_all_heads_reduces_to_per_head_for_one_head(oracle_mod):
    inp = make_custom([9, 40, 3], num_heads=1, d_qk=8, d_v=8, seed=41, num_targets=[2, 5, 0],
                      pos_len=32, time_len=16, alpha=0.5)
    a = oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_LN_ALL_U)
    b = oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_LN_U)
    assert np.array_equal(a, b)


def test_ln_all_heads_moments_and_scale_invariance(oracle_mod):
    """With u = 1 every token's H * d_v outputs have mean 0 and a mean square
    of at most 1 (exactly var / (var + eps)); scaling v by 1000 leaves them
    unchanged up to the epsilon's share; per-head normalisation does not give
    zero-mean heads' concatenation a unit second moment per head."""
    inp = make_custom([30, 17], num_heads=3, d_qk=8, d_v=8, seed=42, pos_len=64, alpha=0.7,
                      eps=1e-12)
    inp.u = np.ones_like(inp.u)
    a = oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_LN_ALL_U).reshape(inp.total_tokens, -1)
    assert np.abs(a.mean(-1)).max() < 1e-12
    ms = (a ** 2).mean(-1)
    assert np.all(ms <= 1.0 + 1e-12) and np.all(ms > 1.0 - 1e-6)
    inp.v = inp.v * 1000.0
    b = oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_LN_ALL_U).reshape(inp.total_tokens, -1)
    assert np.abs(a - b).max() < 1e-6
    per_head = oracle_mod.forward(inp, epilogue=oracle_mod.EPILOGUE_LN_U).reshape(
        inp.total_tokens, 3, 8)
    assert not np.allclose(per_head.reshape(inp.total_tokens, -1), b, atol=1e-3)


# ---------------------------------------------------------------------------
# Full layer (o_i = W_o[U_i * Norm(sum_j A_ij V_j)] + x_i, "HSTU tensor by
# tensor", teaching equation of "Similar shape, different aggregation").
# ---------------------------------------------------------------------------
def _small_layer(seed, lengths, targets=None, alpha=0.2, pos=True):
    rng = np.random.default_rng(seed)
    H, d, D = 2, 16, 64
    inp = make_custom(lengths, num_heads=H, d_qk=d, d_v=d, seed=seed, num_targets=targets,
                      pos_len=64 if pos else 0, time_len=16, alpha=alpha)
    N = inp.total_tokens
    inp.layer = {"x": rng.standard_normal((N, D)),
                 "w_uvqk": 0.3 * rng.standard_normal((4 * H * d, D)),
                 "b_uvqk": 0.3 * rng.standard_normal(4 * H * d),
                 "w_o": 0.3 * rng.standard_normal((D, H * d))}
    return inp


def test_layer_zero_scores_is_identity(oracle_mod):
    """alpha = 0 and no bias tables: every score is 0, SiLU(0) = 0, the
    aggregate and its normalisation are 0, so y = x exactly."""
    inp = _small_layer(50, [7, 20, 1], targets=[2, 3, 0], alpha=0.0, pos=False)
    inp.time_table = None
    inp.timestamps = None
    y = oracle_mod.layer_forward(inp)
    assert np.array_equal(y, inp.layer["x"])


def test_layer_single_token_closed_form(oracle_mod):
    """One-token sequences: o = SiLU(s)/n * v with s = alpha q.k + pos[0] +
    time[0], and LayerNorm(c v) = sign(c) LayerNorm(v) (eps negligible), so
    y = W_o (u * sign(SiLU(s)) * LN(v)) + x, computed here from the projected
    branches without the attention loop."""
    inp = _small_layer(51, [1, 1, 1, 1], alpha=0.7)
    inp.eps = 1e-12
    y = oracle_mod.layer_forward(inp)
    L = inp.layer
    x = L["x"]
    xn = (x - x.mean(1, keepdims=True)) / np.sqrt(x.var(1, keepdims=True) + float(np.float32(1e-12)))
    z = xn @ L["w_uvqk"].T + L["b_uvqk"]
    br = z / (1 + np.exp(-z))
    H, d = 2, 16
    U, V = br[:, :H * d].reshape(-1, H, d), br[:, H * d:2 * H * d].reshape(-1, H, d)
    Q, K = br[:, 2 * H * d:3 * H * d].reshape(-1, H, d), br[:, 3 * H * d:].reshape(-1, H, d)
    s = inp.alpha * (Q * K).sum(-1) + inp.pos_table[0] + inp.time_table[0]
    sgn = np.sign(s / (1 + np.exp(-s)))[..., None]
    lnv = (V - V.mean(-1, keepdims=True)) / V.std(-1, keepdims=True)
    want = (U * sgn * lnv).reshape(-1, H * d) @ L["w_o"].T + x
    assert np.abs(y - want).max() < 1e-6 * np.abs(want).max()


def _allowed_count(oracle_mod, inp, b, i):
    """Allowed keys of row i of sequence b, counted with the rule predicate
    (pinned by the hand-worked masks and the dense brute force)."""
    L = int(inp.lengths[b])
    t = 0 if inp.num_targets is None else int(inp.num_targets[b])
    return sum(oracle_mod.allowed(L, t, inp.contextual_len, inp.max_attn_len, i, j)
               for j in range(L))


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _ln_rows(a, eps):
    mu = a.mean(axis=-1, keepdims=True)
    return (a - mu) / np.sqrt(((a - mu) ** 2).mean(axis=-1, keepdims=True) + eps)


@pytest.mark.parametrize("rules", [dict(num_targets=[3, 0, 5], contextual_len=2),
                                   dict(num_targets=[2, 4, 0], max_attn_len=5)])
def test_layer_constant_branches_closed_form(oracle_mod, rules):
    """Zero projection weights and a different bias on every column make the
    four branches per-head constant vectors, U = SiLU(b_U), V = SiLU(b_V),
    Q = SiLU(b_Q), K = SiLU(b_K) (the split order U | V | Q | K, the bias and
    SiLU on every column, "HSTU tensor by tensor": "Trace four projections").
    With no bias tables every allowed score of head h is alpha <Q_h, K_h>, so
    row i aggregates n_i SiLU(s_h) / n_scale V_h, n_i = its allowed keys; the
    closed form needs no attention loop.  A wrong block order, a missing bias
    or SiLU skipped on a block all change the result."""
    H, d, D = 2, 16, 64
    rng = np.random.default_rng(60)
    inp = make_custom([9, 14, 6], num_heads=H, d_qk=d, d_v=d, seed=60, alpha=0.7,
                      n_scale=11.0, **rules)
    inp.pos_table = inp.time_table = inp.timestamps = None
    N = inp.total_tokens
    bias = rng.standard_normal(4 * H * d)
    inp.layer = {"x": rng.standard_normal((N, D)), "w_uvqk": np.zeros((4 * H * d, D)),
                 "b_uvqk": bias, "w_o": 0.3 * rng.standard_normal((D, H * d))}
    y = oracle_mod.layer_forward(inp)

    U, V, Q, K = (_silu(bias[k * H * d:(k + 1) * H * d]).reshape(H, d) for k in range(4))
    s = inp.alpha * (Q * K).sum(-1)                        # [H]
    eps = float(np.float32(inp.eps))
    want = np.empty_like(y)
    for b in range(inp.num_seqs):
        s0 = int(inp.offsets[b])
        for i in range(int(inp.lengths[b])):
            c = _allowed_count(oracle_mod, inp, b, i) * _silu(s) / inp.n_scale   # [H]
            gate = U * _ln_rows(c[:, None] * V, eps)        # [H, d]
            want[s0 + i] = inp.layer["x"][s0 + i] + inp.layer["w_o"] @ gate.reshape(-1)
    assert np.abs(y - want).max() <= 1e-12 * np.abs(want).max()
    # the same closed form with the U and V blocks exchanged is far off
    swapped = np.empty_like(y)
    for b in range(inp.num_seqs):
        s0 = int(inp.offsets[b])
        for i in range(int(inp.lengths[b])):
            c = _allowed_count(oracle_mod, inp, b, i) * _silu(s) / inp.n_scale
            gate = V * _ln_rows(c[:, None] * U, eps)
            swapped[s0 + i] = inp.layer["x"][s0 + i] + inp.layer["w_o"] @ gate.reshape(-1)
    assert np.abs(y - swapped).max() > 1e-3 * np.abs(want).max()


def test_layer_u_branch_reads_normalised_input(oracle_mod):
    """Only the U block of the projection has weights; V, Q, K are constant
    (biases), and W_o = [I; 0] copies the gated heads into the first H d
    columns of y - x.  Then (y - x)[:, :Hd] = SiLU(LN(x) W_U^T + b_U) * g_i with
    g_i the closed-form normalised aggregate of the constant V, and LN(x) is
    torch's layer_norm (no affine, eps from the inputs).  Rows scaled by 1e-3
    have a variance below eps, so a wrong epsilon shows."""
    torch = pytest.importorskip("torch")
    H, d, D = 2, 16, 64
    rng = np.random.default_rng(61)
    inp = make_custom([7, 12], num_heads=H, d_qk=d, d_v=d, seed=61, alpha=0.4, n_scale=9.0,
                      num_targets=[2, 3])
    inp.pos_table = inp.time_table = inp.timestamps = None
    N, Hd = inp.total_tokens, H * d
    x = rng.standard_normal((N, D))
    x[::3] *= 1e-3
    w = np.zeros((4 * Hd, D))
    w[:Hd] = 0.5 * rng.standard_normal((Hd, D))
    bias = rng.standard_normal(4 * Hd)
    w_o = np.zeros((D, Hd))
    w_o[:Hd, :Hd] = np.eye(Hd)
    inp.layer = {"x": x, "w_uvqk": w, "b_uvqk": bias, "w_o": w_o}
    y = oracle_mod.layer_forward(inp)

    eps = float(np.float32(inp.eps))
    xn = torch.nn.functional.layer_norm(torch.from_numpy(x), (D,), eps=eps).numpy()
    U = _silu(xn @ w[:Hd].T + bias[:Hd]).reshape(N, H, d)
    V, Q, K = (_silu(bias[k * Hd:(k + 1) * Hd]).reshape(H, d) for k in (1, 2, 3))
    s = inp.alpha * (Q * K).sum(-1)
    got = (y - x)[:, :Hd].reshape(N, H, d)
    assert np.all((y - x)[:, Hd:] == 0)
    for b in range(inp.num_seqs):
        s0 = int(inp.offsets[b])
        for i in range(int(inp.lengths[b])):
            c = _allowed_count(oracle_mod, inp, b, i) * _silu(s) / inp.n_scale
            want = U[s0 + i] * _ln_rows(c[:, None] * V, eps)
            assert np.abs(got[s0 + i] - want).max() <= 1e-12 * max(np.abs(want).max(), 1e-300)


def test_layer_head_relabelling_invariance(oracle_mod):
    """Heads are independent and each is a contiguous d-wide slice of every
    branch block: relabelling the heads the same way in all four blocks of the
    projection and in the columns of W_o leaves the layer output unchanged."""
    inp = _small_layer(62, [11, 25, 4], targets=[3, 5, 0])
    H, d = inp.num_heads, inp.d_v
    y = oracle_mod.layer_forward(inp)
    perm = np.array([1, 0])
    L = inp.layer
    rows = np.concatenate([blk * H * d + (perm[h] * d + np.arange(d))
                           for blk in range(4) for h in range(H)])
    cols = np.concatenate([perm[h] * d + np.arange(d) for h in range(H)])
    inp2 = dataclasses.replace(inp, layer={"x": L["x"], "w_uvqk": L["w_uvqk"][rows],
                                           "b_uvqk": L["b_uvqk"][rows],
                                           "w_o": L["w_o"][:, cols]})
    y2 = oracle_mod.layer_forward(inp2)
    assert np.abs(y - y2).max() <= 1e-12 * np.abs(y).max()
    # relabelling only the projection (not W_o) does change it
    inp3 = dataclasses.replace(inp2, layer=dict(inp2.layer, w_o=L["w_o"]))
    assert np.abs(y - oracle_mod.layer_forward(inp3)).max() > 1e-6 * np.abs(y).max()


def test_layer_rows_subset(oracle_mod):
    inp = _small_layer(52, [30, 9, 40], targets=[3, 0, 5])
    full = oracle_mod.layer_forward(inp)
    rows = np.array([0, 5, 29, 33, 77, 78])
    part = oracle_mod.layer_forward(inp, rows=rows)
    assert np.abs(full[rows] - part[rows]).max() <= 1e-12 * np.abs(full).max()


# ---------------------------------------------------------------------------
# Position bias at clamped positions (alternative reading of the candidate
# clamp, "HSTU-MUSA", section "Mathematical Equivalence": every candidate sits
# at the history end).  Pinned by what the clamp is for -- candidates become
# interchangeable ("Scaling HSTU", section "Many candidates make reuse
# valuable") -- and by the dense form built from a clamped position vector.
# ---------------------------------------------------------------------------
def _clamp_case(seed, T=6, L=40, W=0, c=0):
    return make_custom([L, 23, L + 5], num_heads=2, d_qk=8, d_v=8, seed=seed,
                       num_targets=[T, 3, T], contextual_len=c, max_attn_len=W, pos_len=64,
                       pos_std=0.5, time_len=16, time_std=0.5, alpha=0.5)


def test_pos_clamp_without_candidates_changes_nothing(oracle_mod):
    inp = make_custom([30, 17], num_heads=2, d_qk=8, d_v=8, seed=3, pos_len=64, pos_std=0.5,
                      time_len=16, alpha=0.5)
    a = oracle_mod.forward(inp)
    b = oracle_mod.forward(inp, pos_clamp=True)
    assert np.array_equal(a, b)


def test_pos_clamp_leaves_history_rows(oracle_mod):
    inp = _clamp_case(5, W=9, c=3)
    a = oracle_mod.forward(inp)
    b = oracle_mod.forward(inp, pos_clamp=True)
    hist = []
    for bq in range(inp.num_seqs):
        s0, s1 = int(inp.offsets[bq]), int(inp.offsets[bq + 1])
        hist.extend(range(s0, s1 - int(inp.num_targets[bq])))
    assert np.array_equal(a[hist], b[hist])
    assert not np.allclose(a, b)        # the candidates' rows do change


@pytest.mark.parametrize("W", [0, 7])
def test_pos_clamp_makes_candidates_interchangeable(oracle_mod, W):
    """Permuting the candidates of a sequence (all their inputs, timestamps
    included) permutes their outputs when the bias is clamped -- and not with
    the raw bias, which tells candidates apart by position."""
    inp = _clamp_case(7, W=W)
    s0, s1 = int(inp.offsets[0]), int(inp.offsets[1])
    cand = np.arange(s1 - 6, s1)
    perm = cand[np.random.default_rng(1).permutation(6)]
    order = np.arange(inp.total_tokens)
    order[cand] = perm
    shuffled = dataclasses.replace(
        inp, q=inp.q[order], k=inp.k[order], v=inp.v[order], u=inp.u[order],
        timestamps=inp.timestamps[order])
    a = oracle_mod.forward(inp, pos_clamp=True)
    b = oracle_mod.forward(shuffled, pos_clamp=True)
    assert np.allclose(b[cand], a[perm], rtol=0, atol=1e-12)
    raw_a = oracle_mod.forward(inp)
    raw_b = oracle_mod.forward(shuffled)
    assert not np.allclose(raw_b[cand], raw_a[perm], rtol=0, atol=1e-9)


@pytest.mark.parametrize("seed", range(12))
def test_pos_clamp_equals_dense_bruteforce(oracle_mod, seed):
    inp = _random_case(100 + seed)
    for ep in (oracle_mod.EPILOGUE_NONE, oracle_mod.EPILOGUE_LN_U):
        a = oracle_mod.forward(inp, epilogue=ep, pos_clamp=True)
        b = oracle_mod.dense_forward(inp, epilogue=ep, pos_clamp=True)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
