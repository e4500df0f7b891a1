"""Pins the oracle's backward to the oracle's forward, which the other pin
file ties to the pages.

The backward (dq, dk, dv, du and the two bias-table gradients) is the chain
rule of the forward; none of these tests retypes it.  They compare it with
central finite differences of the fp64 forward -- the definition of a
derivative -- along random directions and entry by entry, and check the
causality the teaching equation of "HSTU tensor by tensor: SiLU aggregation,
temporal bias and gating" (section "Similar shape, different aggregation")
fixes: a loss on early rows cannot depend on later tokens.
"""
import dataclasses

import numpy as np
import pytest

from jagged_hstu_attention_attn_amd.inputs import make_custom

_KEYS = {"q": "dq", "k": "dk", "v": "dv", "u": "du", "pos_table": "dpos",
         "time_table": "dtime"}


def _loss(oracle_mod, inp, dout, epilogue, pos_clamp=False, **repl):
    x = dataclasses.replace(inp, **repl)
    return float((oracle_mod.forward(x, epilogue=epilogue, nthreads=2,
                                     pos_clamp=pos_clamp) * dout).sum())


def _fd_dir(oracle_mod, inp, dout, epilogue, name, direction, h=1e-6, pos_clamp=False):
    x = getattr(inp, name).astype(np.float64)
    plus = _loss(oracle_mod, inp, dout, epilogue, pos_clamp, **{name: x + h * direction})
    minus = _loss(oracle_mod, inp, dout, epilogue, pos_clamp, **{name: x - h * direction})
    return (plus - minus) / (2 * h)


_GEOMS = {
    # causal only, one head
    "causal": dict(lengths=[7, 1, 12], num_heads=1),
    # bidirectional prefix + candidates + window, two heads
    "all_rules": dict(lengths=[9, 14, 5], num_heads=2, num_targets=[3, 4, 5],
                      contextual_len=3, max_attn_len=4),
    # window shorter than the history, candidates on every sequence
    "window": dict(lengths=[16, 11], num_heads=2, num_targets=[2, 6], max_attn_len=2),
}


def _case(geom, seed):
    kw = dict(_GEOMS[geom])
    inp = make_custom(kw.pop("lengths"), d_qk=4, d_v=4, pos_len=7, pos_std=0.5,
                      time_len=6, time_std=0.5, alpha=0.6, seed=seed, **kw)
    dout = np.random.default_rng(seed + 100).standard_normal(inp.v.shape)
    return inp, dout


@pytest.mark.parametrize("geom", sorted(_GEOMS))
@pytest.mark.parametrize("epilogue", [0, 1, 2])
def test_directional_derivatives(oracle_mod, geom, epilogue):
    """<grad, d> equals the central difference of the forward along d, for a
    random direction d of every input (a dropped term, wrong sign or index in
    any gradient moves this far beyond the 1e-6 bar)."""
    inp, dout = _case(geom, seed=7)
    g = oracle_mod.backward(inp, dout, epilogue=epilogue, nthreads=2)
    rng = np.random.default_rng(5)
    for name, key in _KEYS.items():
        x = getattr(inp, name)
        d = rng.standard_normal(x.shape)
        fd = _fd_dir(oracle_mod, inp, dout, epilogue, name, d)
        an = float((g[key] * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    if epilogue == oracle_mod.EPILOGUE_NONE:
        assert not np.any(g["du"])      # u plays no part without the gate


@pytest.mark.parametrize("epilogue", [0, 2])
def test_table_gradients_entry_by_entry(oracle_mod, epilogue):
    """Every entry of d(pos_table) and d(time_table), including the clamped
    last buckets and buckets no pair uses (gradient exactly 0)."""
    inp, dout = _case("all_rules", seed=11)
    g = oracle_mod.backward(inp, dout, epilogue=epilogue, nthreads=2)
    for name, key in (("pos_table", "dpos"), ("time_table", "dtime")):
        n = getattr(inp, name).shape[0]
        for e in range(n):
            d = np.zeros(n)
            d[e] = 1.0
            fd = _fd_dir(oracle_mod, inp, dout, epilogue, name, d)
            assert abs(fd - g[key][e]) <= 1e-6 * max(1.0, abs(g[key][e])), (name, e)


def test_token_gradients_entry_by_entry(oracle_mod):
    """Single entries of dq, dk, dv, du: a history token, a prefix token and a
    candidate token (which only its own row sees), of both heads."""
    inp, dout = _case("all_rules", seed=13)
    g = oracle_mod.backward(inp, dout, epilogue=0, nthreads=2)
    # sequence 1 spans tokens 9..22 with c = 3 and 4 candidates (19..22)
    for tok in (9, 10, 15, 19, 22):
        for h in (0, 1):
            for name, key in _KEYS.items():
                if name in ("pos_table", "time_table"):
                    continue
                x = getattr(inp, name)
                e = (tok + h) % x.shape[2]
                d = np.zeros(x.shape)
                d[tok, h, e] = 1.0
                fd = _fd_dir(oracle_mod, inp, dout, 0, name, d)
                an = g[key][tok, h, e]
                assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, tok, h)


def test_causality_of_gradients(oracle_mod):
    """A loss on the first r rows of a causal sequence has zero gradient with
    respect to every later token's q, k, v and u."""
    inp, _ = _case("causal", seed=17)
    r = 5                                 # rows 0..4 of sequence 0 (length 7)
    dout = np.zeros(inp.v.shape)
    dout[:r] = np.random.default_rng(3).standard_normal(dout[:r].shape)
    g = oracle_mod.backward(inp, dout, epilogue=0, nthreads=2)
    for key in ("dq", "dk", "dv", "du"):
        assert not np.any(g[key][r:]), key
        assert np.any(g[key][:r]), key


def test_zero_upstream_gives_zero(oracle_mod):
    inp, dout = _case("window", seed=19)
    g = oracle_mod.backward(inp, np.zeros_like(dout), epilogue=0, nthreads=2)
    for key, val in g.items():
        assert not np.any(val), key


def test_empty_batch(oracle_mod):
    inp = make_custom([0, 0], d_qk=4, d_v=4, pos_len=3, time_len=2)
    g = oracle_mod.backward(inp, np.zeros((0, 1, 4)), epilogue=0)
    assert g["dq"].shape == (0, 1, 4)
    assert not np.any(g["dpos"]) and not np.any(g["dtime"])


@pytest.mark.parametrize("geom", ["all_rules", "window"])
def test_clamped_position_bias_gradients(oracle_mod, geom):
    """With the position bias taken at clamped positions (p = min(position,
    n_h), the candidate clamp of the mask applied to the bias), every
    gradient still equals the central difference of the clamped forward:
    along random directions for all inputs and entry by entry for the
    position table, whose candidate pairs now land on |n_h - j|.  The
    clamped and raw readings must differ here (the geometry has candidates
    whose bias index changes)."""
    inp, dout = _case(geom, seed=17)
    g = oracle_mod.backward(inp, dout, epilogue=0, nthreads=2, pos_clamp=True)
    raw = oracle_mod.backward(inp, dout, epilogue=0, nthreads=2)
    assert not np.allclose(g["dpos"], raw["dpos"])
    rng = np.random.default_rng(9)
    for name, key in _KEYS.items():
        x = getattr(inp, name)
        d = rng.standard_normal(x.shape)
        fd = _fd_dir(oracle_mod, inp, dout, 0, name, d, pos_clamp=True)
        an = float((g[key] * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    n = inp.pos_table.shape[0]
    for e in range(n):
        d = np.zeros(n)
        d[e] = 1.0
        fd = _fd_dir(oracle_mod, inp, dout, 0, "pos_table", d, pos_clamp=True)
        assert abs(fd - g["dpos"][e]) <= 1e-6 * max(1.0, abs(g["dpos"][e])), e
