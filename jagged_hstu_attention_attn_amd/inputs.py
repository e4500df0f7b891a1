"""Seeded synthetic inputs for jagged HSTU attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path and the CPU oracle take their inputs
from here, so that they see bit-identical values.

Workloads (sizes and distributions follow the HSTU ranking setup of the
"HSTU-MUSA" page, section "Accuracy Alignment with recsys-examples", and the
jagged-layout discussion of "Scaling HSTU: ragged execution, candidate
amortization and content features", section "Variable length is a central
systems issue"):

  tiny      lengths [10,100,1000], 1 head, d=8, fp32, causal, position bias only
  ranking   128 sequences, history ~ U[20,200] + 20 candidates, 4 heads, d=128, bf16
  longtail  32 sequences, length clamp(rint(lognormal(6,1)),16,4096), 6-token
            bidirectional prefix, 4 heads, d=128, bf16
  windowed  16 sequences, length ~ U[2048,8192], window 1024, 50 candidates
  layer     64 sequences, history clamp(rint(lognormal(6.5,0.8)),32,2048) + 20
            candidates; inputs of a full HSTU layer (x and weights)

Draw order (fixed): lengths -> per-sequence timestamps -> pos_table ->
time_table -> Q -> K -> V -> U -> layer weights.  Integer draws use numpy.rint
(half to even) before clamping; U[a,b] is inclusive.  Timestamps are
t0 + cumsum(rint(Exp(3600))) with a first gap of 0, in int64 seconds.
Floating inputs are float32 standard normal draws, rounded to bfloat16 (round
to nearest even) when the workload is bf16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "JaggedInputs",
    "make_inputs",
    "make_custom",
    "bf16_round",
    "bf16_bits",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_heads: int
    d_qk: int
    d_v: int
    dtype: str                      # "f32" | "bf16"
    lengths: str                    # "fixed" | "ranking" | "lognormal" | "uniform"
    fixed_lengths: tuple = ()
    hist_lo: int = 0                # ranking: history ~ U[hist_lo, hist_hi]
    hist_hi: int = 0
    ln_mu: float = 0.0              # lognormal parameters
    ln_sigma: float = 0.0
    len_lo: int = 0                 # clamp / uniform bounds
    len_hi: int = 0
    num_candidates: int = 0         # candidates appended per sequence
    candidates_in_length: bool = False  # True: the drawn length already includes them
    contextual_len: int = 0
    max_attn_len: int = 0
    pos_len: int = 0
    pos_std: float = 0.0
    time_len: int = 0
    time_std: float = 0.0
    alpha: float = 1.0
    seed: int = 1234
    hidden: int = 0                 # layer workload only
    weight_std: float = 0.0


WORKLOADS = {
    "tiny": Workload(
        name="tiny", num_seqs=3, num_heads=1, d_qk=8, d_v=8, dtype="f32",
        lengths="fixed", fixed_lengths=(10, 100, 1000),
        pos_len=1024, pos_std=0.1, alpha=1.0 / math.sqrt(8.0), seed=0),
    "ranking": Workload(
        name="ranking", num_seqs=128, num_heads=4, d_qk=128, d_v=128, dtype="bf16",
        lengths="ranking", hist_lo=20, hist_hi=200, num_candidates=20,
        pos_len=4096, pos_std=0.02, time_len=64, time_std=0.02,
        alpha=1.0 / math.sqrt(128.0), seed=1234),
    "longtail": Workload(
        name="longtail", num_seqs=32, num_heads=4, d_qk=128, d_v=128, dtype="bf16",
        lengths="lognormal", ln_mu=6.0, ln_sigma=1.0, len_lo=16, len_hi=4096,
        contextual_len=6,
        pos_len=4096, pos_std=0.02, time_len=64, time_std=0.02,
        alpha=1.0 / math.sqrt(128.0), seed=1234),
    "windowed": Workload(
        name="windowed", num_seqs=16, num_heads=4, d_qk=128, d_v=128, dtype="bf16",
        lengths="uniform", len_lo=2048, len_hi=8192, num_candidates=50,
        candidates_in_length=True, max_attn_len=1024,
        pos_len=4096, pos_std=0.02, time_len=64, time_std=0.02,
        alpha=1.0 / math.sqrt(128.0), seed=1234),
    "layer": Workload(
        name="layer", num_seqs=64, num_heads=4, d_qk=128, d_v=128, dtype="bf16",
        lengths="lognormal", ln_mu=6.5, ln_sigma=0.8, len_lo=32, len_hi=2048,
        num_candidates=20,
        pos_len=4096, pos_std=0.02, time_len=64, time_std=0.02,
        alpha=1.0 / math.sqrt(128.0), seed=1234, hidden=512, weight_std=0.02),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16, returned as float32."""
    bits = bf16_bits(x).astype(np.uint32) << 16
    return bits.view(np.float32)


@dataclasses.dataclass
class JaggedInputs:
    """One batch of jagged inputs.  Tensors are [total_tokens, H, d] row-major
    (token stride H*d elements), holding exactly the values the device sees
    (already bf16-rounded for bf16 workloads, stored as float32)."""
    workload: str
    dtype: str
    offsets: np.ndarray             # int32 [B+1]
    num_targets: Optional[np.ndarray]   # int32 [B] or None
    timestamps: Optional[np.ndarray]    # int64 [N] or None
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    u: np.ndarray
    pos_table: Optional[np.ndarray]     # float32 [P] or None
    time_table: Optional[np.ndarray]    # float32 [Tt] or None
    contextual_len: int
    max_attn_len: int
    alpha: float
    n_scale: float
    eps: float = 1e-5
    layer: Optional[dict] = None

    @property
    def num_seqs(self) -> int:
        return int(self.offsets.shape[0] - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.offsets[-1])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def d_qk(self) -> int:
        return int(self.q.shape[2])

    @property
    def d_v(self) -> int:
        return int(self.v.shape[2])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets.astype(np.int64))


def _draw_lengths(w: Workload, rng: np.random.Generator):
    """Returns (total lengths, number of candidates per sequence)."""
    B = w.num_seqs
    if w.lengths == "fixed":
        hist = np.asarray(w.fixed_lengths, dtype=np.int64)
    elif w.lengths == "ranking":
        hist = rng.integers(w.hist_lo, w.hist_hi + 1, size=B).astype(np.int64)
    elif w.lengths == "lognormal":
        raw = rng.lognormal(mean=w.ln_mu, sigma=w.ln_sigma, size=B)
        hist = np.clip(np.rint(raw), w.len_lo, w.len_hi).astype(np.int64)
    elif w.lengths == "uniform":
        hist = rng.integers(w.len_lo, w.len_hi + 1, size=B).astype(np.int64)
    else:
        raise ValueError(w.lengths)
    cand = np.full(B, w.num_candidates, dtype=np.int64)
    total = hist if w.candidates_in_length else hist + cand
    return total, cand


def _draw_timestamps(lengths: np.ndarray, rng: np.random.Generator, t0: int) -> np.ndarray:
    parts = []
    for L in lengths.tolist():
        gaps = np.rint(rng.exponential(3600.0, size=L)).astype(np.int64)
        if L > 0:
            gaps[0] = 0
        parts.append(t0 + np.cumsum(gaps))
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(parts).astype(np.int64)


def _normal(rng, shape, dtype: str, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def make_inputs(name: str, seed: Optional[int] = None, *, num_seqs: Optional[int] = None,
                t0: int = 1_700_000_000, dtype: Optional[str] = None) -> JaggedInputs:
    """Inputs for a named workload.  `num_seqs` truncates the batch (the draws
    are made for the full batch first, so a truncated batch is a prefix of the
    full one); `dtype` overrides the element type (f32 shadow runs)."""
    w = WORKLOADS[name]
    seed = w.seed if seed is None else seed
    dt = w.dtype if dtype is None else dtype
    rng = np.random.default_rng(seed)
    lengths, cand = _draw_lengths(w, rng)
    ts_all = _draw_timestamps(lengths, rng, t0) if w.time_len else None
    pos = _normal(rng, (w.pos_len,), "f32", w.pos_std) if w.pos_len else None
    tim = _normal(rng, (w.time_len,), "f32", w.time_std) if w.time_len else None
    B_full = w.num_seqs
    N_full = int(lengths.sum())
    H = w.num_heads
    q = _normal(rng, (N_full, H, w.d_qk), dt)
    k = _normal(rng, (N_full, H, w.d_qk), dt)
    v = _normal(rng, (N_full, H, w.d_v), dt)
    u = _normal(rng, (N_full, H, w.d_v), dt)
    layer = None
    if w.hidden:
        D = w.hidden
        layer = {
            "x": _normal(rng, (N_full, D), dt),
            "w_uvqk": _normal(rng, (2 * H * w.d_v + 2 * H * w.d_qk, D), dt, w.weight_std),
            "b_uvqk": _normal(rng, (2 * H * w.d_v + 2 * H * w.d_qk,), dt, w.weight_std),
            "w_o": _normal(rng, (D, H * w.d_v), dt, w.weight_std),
        }
    B = B_full if num_seqs is None else min(num_seqs, B_full)
    lengths = lengths[:B]
    cand = cand[:B]
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lengths)
    N = int(offsets[-1])
    targets = cand.astype(np.int32) if w.num_candidates else None
    ts = ts_all[:N].copy() if ts_all is not None else None
    if layer is not None:
        layer = dict(layer)
        layer["x"] = layer["x"][:N].copy()
    n_scale = float(lengths.max()) if B > 0 else 1.0
    return JaggedInputs(
        workload=name, dtype=dt, offsets=offsets.astype(np.int32), num_targets=targets,
        timestamps=ts, q=q[:N].copy(), k=k[:N].copy(), v=v[:N].copy(), u=u[:N].copy(),
        pos_table=pos, time_table=tim, contextual_len=w.contextual_len,
        max_attn_len=w.max_attn_len, alpha=float(w.alpha), n_scale=n_scale, layer=layer)


def make_custom(lengths, *, num_heads: int = 1, d_qk: int = 8, d_v: int = 8,
                dtype: str = "f32", seed: int = 0, num_targets=None,
                contextual_len: int = 0, max_attn_len: int = 0,
                pos_len: int = 0, pos_std: float = 0.02,
                time_len: int = 0, time_std: float = 0.02,
                alpha: float = 1.0, n_scale: Optional[float] = None,
                t0: int = 1_700_000_000, eps: float = 1e-5) -> JaggedInputs:
    """Small hand-shaped inputs for edge cases (same draw order as make_inputs)."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(list(lengths), dtype=np.int64)
    B = lengths.shape[0]
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lengths)
    N = int(offsets[-1])
    ts = _draw_timestamps(lengths, rng, t0) if time_len else None
    pos = _normal(rng, (pos_len,), "f32", pos_std) if pos_len else None
    tim = _normal(rng, (time_len,), "f32", time_std) if time_len else None
    q = _normal(rng, (N, num_heads, d_qk), dtype)
    k = _normal(rng, (N, num_heads, d_qk), dtype)
    v = _normal(rng, (N, num_heads, d_v), dtype)
    u = _normal(rng, (N, num_heads, d_v), dtype)
    if num_targets is not None:
        num_targets = np.asarray(num_targets, dtype=np.int32)
    if n_scale is None:
        n_scale = float(lengths.max()) if B and lengths.max() > 0 else 1.0
    return JaggedInputs(
        workload="custom", dtype=dtype, offsets=offsets.astype(np.int32),
        num_targets=num_targets, timestamps=ts, q=q, k=k, v=v, u=u,
        pos_table=pos, time_table=tim, contextual_len=contextual_len,
        max_attn_len=max_attn_len, alpha=float(alpha), n_scale=float(n_scale), eps=eps)
