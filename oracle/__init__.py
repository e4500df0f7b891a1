"""CPU oracle for jagged HSTU attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
touches it, and it shares no code with them: the only common module is the
seeded input generator, which holds none of the method's arithmetic.

The backward (`backward`) is the chain rule through the same steps, one
allowed pair at a time, in the same C file.

Two independent formulations of the forward live here:
  * `forward`  -- the fp64 C loop in hstu_oracle.c (one pair at a time, only
    allowed pairs evaluated), built by `build()` with gcc -O2 -fopenmp.
  * `dense_forward` -- the padded dense form of the teaching snippet on the
    page "HSTU tensor by tensor: SiLU aggregation, temporal bias and gating"
    (section "Trace four projections"): SiLU over the whole padded score
    matrix, then masked_fill of illegal entries with 0, then A @ V.  numpy
    fp64, for tiny inputs only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hstu_oracle.c")
_LIB = os.path.join(_HERE, "libhstu_oracle.so")

EPILOGUE_LN_U = 0
EPILOGUE_NONE = 1
EPILOGUE_LN_ALL_U = 2   # LayerNorm over all heads' d_v of a token, then * u

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle (plain fp64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.hstu_oracle_fwd.restype = ctypes.c_int
        lib.hstu_oracle_fwd.argtypes = [
            i32, P, i32, i32, i32,
            P, i64, P, i64, P, i64, P, i64,
            P, P, i32, i32, f64, f64,
            P, i32, P, i32, f64, i32, P, i64, P, i32, i32]
        lib.hstu_oracle_bwd.restype = ctypes.c_int
        lib.hstu_oracle_bwd.argtypes = [
            i32, P, i32, i32, i32,
            P, i64, P, i64, P, i64, P, i64,
            P, P, i32, i32, f64, f64,
            P, i32, P, i32, f64, i32, P, i64,
            P, P, P, P, P, P, i32, i32]
        lib.hstu_oracle_count_allowed.restype = i64
        lib.hstu_oracle_count_allowed.argtypes = [i32, P, P, i32, i32]
        lib.hstu_oracle_time_bucket.restype = ctypes.c_int
        lib.hstu_oracle_time_bucket.argtypes = [i64, i64]
        lib.hstu_oracle_silu.restype = f64
        lib.hstu_oracle_silu.argtypes = [f64]
        lib.hstu_oracle_allowed.restype = ctypes.c_int
        lib.hstu_oracle_allowed.argtypes = [i64, i64, i64, i64, i64, i64]
        lib.hstu_oracle_max_threads.restype = ctypes.c_int
        lib.hstu_oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def forward_arrays(offsets, q, k, v, u, *, timestamps=None, num_targets=None,
                   contextual_len=0, max_attn_len=0, alpha=1.0, n_scale=1.0,
                   pos_table=None, time_table=None, eps=1e-5, epilogue=EPILOGUE_LN_U,
                   rows=None, nthreads: Optional[int] = None, pos_clamp=False) -> np.ndarray:
    """fp64 forward on [N, H, d] arrays (any float dtype; upcast exactly).
    `rows`: optional token indices; only those output rows are computed (the
    others are NaN).  `pos_clamp`: position bias at clamped positions
    min(position, n_h) (the alternative reading of the candidate clamp)."""
    lib = _load()
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    N, H, dqk = q.shape
    dv = v.shape[2]
    ts = None if timestamps is None else np.ascontiguousarray(timestamps, dtype=np.int64)
    nt = None if num_targets is None else np.ascontiguousarray(num_targets, dtype=np.int32)
    pos = None if pos_table is None else np.ascontiguousarray(pos_table, dtype=np.float64)
    tim = None if time_table is None else np.ascontiguousarray(time_table, dtype=np.float64)
    sel = None
    if rows is not None:
        sel = np.zeros(N, dtype=np.uint8)
        sel[np.asarray(rows, dtype=np.int64)] = 1
        out = np.full((N, H, dv), np.nan, dtype=np.float64)
    else:
        out = np.zeros((N, H, dv), dtype=np.float64)
    rc = lib.hstu_oracle_fwd(
        offsets.shape[0] - 1, _ptr(offsets), H, dqk, dv,
        _ptr(q), H * dqk, _ptr(k), H * dqk, _ptr(v), H * dv, _ptr(u), H * dv,
        _ptr(ts), _ptr(nt), int(contextual_len), int(max_attn_len),
        float(alpha), float(n_scale),
        _ptr(pos), 0 if pos is None else pos.shape[0],
        _ptr(tim), 0 if tim is None else tim.shape[0],
        float(np.float32(eps)), int(epilogue), _ptr(out), H * dv, _ptr(sel),
        int(nthreads if nthreads is not None else default_threads()), int(bool(pos_clamp)))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def forward(inp, *, epilogue=EPILOGUE_LN_U, rows=None,
            nthreads: Optional[int] = None, pos_clamp=False) -> np.ndarray:
    """fp64 forward of a `JaggedInputs` batch (optionally only token `rows`)."""
    return forward_arrays(
        inp.offsets, inp.q, inp.k, inp.v, inp.u, timestamps=inp.timestamps,
        num_targets=inp.num_targets, contextual_len=inp.contextual_len,
        max_attn_len=inp.max_attn_len, alpha=inp.alpha, n_scale=inp.n_scale,
        pos_table=inp.pos_table, time_table=inp.time_table, eps=inp.eps,
        epilogue=epilogue, rows=rows, nthreads=nthreads, pos_clamp=pos_clamp)


def layer_forward(inp, *, rows=None, nthreads: Optional[int] = None) -> np.ndarray:
    """fp64 forward of the full HSTU layer on a batch with `inp.layer` weights
    ("HSTU tensor by tensor: SiLU aggregation, temporal bias and gating":
    "Trace four projections" -- normalised inputs give U/V/Q/K through one
    projection; the teaching equation of "Similar shape, different
    aggregation" -- o_i = W_o[U_i * Norm(sum_j A_ij V_j)] + x_i):
        xn = LayerNorm(x) (no affine), uvqk = SiLU(xn W_uvqk^T + b),
        U, V, Q, K = column blocks of uvqk (widths H d_v, H d_v, H d_qk, H d_qk),
        a = attention with the per-(token, head) LayerNorm * U gate,
        y = a W_o^T + x.
    `rows`: optional token indices; only those rows of y are meaningful."""
    L = inp.layer
    f64 = np.float64
    x = L["x"].astype(f64)
    N, D = x.shape
    H, dqk, dv = inp.num_heads, inp.d_qk, inp.d_v
    eps = float(np.float32(inp.eps))
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    xn = (x - mu) / np.sqrt(var + eps)
    z = xn @ L["w_uvqk"].astype(f64).T + L["b_uvqk"].astype(f64)
    with np.errstate(over="ignore"):
        uvqk = z / (1.0 + np.exp(-z))
    c0, c1, c2 = H * dv, 2 * H * dv, 2 * H * dv + H * dqk
    U = uvqk[:, :c0].reshape(N, H, dv)
    V = uvqk[:, c0:c1].reshape(N, H, dv)
    Q = uvqk[:, c1:c2].reshape(N, H, dqk)
    K = uvqk[:, c2:].reshape(N, H, dqk)
    a = forward_arrays(inp.offsets, Q, K, V, U, timestamps=inp.timestamps,
                       num_targets=inp.num_targets, contextual_len=inp.contextual_len,
                       max_attn_len=inp.max_attn_len, alpha=inp.alpha, n_scale=inp.n_scale,
                       pos_table=inp.pos_table, time_table=inp.time_table, eps=inp.eps,
                       epilogue=EPILOGUE_LN_U, rows=rows, nthreads=nthreads)
    a = a.reshape(N, H * dv)
    if rows is not None:
        y = np.full((N, D), np.nan)
        r = np.asarray(rows, dtype=np.int64)
        y[r] = a[r] @ L["w_o"].astype(f64).T + x[r]
        return y
    return a @ L["w_o"].astype(f64).T + x


def backward_arrays(offsets, q, k, v, u, dout, *, timestamps=None, num_targets=None,
                    contextual_len=0, max_attn_len=0, alpha=1.0, n_scale=1.0,
                    pos_table=None, time_table=None, eps=1e-5, epilogue=EPILOGUE_LN_U,
                    nthreads: Optional[int] = None, pos_clamp=False) -> dict:
    """fp64 gradients of sum(dout * forward(...)) with respect to q, k, v, u,
    pos_table and time_table (the C oracle's chain rule; [N, H, d] arrays;
    `pos_clamp` as for `forward`).  Returns a dict with keys dq, dk, dv, du,
    dpos (or None), dtime (or None)."""
    lib = _load()
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    dout = np.ascontiguousarray(dout, dtype=np.float64)
    N, H, dqk = q.shape
    dv = v.shape[2]
    assert dout.shape == (N, H, dv)
    ts = None if timestamps is None else np.ascontiguousarray(timestamps, dtype=np.int64)
    nt = None if num_targets is None else np.ascontiguousarray(num_targets, dtype=np.int32)
    pos = None if pos_table is None else np.ascontiguousarray(pos_table, dtype=np.float64)
    tim = None if time_table is None else np.ascontiguousarray(time_table, dtype=np.float64)
    g = {"dq": np.empty_like(q), "dk": np.empty_like(k), "dv": np.empty_like(v),
         "du": np.empty_like(u),
         "dpos": None if pos is None else np.empty_like(pos),
         "dtime": None if tim is None else np.empty_like(tim)}
    rc = lib.hstu_oracle_bwd(
        offsets.shape[0] - 1, _ptr(offsets), H, dqk, dv,
        _ptr(q), H * dqk, _ptr(k), H * dqk, _ptr(v), H * dv, _ptr(u), H * dv,
        _ptr(ts), _ptr(nt), int(contextual_len), int(max_attn_len),
        float(alpha), float(n_scale),
        _ptr(pos), 0 if pos is None else pos.shape[0],
        _ptr(tim), 0 if tim is None else tim.shape[0],
        float(np.float32(eps)), int(epilogue), _ptr(dout), H * dv,
        _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["du"]),
        _ptr(g["dpos"]), _ptr(g["dtime"]),
        int(nthreads if nthreads is not None else default_threads()), int(bool(pos_clamp)))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return g


def backward(inp, dout, *, epilogue=EPILOGUE_LN_U, nthreads: Optional[int] = None,
             pos_clamp=False) -> dict:
    """fp64 gradients for a `JaggedInputs` batch and output gradient `dout`."""
    return backward_arrays(
        inp.offsets, inp.q, inp.k, inp.v, inp.u, dout, timestamps=inp.timestamps,
        num_targets=inp.num_targets, contextual_len=inp.contextual_len,
        max_attn_len=inp.max_attn_len, alpha=inp.alpha, n_scale=inp.n_scale,
        pos_table=inp.pos_table, time_table=inp.time_table, eps=inp.eps,
        epilogue=epilogue, nthreads=nthreads, pos_clamp=pos_clamp)


def count_allowed(offsets, num_targets=None, contextual_len=0, max_attn_len=0) -> int:
    lib = _load()
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    nt = None if num_targets is None else np.ascontiguousarray(num_targets, dtype=np.int32)
    return int(lib.hstu_oracle_count_allowed(offsets.shape[0] - 1, _ptr(offsets), _ptr(nt),
                                             int(contextual_len), int(max_attn_len)))


def time_bucket(t_i: int, t_j: int) -> int:
    return int(_load().hstu_oracle_time_bucket(int(t_i), int(t_j)))


def silu(x: float) -> float:
    return float(_load().hstu_oracle_silu(float(x)))


def allowed(L, num_targets, contextual_len, max_attn_len, i, j) -> bool:
    return bool(_load().hstu_oracle_allowed(L, num_targets, contextual_len, max_attn_len, i, j))


def max_threads() -> int:
    return int(_load().hstu_oracle_max_threads())


# --------------------------------------------------------------------------
# Dense padded brute force (tiny inputs only).
# --------------------------------------------------------------------------

def _dense_mask(L: int, T: int, c: int, W: int, Lpad: int) -> np.ndarray:
    """[Lpad, Lpad] boolean matrix of allowed pairs, built from whole-matrix
    boolean algebra (rows = queries, cols = keys)."""
    n_h = L - min(max(T, 0), L)
    c = min(max(c, 0), n_h)
    i = np.arange(Lpad)[:, None]
    j = np.arange(Lpad)[None, :]
    valid = (i < L) & (j < L)
    tril = j <= i
    prefix_block = (i < c) & (j < c)
    history_rows = (i >= c) & (i < n_h)
    cand_rows = i >= n_h
    cand_ok = (j < n_h) | (j == i)
    m = prefix_block | (history_rows & tril) | (cand_rows & cand_ok)
    if W > 0:
        p = np.minimum(i, n_h)
        m = m & ((p - j) <= W)
    return m & valid


def dense_forward(inp, *, epilogue=EPILOGUE_LN_U, pos_clamp=False) -> np.ndarray:
    """Padded dense evaluation: SiLU on every padded entry, then zero the
    illegal ones, then aggregate.  numpy fp64; tiny inputs only.  With
    `pos_clamp` the position-bias matrix of each sequence is built from the
    clamped position vector p = min(arange(L), n_h)."""
    B = inp.num_seqs
    L = inp.lengths
    Lpad = int(L.max()) if B else 0
    H, dqk, dv = inp.num_heads, inp.d_qk, inp.d_v
    out = np.zeros((inp.total_tokens, H, dv), dtype=np.float64)
    if Lpad == 0:
        return out
    f64 = np.float64
    Qp = np.zeros((B, H, Lpad, dqk), f64)
    Kp = np.zeros((B, H, Lpad, dqk), f64)
    Vp = np.zeros((B, H, Lpad, dv), f64)
    Up = np.zeros((B, H, Lpad, dv), f64)
    Tp = np.zeros((B, Lpad), np.int64)
    for b in range(B):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        Qp[b, :, : e - s] = inp.q[s:e].astype(f64).transpose(1, 0, 2)
        Kp[b, :, : e - s] = inp.k[s:e].astype(f64).transpose(1, 0, 2)
        Vp[b, :, : e - s] = inp.v[s:e].astype(f64).transpose(1, 0, 2)
        Up[b, :, : e - s] = inp.u[s:e].astype(f64).transpose(1, 0, 2)
        if inp.timestamps is not None:
            Tp[b, : e - s] = inp.timestamps[s:e]
    S = inp.alpha * (Qp @ np.swapaxes(Kp, -1, -2))           # [B,H,Lpad,Lpad]
    ii = np.arange(Lpad)[:, None]
    jj = np.arange(Lpad)[None, :]
    if inp.pos_table is not None:
        P = inp.pos_table.shape[0]
        if pos_clamp:
            for b in range(B):
                T = 0 if inp.num_targets is None else int(inp.num_targets[b])
                n_h = int(L[b]) - min(max(T, 0), int(L[b]))
                p = np.minimum(np.arange(Lpad), n_h)
                rel = np.minimum(np.abs(p[:, None] - p[None, :]), P - 1)
                S[b] = S[b] + inp.pos_table.astype(f64)[rel][None]
        else:
            rel = np.minimum(np.abs(ii - jj), P - 1)
            S = S + inp.pos_table.astype(f64)[rel][None, None]
    if inp.time_table is not None:
        Tt = inp.time_table.shape[0]
        dt = np.abs(Tp[:, :, None] - Tp[:, None, :]).astype(np.uint64)
        # floor(log2(1+dt)) via Python's exact integer bit_length, elementwise
        blen = np.vectorize(lambda x: (int(x) + 1).bit_length() - 1, otypes=[np.int64])(dt)
        S = S + inp.time_table.astype(f64)[np.minimum(blen, Tt - 1)][:, None]
    with np.errstate(over="ignore"):
        A = S / (1.0 + np.exp(-S)) / inp.n_scale
    for b in range(B):
        T = 0 if inp.num_targets is None else int(inp.num_targets[b])
        mask = _dense_mask(int(L[b]), T, inp.contextual_len, inp.max_attn_len, Lpad)
        A[b] = np.where(mask[None], A[b], 0.0)
    O = A @ Vp                                                # [B,H,Lpad,dv]
    if epilogue == EPILOGUE_LN_U:
        mu = O.mean(-1, keepdims=True)
        var = ((O - mu) ** 2).mean(-1, keepdims=True)
        O = (O - mu) / np.sqrt(var + float(np.float32(inp.eps))) * Up
    elif epilogue == EPILOGUE_LN_ALL_U:
        Ot = np.swapaxes(O, 1, 2).reshape(B, Lpad, H * dv)    # a token's heads side by side
        mu = Ot.mean(-1, keepdims=True)
        var = ((Ot - mu) ** 2).mean(-1, keepdims=True)
        Ot = (Ot - mu) / np.sqrt(var + float(np.float32(inp.eps)))
        O = np.swapaxes(Ot.reshape(B, Lpad, H, dv), 1, 2) * Up
    for b in range(B):
        s, e = int(inp.offsets[b]), int(inp.offsets[b + 1])
        out[s:e] = O[b, :, : e - s].transpose(1, 0, 2)
    return out


def timed_forward(inp, *, nthreads: Optional[int] = None):
    """Runs `forward` and returns (output, seconds, threads used)."""
    n = nthreads if nthreads is not None else default_threads()
    t0 = time.perf_counter()
    out = forward(inp, nthreads=n)
    return out, time.perf_counter() - t0, n
