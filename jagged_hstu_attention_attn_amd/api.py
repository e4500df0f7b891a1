"""Python binding of the jagged HSTU attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libhstu_attn.so.  PyTorch supplies device memory and the current
stream; nothing here computes on tensors.

    out = jagged_attn_fwd(q, k, v, u, offsets, timestamps=ts, num_targets=nt,
                          contextual_len=0, max_attn_len=0, alpha=a, n_scale=n,
                          pos_table=pos, time_table=tim)

q, k: [N, H, d_qk]; v, u: [N, H, d_v]; bf16 or fp32 CUDA (HIP) tensors whose
last two dimensions are contiguous (the token stride may be larger, e.g. views
into a fused projection output).  offsets: int32 [B+1]; timestamps: int64 [N];
num_targets: int32 [B]; tables: float32.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import _lib

__all__ = ["jagged_attn_fwd", "layer_fwd", "HstuLayer", "plan", "run", "make_desc",
           "workspace_bytes", "valid_pairs",
           "JaggedAttnCall"]

_DTYPES = {torch.float32: _lib.HSTU_DTYPE_F32, torch.bfloat16: _lib.HSTU_DTYPE_BF16}
_EPILOGUES = {"ln_u": _lib.HSTU_EPILOGUE_LN_U, "none": _lib.HSTU_EPILOGUE_NONE,
              "ln_all_u": _lib.HSTU_EPILOGUE_LN_ALL_U}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _token_stride(t: torch.Tensor, name: str) -> int:
    if t.dim() != 3:
        raise ValueError(f"{name} must be [tokens, heads, dim], got shape {tuple(t.shape)}")
    if t.numel() == 0:
        return int(t.shape[1] * t.shape[2])
    if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name}: the head and feature dimensions must be contiguous")
    return int(t.stride(0)) if t.shape[0] > 1 else int(t.shape[1] * t.shape[2])


def make_desc(q, k, v, u, out, num_seqs: int, *, pos_table=None, time_table=None,
              eps: float = 1e-5, epilogue: str = "ln_u",
              pos_clamp: bool = False) -> _lib.HstuAttnDesc:
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k", k), ("v", v), ("out", out)) + ((("u", u),) if u is not None else ()):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
    d = _lib.HstuAttnDesc()
    d.num_seqs = int(num_seqs)
    d.total_tokens = int(q.shape[0])
    d.num_heads = int(q.shape[1])
    d.d_qk = int(q.shape[2])
    d.d_v = int(v.shape[2])
    d.dtype = _DTYPES[q.dtype]
    d.ld_q = _token_stride(q, "q")
    d.ld_k = _token_stride(k, "k")
    d.ld_v = _token_stride(v, "v")
    d.ld_u = _token_stride(u, "u") if u is not None else d.num_heads * d.d_v
    d.ld_out = _token_stride(out, "out")
    d.pos_table_len = 0 if pos_table is None else int(pos_table.numel())
    d.time_table_len = 0 if time_table is None else int(time_table.numel())
    d.ln_eps = float(eps)
    d.epilogue = _EPILOGUES[epilogue]
    d.pos_clamp = 1 if pos_clamp else 0
    return d


FWD_KERNELS = {"auto": _lib.HSTU_FWD_KERNEL_AUTO, "four_wave": _lib.HSTU_FWD_KERNEL_FOUR_WAVE,
               "eight_wave": _lib.HSTU_FWD_KERNEL_EIGHT_WAVE,
               "sixteen_row": _lib.HSTU_FWD_KERNEL_SIXTEEN_ROW,
               "thirtytwo_row": _lib.HSTU_FWD_KERNEL_THIRTYTWO_ROW}


def set_fwd_kernel(name: str) -> None:
    """Process-wide forward kernel choice ("auto", "four_wave", "eight_wave",
    "sixteen_row", "thirtytwo_row");
    a plan and the runs that use it must see the same choice."""
    _lib.check(_lib.load().hstu_jagged_attn_set_fwd_kernel(FWD_KERNELS[name]))


def fwd_kernel_of(desc: _lib.HstuAttnDesc) -> str:
    """Which forward kernel the library runs for `desc` under the current choice."""
    r = _lib.load().hstu_jagged_attn_fwd_kernel_of(ctypes.byref(desc))
    if r < 0:
        raise _lib.HstuError(r, _lib.last_error())
    return {v: k for k, v in FWD_KERNELS.items()}[r]


class fwd_kernel:
    """Context manager: run the enclosed calls with one forward kernel."""

    def __init__(self, name: str):
        self.name = name

    def __enter__(self):
        set_fwd_kernel(self.name)
        return self

    def __exit__(self, *exc):
        set_fwd_kernel("auto")
        return False


def workspace_bytes(desc: _lib.HstuAttnDesc) -> int:
    n = _lib.load().hstu_jagged_attn_workspace_bytes(ctypes.byref(desc))
    if n == 0:
        raise _lib.HstuError(_lib.HSTU_ERR_INVALID_ARG, _lib.last_error())
    return int(n)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def plan(desc, offsets, num_targets, contextual_len, max_attn_len, workspace,
         candidates_only: bool = False) -> None:
    """Enqueue the scheduler kernel (writes the work list into `workspace`).
    With `candidates_only`, the work list covers only the candidate rows."""
    fn = (_lib.load().hstu_jagged_attn_plan_candidates if candidates_only
          else _lib.load().hstu_jagged_attn_plan)
    _lib.check(fn(
        ctypes.byref(desc), _ptr(offsets), _ptr(num_targets), int(contextual_len),
        int(max_attn_len), _ptr(workspace), int(workspace.numel()), _stream(workspace.device)))


def _run_like(fn_name, desc, q, k, v, u, offsets, timestamps, num_targets, contextual_len,
              max_attn_len, alpha, n_scale, pos_table, time_table, out, workspace):
    fn = getattr(_lib.load(), fn_name)
    _lib.check(fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(offsets),
                  _ptr(timestamps), _ptr(num_targets), int(contextual_len), int(max_attn_len),
                  float(alpha), float(n_scale), _ptr(pos_table), _ptr(time_table), _ptr(out),
                  _ptr(workspace), int(workspace.numel()), _stream(q.device)))


def run(desc, q, k, v, u, offsets, timestamps, num_targets, contextual_len, max_attn_len,
        alpha, n_scale, pos_table, time_table, out, workspace) -> None:
    """Enqueue the attention kernel on a work list made by `plan`."""
    _run_like("hstu_jagged_attn_run", desc, q, k, v, u, offsets, timestamps, num_targets,
              contextual_len, max_attn_len, alpha, n_scale, pos_table, time_table, out,
              workspace)


def run_timed(desc, q, k, v, u, offsets, timestamps, num_targets, contextual_len,
              max_attn_len, alpha, n_scale, pos_table, time_table, out, workspace,
              start: torch.cuda.Event, stop: torch.cuda.Event) -> None:
    """`run`, with the attention kernel's own start and end times taken into
    two timing events (each must have been recorded once, so that it exists)."""
    _lib.check(_lib.load().hstu_jagged_attn_run_timed(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(offsets),
        _ptr(timestamps), _ptr(num_targets), int(contextual_len), int(max_attn_len),
        float(alpha), float(n_scale), _ptr(pos_table), _ptr(time_table), _ptr(out),
        _ptr(workspace), int(workspace.numel()), _stream(q.device),
        ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)))


def _check_aux(offsets, timestamps, num_targets, pos_table, time_table, device):
    if offsets.dtype != torch.int32 or offsets.dim() != 1 or not offsets.is_contiguous():
        raise TypeError("offsets must be a contiguous int32 vector")
    if timestamps is not None and (timestamps.dtype != torch.int64 or not timestamps.is_contiguous()):
        raise TypeError("timestamps must be a contiguous int64 vector")
    if num_targets is not None and (num_targets.dtype != torch.int32 or not num_targets.is_contiguous()):
        raise TypeError("num_targets must be a contiguous int32 vector")
    for name, t in (("pos_table", pos_table), ("time_table", time_table)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous float32 vector")
    for t in (offsets, timestamps, num_targets, pos_table, time_table):
        if t is not None and t.device != device:
            raise ValueError("all tensors must live on the same GPU")


class JaggedAttnCall:
    """A reusable call: owns its descriptor and workspace, so the work list
    built by `plan()` can serve several `run()` calls on the same batch."""

    def __init__(self, q, k, v, u, offsets, *, timestamps=None, num_targets=None,
                 contextual_len=0, max_attn_len=0, alpha, n_scale, pos_table=None,
                 time_table=None, eps=1e-5, epilogue="ln_u", out=None,
                 candidates_only: bool = False, pos_clamp: bool = False,
                 save_o: bool = False, workspace: Optional[torch.Tensor] = None):
        if not q.is_cuda:
            raise ValueError("tensors must be on a GPU")
        _check_aux(offsets, timestamps, num_targets, pos_table, time_table, q.device)
        self.q, self.k, self.v, self.u = q, k, v, u
        self.offsets, self.timestamps, self.num_targets = offsets, timestamps, num_targets
        self.contextual_len, self.max_attn_len = int(contextual_len), int(max_attn_len)
        self.alpha, self.n_scale = float(alpha), float(n_scale)
        self.pos_table, self.time_table = pos_table, time_table
        self.candidates_only = bool(candidates_only)
        if out is None:
            out = torch.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=q.dtype,
                              device=q.device)
        self.out = out
        self.desc = make_desc(q, k, v, u, out, offsets.numel() - 1, pos_table=pos_table,
                              time_table=time_table, eps=eps, epilogue=epilogue,
                              pos_clamp=pos_clamp)
        need = workspace_bytes(self.desc)
        if workspace is not None and (workspace.dtype != torch.uint8 or workspace.numel() < need
                                      or workspace.device != q.device):
            raise ValueError(f"workspace must be a uint8 tensor of >= {need} bytes on {q.device}")
        self.workspace = (workspace[:need] if workspace is not None else
                          torch.empty(need, dtype=torch.uint8, device=q.device))
        # save_o: the call also keeps o / n_scale before the gate (training)
        self.o_raw = (torch.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=q.dtype,
                                  device=q.device) if save_o else None)
        if save_o and candidates_only:
            raise ValueError("save_o is for full forwards")

    def kernel_name(self) -> str:
        """The forward kernel this call runs under the current choice."""
        return fwd_kernel_of(self.desc)

    def plan(self) -> None:
        plan(self.desc, self.offsets, self.num_targets, self.contextual_len, self.max_attn_len,
             self.workspace, self.candidates_only)

    def run(self) -> torch.Tensor:
        run(self.desc, self.q, self.k, self.v, self.u, self.offsets, self.timestamps,
            self.num_targets, self.contextual_len, self.max_attn_len, self.alpha, self.n_scale,
            self.pos_table, self.time_table, self.out, self.workspace)
        return self.out

    def run_timed(self, start: torch.cuda.Event, stop: torch.cuda.Event) -> torch.Tensor:
        run_timed(self.desc, self.q, self.k, self.v, self.u, self.offsets, self.timestamps,
                  self.num_targets, self.contextual_len, self.max_attn_len, self.alpha,
                  self.n_scale, self.pos_table, self.time_table, self.out, self.workspace,
                  start, stop)
        return self.out

    def __call__(self) -> torch.Tensor:
        if self.o_raw is not None:
            _lib.check(_lib.load().hstu_jagged_attn_fwd_train(
                ctypes.byref(self.desc), _ptr(self.q), _ptr(self.k), _ptr(self.v),
                _ptr(self.u), _ptr(self.offsets), _ptr(self.timestamps), _ptr(self.num_targets),
                self.contextual_len, self.max_attn_len, self.alpha, self.n_scale,
                _ptr(self.pos_table), _ptr(self.time_table), _ptr(self.out), _ptr(self.o_raw),
                _ptr(self.workspace), int(self.workspace.numel()), _stream(self.q.device)))
            return self.out
        _run_like("hstu_jagged_attn_fwd_candidates" if self.candidates_only
                  else "hstu_jagged_attn_fwd", self.desc, self.q, self.k, self.v, self.u,
                  self.offsets, self.timestamps, self.num_targets, self.contextual_len,
                  self.max_attn_len, self.alpha, self.n_scale, self.pos_table, self.time_table,
                  self.out, self.workspace)
        return self.out


# One-shot calls reuse one workspace per (device, stream): work on a stream
# runs in order, so a call's scratch is free again for the next call on that
# stream.  The cache keeps the largest size asked for (until the process ends).
_ws_cache: dict = {}


def _stream_workspace(device, nbytes: int) -> torch.Tensor:
    key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def jagged_attn_fwd(q, k, v, u, offsets, *, timestamps=None, num_targets=None,
                    contextual_len: int = 0, max_attn_len: int = 0, alpha: float,
                    n_scale: float, pos_table=None, time_table=None, eps: float = 1e-5,
                    epilogue: str = "ln_u", out=None,
                    candidates_only: bool = False, pos_clamp: bool = False) -> torch.Tensor:
    """One full forward (scheduler + attention) on the current stream.  With
    `candidates_only`, only the candidate rows of `out` are computed and
    written (history rows keep their contents).  The scheduler's workspace
    is reused across calls on the same device and stream."""
    if not q.is_cuda:
        raise ValueError("tensors must be on a GPU")
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=q.dtype, device=q.device)
    desc = make_desc(q, k, v, u, out, offsets.numel() - 1, pos_table=pos_table,
                     time_table=time_table, eps=eps, epilogue=epilogue, pos_clamp=pos_clamp)
    ws = _stream_workspace(q.device, workspace_bytes(desc))
    call = JaggedAttnCall(q, k, v, u, offsets, timestamps=timestamps, num_targets=num_targets,
                          contextual_len=contextual_len, max_attn_len=max_attn_len,
                          alpha=alpha, n_scale=n_scale, pos_table=pos_table,
                          time_table=time_table, eps=eps, epilogue=epilogue, out=out,
                          candidates_only=candidates_only, pos_clamp=pos_clamp, workspace=ws)
    return call()


class JaggedAttnBwdCall:
    """A reusable backward call (owns its descriptor, workspace and gradient
    buffers).  `__call__(dout)` enqueues the whole backward on the current
    stream and returns (dq, dk, dv, du, dpos, dtime); du is None for epilogue
    "none", dpos / dtime are None when the table is."""

    def __init__(self, q, k, v, u, offsets, *, timestamps=None, num_targets=None,
                 contextual_len=0, max_attn_len=0, alpha, n_scale, pos_table=None,
                 time_table=None, eps=1e-5, epilogue="ln_u", pos_clamp: bool = False):
        if not q.is_cuda:
            raise ValueError("tensors must be on a GPU")
        _check_aux(offsets, timestamps, num_targets, pos_table, time_table, q.device)
        self.q, self.k, self.v, self.u = q, k, v, u
        self.offsets, self.timestamps, self.num_targets = offsets, timestamps, num_targets
        self.contextual_len, self.max_attn_len = int(contextual_len), int(max_attn_len)
        self.alpha, self.n_scale = float(alpha), float(n_scale)
        self.pos_table, self.time_table = pos_table, time_table
        self.epilogue = epilogue
        shape_o = (q.shape[0], q.shape[1], v.shape[2])
        out_like = torch.empty(shape_o, dtype=q.dtype, device=q.device)
        self.desc = make_desc(q, k, v, u, out_like, offsets.numel() - 1, pos_table=pos_table,
                              time_table=time_table, eps=eps, epilogue=epilogue,
                              pos_clamp=pos_clamp)
        n = _lib.load().hstu_jagged_attn_bwd_workspace_bytes(ctypes.byref(self.desc))
        if n == 0:
            raise _lib.HstuError(_lib.HSTU_ERR_INVALID_ARG, _lib.last_error())
        self.workspace = torch.empty(int(n), dtype=torch.uint8, device=q.device)
        # gradients share the layouts of their inputs (token strides included)
        self.dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
        self.dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
        self.dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device)
        self.du = (None if epilogue == "none" else
                   torch.empty_strided(u.shape, u.stride(), dtype=u.dtype, device=u.device))
        self.dpos = None if pos_table is None else torch.empty_like(pos_table)
        self.dtime = None if time_table is None else torch.empty_like(time_table)

    def __call__(self, dout, o_saved=None):
        """o_saved: the raw aggregation a training forward kept (see
        JaggedAttnCall(save_o=True)), or None to recompute it."""
        if o_saved is not None and (o_saved.shape != dout.shape or o_saved.dtype != dout.dtype
                                    or not o_saved.is_contiguous()):
            raise ValueError("o_saved must be a contiguous tensor shaped and typed like dout")
        if dout.shape != (self.q.shape[0], self.q.shape[1], self.v.shape[2]):
            raise ValueError(f"dout has shape {tuple(dout.shape)}")
        if dout.dtype != self.q.dtype:
            raise TypeError(f"dout has dtype {dout.dtype}, q has {self.q.dtype}")
        if _token_stride(dout, "dout") != self.desc.ld_out:
            raise ValueError("dout must be contiguous in its token dimension")
        _lib.check(_lib.load().hstu_jagged_attn_bwd(
            ctypes.byref(self.desc), _ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.u),
            _ptr(self.offsets), _ptr(self.timestamps), _ptr(self.num_targets),
            self.contextual_len, self.max_attn_len, self.alpha, self.n_scale,
            _ptr(self.pos_table), _ptr(self.time_table), _ptr(dout), _ptr(o_saved), _ptr(self.dq),
            _ptr(self.dk), _ptr(self.dv), _ptr(self.du), _ptr(self.dpos), _ptr(self.dtime),
            _ptr(self.workspace), int(self.workspace.numel()), _stream(self.q.device)))
        return self.dq, self.dk, self.dv, self.du, self.dpos, self.dtime


def jagged_attn_bwd(q, k, v, u, offsets, dout, *, timestamps=None, num_targets=None,
                    contextual_len: int = 0, max_attn_len: int = 0, alpha: float,
                    n_scale: float, pos_table=None, time_table=None, eps: float = 1e-5,
                    epilogue: str = "ln_u", o_saved=None, pos_clamp: bool = False):
    """Gradients (dq, dk, dv, du, dpos, dtime) of sum(dout * forward(...)),
    computed on the GPU on the current stream (o_saved: see
    JaggedAttnBwdCall.__call__; pos_clamp: the position bias at clamped
    positions, as for the forward)."""
    call = JaggedAttnBwdCall(q, k, v, u, offsets, timestamps=timestamps,
                             num_targets=num_targets, contextual_len=contextual_len,
                             max_attn_len=max_attn_len, alpha=alpha, n_scale=n_scale,
                             pos_table=pos_table, time_table=time_table, eps=eps,
                             epilogue=epilogue, pos_clamp=pos_clamp)
    return call(dout, o_saved)


def valid_pairs(offsets, num_targets=None, contextual_len: int = 0, max_attn_len: int = 0) -> int:
    """Exact allowed-pair count per head, from host copies of the metadata."""
    off = np.ascontiguousarray(np.asarray(offsets), dtype=np.int32)
    nt = None if num_targets is None else np.ascontiguousarray(np.asarray(num_targets),
                                                                dtype=np.int32)
    n = _lib.load().hstu_jagged_attn_valid_pairs(
        off.shape[0] - 1, off.ctypes.data_as(ctypes.c_void_p),
        None if nt is None else nt.ctypes.data_as(ctypes.c_void_p),
        int(contextual_len), int(max_attn_len))
    if n < 0:
        raise _lib.HstuError(_lib.HSTU_ERR_INVALID_ARG, _lib.last_error())
    return int(n)


class HstuLayer:
    """The full layer forward on one batch: owns its descriptor, workspace and
    output; x [N, hidden], w_uvqk [H (2 d_v + 2 d_qk), hidden], b_uvqk [..],
    w_o [hidden, H d_v], all bf16 on one GPU."""

    def __init__(self, x, w_uvqk, b_uvqk, w_o, offsets, *, num_heads, d_qk, d_v,
                 timestamps=None, num_targets=None, contextual_len=0, max_attn_len=0, alpha,
                 n_scale, pos_table=None, time_table=None, eps=1e-5):
        if not x.is_cuda:
            raise ValueError("tensors must be on a GPU")
        for name, t in (("x", x), ("w_uvqk", w_uvqk), ("b_uvqk", b_uvqk), ("w_o", w_o)):
            if t.dtype != torch.bfloat16 or not t.is_contiguous():
                raise TypeError(f"{name} must be a contiguous bfloat16 tensor")
        _check_aux(offsets, timestamps, num_targets, pos_table, time_table, x.device)
        self.args = (x, w_uvqk, b_uvqk, w_o, offsets, timestamps, num_targets)
        self.contextual_len, self.max_attn_len = int(contextual_len), int(max_attn_len)
        self.alpha, self.n_scale = float(alpha), float(n_scale)
        self.pos_table, self.time_table = pos_table, time_table
        d = _lib.HstuLayerDesc()
        d.num_seqs = offsets.numel() - 1
        d.total_tokens = x.shape[0]
        d.num_heads, d.d_qk, d.d_v, d.hidden = int(num_heads), int(d_qk), int(d_v), x.shape[1]
        d.pos_table_len = 0 if pos_table is None else pos_table.numel()
        d.time_table_len = 0 if time_table is None else time_table.numel()
        d.ln_eps = float(eps)
        self.desc = d
        n = _lib.load().hstu_layer_workspace_bytes(ctypes.byref(d))
        if n == 0:
            raise _lib.HstuError(_lib.HSTU_ERR_INVALID_ARG, _lib.last_error())
        self.workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
        self.y = torch.empty_like(x)

    def __call__(self) -> torch.Tensor:
        x, w_uvqk, b_uvqk, w_o, offsets, timestamps, num_targets = self.args
        _lib.check(_lib.load().hstu_layer_fwd(
            ctypes.byref(self.desc), _ptr(x), _ptr(w_uvqk), _ptr(b_uvqk), _ptr(w_o),
            _ptr(offsets), _ptr(timestamps), _ptr(num_targets), self.contextual_len,
            self.max_attn_len, self.alpha, self.n_scale, _ptr(self.pos_table),
            _ptr(self.time_table), _ptr(self.y), _ptr(self.workspace),
            int(self.workspace.numel()), _stream(x.device)))
        return self.y


def layer_fwd(x, w_uvqk, b_uvqk, w_o, offsets, **kw) -> torch.Tensor:
    """One full layer forward on the current stream (see HstuLayer)."""
    return HstuLayer(x, w_uvqk, b_uvqk, w_o, offsets, **kw)()
