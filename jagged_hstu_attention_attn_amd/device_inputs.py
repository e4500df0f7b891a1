"""Moves a seeded `JaggedInputs` batch onto a GPU as torch tensors.

Marshalling only (numpy -> torch, exact: bf16 workloads already hold
bf16-representable values).  Optional token strides reproduce strided views,
e.g. slices of a fused projection output.
"""
from __future__ import annotations

import numpy as np
import torch

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def _tokens(x: np.ndarray, dtype, device, ld=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device=device, dtype=dtype)
    if ld is None or x.shape[0] == 0:
        return t
    N, H, d = t.shape
    assert ld >= H * d
    buf = torch.zeros((N, ld), dtype=dtype, device=device)
    view = buf.as_strided((N, H, d), (ld, d, 1))
    view.copy_(t)
    return view


def to_device(inp, device="cuda", ld=None) -> dict:
    """Tensors for `jagged_attn_fwd`; `ld` (elements) makes strided views."""
    dt = _TORCH[inp.dtype]
    dev = torch.device(device)
    t = lambda a, d: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, d)
    return dict(
        q=_tokens(inp.q, dt, dev, ld), k=_tokens(inp.k, dt, dev, ld),
        v=_tokens(inp.v, dt, dev, ld), u=_tokens(inp.u, dt, dev, ld),
        offsets=t(inp.offsets, torch.int32),
        timestamps=t(inp.timestamps, torch.int64),
        num_targets=t(inp.num_targets, torch.int32),
        pos_table=t(inp.pos_table, torch.float32),
        time_table=t(inp.time_table, torch.float32),
    )


def call_kwargs(inp, dev: dict) -> dict:
    """Keyword arguments of `jagged_attn_fwd` / `JaggedAttnCall`."""
    return dict(timestamps=dev["timestamps"], num_targets=dev["num_targets"],
                contextual_len=inp.contextual_len, max_attn_len=inp.max_attn_len,
                alpha=inp.alpha, n_scale=inp.n_scale, pos_table=dev["pos_table"],
                time_table=dev["time_table"], eps=inp.eps)
