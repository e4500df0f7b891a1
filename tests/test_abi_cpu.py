"""The C ABI on the host: symbols, argument validation, host helpers.

No compute call runs here (no GPU): every call below either fails validation
before any HIP call, or is expected to report HSTU_ERR_HIP.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from jagged_hstu_attention_attn_amd import _lib
from jagged_hstu_attention_attn_amd.inputs import make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from jagged_hstu_attention_attn_amd import build
        build.build(quiet=True)
    return _lib.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "hstu_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hstu_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)


def test_no_oracle_linkage():
    out = subprocess.run(["ldd", _lib.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out
    out = subprocess.run(["nm", "-D", _lib.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out


def _desc(**kw):
    d = _lib.HstuAttnDesc()
    base = dict(num_seqs=2, total_tokens=100, num_heads=4, d_qk=128, d_v=128,
                dtype=_lib.HSTU_DTYPE_BF16, ld_q=512, ld_k=512, ld_v=512, ld_u=512, ld_out=512,
                pos_table_len=0, time_table_len=0, ln_eps=1e-5, epilogue=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


FAKE = 0x10000  # aligned, never dereferenced by the host


def _fwd(lib, d, ws_bytes=None, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, offsets=FAKE, timestamps=None, num_targets=None,
                contextual_len=0, max_attn_len=0, alpha=0.1, n_scale=10.0, pos_table=None,
                time_table=None, out=FAKE, ws=FAKE)
    args.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.hstu_jagged_attn_workspace_bytes(ctypes.byref(d)) or 1 << 20
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.hstu_jagged_attn_fwd(
        ctypes.byref(d), vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["u"]),
        vp(args["offsets"]), vp(args["timestamps"]), vp(args["num_targets"]),
        args["contextual_len"], args["max_attn_len"], args["alpha"], args["n_scale"],
        vp(args["pos_table"]), vp(args["time_table"]), vp(args["out"]), vp(args["ws"]),
        ws_bytes, None)


@pytest.mark.parametrize("field,value,code", [
    ("num_seqs", -1, _lib.HSTU_ERR_INVALID_ARG),
    ("total_tokens", -5, _lib.HSTU_ERR_INVALID_ARG),
    ("num_heads", 0, _lib.HSTU_ERR_INVALID_ARG),
    ("dtype", 7, _lib.HSTU_ERR_INVALID_ARG),
    ("epilogue", 3, _lib.HSTU_ERR_INVALID_ARG),
    ("d_qk", 96, _lib.HSTU_ERR_UNSUPPORTED),
    ("d_v", 0, _lib.HSTU_ERR_INVALID_ARG),
    ("ld_q", 500, _lib.HSTU_ERR_INVALID_ARG),
    ("ld_k", 516, _lib.HSTU_ERR_INVALID_ARG),          # 1032 bytes: not a multiple of 16
    ("ln_eps", 0.0, _lib.HSTU_ERR_INVALID_ARG),
    ("pos_table_len", 9000, _lib.HSTU_ERR_UNSUPPORTED),
    ("pos_clamp", 2, _lib.HSTU_ERR_INVALID_ARG),
    ("ld_v", (1 << 23) + 8, _lib.HSTU_ERR_UNSUPPORTED),  # a bf16 token row past 16 MiB
    ("ld_out", 1 << 24, _lib.HSTU_ERR_UNSUPPORTED),
])
def test_bad_descriptor(lib, field, value, code):
    d = _desc(**{field: value})
    assert _fwd(lib, d, ws_bytes=1 << 20) == code
    assert _lib.last_error() != ""
    if code == _lib.HSTU_ERR_INVALID_ARG or code == _lib.HSTU_ERR_UNSUPPORTED:
        assert lib.hstu_jagged_attn_workspace_bytes(ctypes.byref(d)) == 0


def test_token_row_of_16_mib_is_accepted(lib):
    """Kernels form a tile copy's offset as a 32-bit row * stride (rows below
    256): a token row of exactly 2^24 bytes is the largest the descriptor
    takes."""
    d = _desc(ld_q=1 << 23, ld_k=1 << 23, ld_v=1 << 23, ld_u=1 << 23, ld_out=1 << 23)
    assert lib.hstu_jagged_attn_workspace_bytes(ctypes.byref(d)) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.HSTU_ERR_INVALID_ARG),
    (dict(out=None), _lib.HSTU_ERR_INVALID_ARG),
    (dict(offsets=None), _lib.HSTU_ERR_INVALID_ARG),
    (dict(v=FAKE + 8), _lib.HSTU_ERR_INVALID_ARG),       # misaligned
    (dict(n_scale=0.0), _lib.HSTU_ERR_INVALID_ARG),
    (dict(n_scale=float("inf")), _lib.HSTU_ERR_INVALID_ARG),
    (dict(alpha=float("nan")), _lib.HSTU_ERR_INVALID_ARG),
    (dict(contextual_len=-1), _lib.HSTU_ERR_INVALID_ARG),
    (dict(max_attn_len=-2), _lib.HSTU_ERR_INVALID_ARG),
    (dict(pos_table=FAKE), _lib.HSTU_ERR_INVALID_ARG),   # pointer without a length
    (dict(ws=None), _lib.HSTU_ERR_WORKSPACE),
])
def test_bad_arguments(lib, kw, code):
    assert _fwd(lib, _desc(), **kw) == code
    assert _lib.last_error() != ""


def _run(lib, d, fn="hstu_jagged_attn_run", ws_bytes=None, **kw):
    """hstu_jagged_attn_run, or the timed run (with two NULL events)."""
    args = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, offsets=FAKE, timestamps=None, num_targets=None,
                contextual_len=0, max_attn_len=0, alpha=0.1, n_scale=10.0, pos_table=None,
                time_table=None, out=FAKE, ws=FAKE)
    args.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.hstu_jagged_attn_workspace_bytes(ctypes.byref(d)) or 1 << 20
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    call = [ctypes.byref(d), vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["u"]),
            vp(args["offsets"]), vp(args["timestamps"]), vp(args["num_targets"]),
            args["contextual_len"], args["max_attn_len"], args["alpha"], args["n_scale"],
            vp(args["pos_table"]), vp(args["time_table"]), vp(args["out"]), vp(args["ws"]),
            ws_bytes, None]
    if fn == "hstu_jagged_attn_run_timed":
        call += [None, None]
    return getattr(lib, fn)(*call)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.HSTU_ERR_INVALID_ARG),
    (dict(v=FAKE + 8), _lib.HSTU_ERR_INVALID_ARG),
    (dict(n_scale=0.0), _lib.HSTU_ERR_INVALID_ARG),
    (dict(ws=None), _lib.HSTU_ERR_WORKSPACE),
])
def test_timed_run_validates_like_run(lib, kw, code):
    """The timed run is the run with two events: it rejects the same calls
    with the same status, before touching the device."""
    assert _run(lib, _desc(), **kw) == code
    assert _run(lib, _desc(), fn="hstu_jagged_attn_run_timed", **kw) == code
    assert _run(lib, _desc(ln_eps=0.0), fn="hstu_jagged_attn_run_timed") == \
        _lib.HSTU_ERR_INVALID_ARG
    assert _run(lib, _desc(num_seqs=0, total_tokens=0), fn="hstu_jagged_attn_run_timed",
                q=None, k=None, v=None, u=None, out=None, offsets=None) == _lib.HSTU_OK


def test_time_table_needs_timestamps(lib):
    d = _desc(time_table_len=64)
    assert _fwd(lib, d, time_table=FAKE) == _lib.HSTU_ERR_INVALID_ARG
    assert "timestamps" in _lib.last_error()


def test_small_workspace(lib):
    d = _desc()
    need = lib.hstu_jagged_attn_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert _fwd(lib, d, ws_bytes=need - 1) == _lib.HSTU_ERR_WORKSPACE


def test_empty_batch_is_a_no_op(lib):
    assert _fwd(lib, _desc(num_seqs=0, total_tokens=0), q=None, k=None, v=None, u=None,
                out=None, offsets=None) == _lib.HSTU_OK
    assert _fwd(lib, _desc(num_seqs=3, total_tokens=0)) == _lib.HSTU_OK


def test_epilogue_none_does_not_need_u(lib):
    rc = _fwd(lib, _desc(epilogue=_lib.HSTU_EPILOGUE_NONE, ld_u=0), u=None)
    assert rc in (_lib.HSTU_OK, _lib.HSTU_ERR_HIP)   # passes validation


def test_fwd_train_needs_o_raw(lib):
    d = _desc()
    ws = lib.hstu_jagged_attn_workspace_bytes(ctypes.byref(d))
    vp = ctypes.c_void_p
    args = [ctypes.byref(d), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, None, 0, 0,
            0.1, 10.0, None, None, vp(FAKE)]
    assert lib.hstu_jagged_attn_fwd_train(*args, None, vp(FAKE), ws, None) == \
        _lib.HSTU_ERR_INVALID_ARG
    assert "o_raw" in _lib.last_error()
    assert lib.hstu_jagged_attn_fwd_train(*args, vp(FAKE + 4), vp(FAKE), ws, None) == \
        _lib.HSTU_ERR_INVALID_ARG


def test_valid_call_without_gpu_reports_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc = _fwd(lib, _desc())
    assert rc == _lib.HSTU_ERR_HIP
    assert _lib.last_error() != ""


def test_supported_set(lib):
    assert lib.hstu_jagged_attn_supported(1, 128, 128) == 1
    assert lib.hstu_jagged_attn_supported(1, 64, 128) == 1
    assert lib.hstu_jagged_attn_supported(1, 128, 64) == 1
    assert lib.hstu_jagged_attn_supported(1, 256, 256) == 1
    assert lib.hstu_jagged_attn_supported(1, 256, 128) == 0
    assert lib.hstu_jagged_attn_supported(0, 256, 256) == 0
    assert lib.hstu_jagged_attn_supported(0, 8, 8) == 1
    assert lib.hstu_jagged_attn_supported(1, 8, 8) == 0
    assert lib.hstu_jagged_attn_supported(0, 64, 128) == 0
    assert lib.hstu_jagged_attn_supported(2, 128, 128) == 0


def _bwd(lib, d, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, offsets=FAKE, dout=FAKE, o_saved=None, dq=FAKE,
                dk=FAKE, dv=FAKE, du=FAKE, ws=FAKE)
    args.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    ws_bytes = lib.hstu_jagged_attn_bwd_workspace_bytes(ctypes.byref(d)) or 1 << 20
    return lib.hstu_jagged_attn_bwd(
        ctypes.byref(d), vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["u"]),
        vp(args["offsets"]), None, None, 0, 0, 0.1, 10.0, None, None, vp(args["dout"]),
        vp(args["o_saved"]),
        vp(args["dq"]), vp(args["dk"]), vp(args["dv"]), vp(args["du"]), None, None,
        vp(args["ws"]), ws_bytes, None)


def test_backward_validation(lib):
    # unequal bf16 head dims pass the checks (and then need a GPU)
    d = _desc(d_qk=64, d_v=128, ld_q=256, ld_k=256)
    assert lib.hstu_jagged_attn_workspace_bytes(ctypes.byref(d)) > 0
    assert _bwd(lib, d) in (_lib.HSTU_OK, _lib.HSTU_ERR_HIP)
    assert _bwd(lib, _desc(), dq=None) == _lib.HSTU_ERR_INVALID_ARG
    assert _bwd(lib, _desc(), du=None) == _lib.HSTU_ERR_INVALID_ARG
    assert _bwd(lib, _desc(), ws=None) == _lib.HSTU_ERR_WORKSPACE
    # the clamped-position bias passes the checks (and then needs a GPU)
    assert _bwd(lib, _desc(pos_clamp=1)) in (_lib.HSTU_OK, _lib.HSTU_ERR_HIP)
    assert _bwd(lib, _desc(pos_clamp=2)) == _lib.HSTU_ERR_INVALID_ARG
    # bf16 d = 256 (per-token kernels) passes the shape check (and then needs a GPU);
    # unequal sizes with a 256-wide side are refused before any HIP call
    d256 = _desc(d_qk=256, d_v=256, ld_q=1024, ld_k=1024, ld_v=1024, ld_u=1024, ld_out=1024)
    assert lib.hstu_jagged_attn_workspace_bytes(ctypes.byref(d256)) > 0
    assert lib.hstu_jagged_attn_bwd_workspace_bytes(ctypes.byref(d256)) > 0
    assert _bwd(lib, d256) in (_lib.HSTU_OK, _lib.HSTU_ERR_HIP)
    d256x = _desc(d_qk=256, d_v=128, ld_q=1024, ld_k=1024)
    assert _bwd(lib, d256x) == _lib.HSTU_ERR_UNSUPPORTED
    assert "d_qk=256, d_v=128" in _lib.last_error()
    # fp32 d = 8 is built: it passes the shape check (and then needs a GPU)
    d8 = _desc(d_qk=8, d_v=8, dtype=_lib.HSTU_DTYPE_F32, ld_q=32, ld_k=32, ld_v=32, ld_u=32,
               ld_out=32)
    assert _bwd(lib, d8) in (_lib.HSTU_OK, _lib.HSTU_ERR_HIP)
    # du is not needed without the gate
    rc = _bwd(lib, _desc(epilogue=_lib.HSTU_EPILOGUE_NONE), du=None)
    assert rc in (_lib.HSTU_OK, _lib.HSTU_ERR_HIP)
    # a table gradient pointer must come with its table
    d = _desc(pos_table_len=16)
    assert lib.hstu_jagged_attn_bwd(
        ctypes.byref(d), *[ctypes.c_void_p(FAKE)] * 5, None, None, 0, 0, 0.1, 10.0,
        ctypes.c_void_p(FAKE), None, ctypes.c_void_p(FAKE), None,
        *[ctypes.c_void_p(FAKE)] * 4, None, None,
        ctypes.c_void_p(FAKE), 1 << 30, None) == _lib.HSTU_ERR_INVALID_ARG
    # o_saved must be aligned
    assert _bwd(lib, _desc(), o_saved=FAKE + 8) == _lib.HSTU_ERR_INVALID_ARG


# The product's host pair count (used for throughput accounting) against the
# oracle's one-pair-at-a-time count.
@pytest.mark.parametrize("name", ["tiny", "ranking", "longtail"])
def test_valid_pairs_matches_oracle(oracle_mod, name):
    from jagged_hstu_attention_attn_amd.api import valid_pairs
    inp = make_inputs(name, num_seqs=12)
    a = valid_pairs(inp.offsets, inp.num_targets, inp.contextual_len, inp.max_attn_len)
    b = oracle_mod.count_allowed(inp.offsets, inp.num_targets, inp.contextual_len,
                                 inp.max_attn_len)
    assert a == b


@pytest.mark.parametrize("seed", range(20))
def test_valid_pairs_random_rules(oracle_mod, seed):
    from jagged_hstu_attention_attn_amd.api import valid_pairs
    rng = np.random.default_rng(seed)
    L = rng.integers(0, 300, size=6)
    off = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    nt = rng.integers(-3, 60, size=6).astype(np.int32)
    c, W = int(rng.integers(0, 40)), int(rng.integers(0, 80))
    assert valid_pairs(off, nt, c, W) == oracle_mod.count_allowed(off, nt, c, W)
    assert valid_pairs(off, None, c, 0) == oracle_mod.count_allowed(off, None, c, 0)


def test_tiny_workload_pair_count():
    from jagged_hstu_attention_attn_amd.api import valid_pairs
    assert valid_pairs([0, 10, 110, 1110]) == 505605


def test_loader_fails_loudly_without_library(tmp_path, monkeypatch):
    import importlib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


def test_forward_kernel_choice(lib):
    """AUTO takes the sixteen-row kernel for bf16 with d = 128 and the
    four-wave kernel elsewhere; the setter forces a kernel where it is
    supported (a host decision: no HIP call is made)."""
    eight, four = _lib.HSTU_FWD_KERNEL_EIGHT_WAVE, _lib.HSTU_FWD_KERNEL_FOUR_WAVE
    w16 = _lib.HSTU_FWD_KERNEL_SIXTEEN_ROW
    long_d = _desc(num_seqs=16, total_tokens=16 * 512)
    short_d = _desc(num_seqs=16, total_tokens=16 * 512 - 1)
    f32_d = _desc(num_seqs=1, total_tokens=4096, dtype=_lib.HSTU_DTYPE_F32)
    d64 = _desc(num_seqs=1, total_tokens=4096, d_qk=64, d_v=64, ld_q=256, ld_k=256, ld_v=256,
                ld_u=256, ld_out=256)
    try:
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(long_d)) == w16
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(short_d)) == w16
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(f32_d)) == four
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(d64)) == four
        assert lib.hstu_jagged_attn_set_fwd_kernel(eight) == _lib.HSTU_OK
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(short_d)) == eight
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(f32_d)) == four   # unsupported
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(long_d)) == eight
        assert lib.hstu_jagged_attn_set_fwd_kernel(four) == _lib.HSTU_OK
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(long_d)) == four
        assert lib.hstu_jagged_attn_set_fwd_kernel(w16) == _lib.HSTU_OK
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(long_d)) == w16
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(d64)) == four      # unsupported
        w32 = _lib.HSTU_FWD_KERNEL_THIRTYTWO_ROW
        assert lib.hstu_jagged_attn_set_fwd_kernel(w32) == _lib.HSTU_OK
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(long_d)) == w32
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(f32_d)) == four    # unsupported
        assert lib.hstu_jagged_attn_set_fwd_kernel(7) == _lib.HSTU_ERR_INVALID_ARG
        assert lib.hstu_jagged_attn_fwd_kernel_of(ctypes.byref(_desc(num_heads=0))) == -1
    finally:
        lib.hstu_jagged_attn_set_fwd_kernel(_lib.HSTU_FWD_KERNEL_AUTO)


def test_workspace_holds_partials_only_when_items_can_split(lib):
    """The scheduler splits only items of 16 or more key tiles, which needs a
    sequence of at least 481 tokens: smaller batches get a workspace without
    the fp32 partial-output slots (2 x 1024 slots of 128 x d_v floats)."""
    small = lib.hstu_jagged_attn_workspace_bytes(ctypes.byref(_desc(num_seqs=2, total_tokens=480)))
    big = lib.hstu_jagged_attn_workspace_bytes(ctypes.byref(_desc(num_seqs=2, total_tokens=481)))
    slots = 2 * 1024 * 128 * 128 * 4
    assert 0 < small < 1 << 20
    assert big - small >= slots
