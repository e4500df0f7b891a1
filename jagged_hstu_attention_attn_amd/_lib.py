"""ctypes view of libhstu_attn.so (the C ABI of include/hstu_attn.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in the package.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhstu_attn.so")

HSTU_OK = 0
HSTU_ERR_INVALID_ARG = -1
HSTU_ERR_UNSUPPORTED = -2
HSTU_ERR_WORKSPACE = -3
HSTU_ERR_HIP = -4

HSTU_DTYPE_F32 = 0
HSTU_DTYPE_BF16 = 1
HSTU_EPILOGUE_LN_U = 0
HSTU_EPILOGUE_NONE = 1
HSTU_EPILOGUE_LN_ALL_U = 2
HSTU_FWD_KERNEL_AUTO = 0
HSTU_FWD_KERNEL_FOUR_WAVE = 1
HSTU_FWD_KERNEL_EIGHT_WAVE = 2
HSTU_FWD_KERNEL_SIXTEEN_ROW = 3
HSTU_FWD_KERNEL_THIRTYTWO_ROW = 4

# every function the header declares
EXPORTS = (
    "hstu_jagged_attn_supported",
    "hstu_jagged_attn_workspace_bytes",
    "hstu_jagged_attn_fwd",
    "hstu_jagged_attn_plan",
    "hstu_jagged_attn_run",
    "hstu_jagged_attn_run_timed",
    "hstu_jagged_attn_plan_candidates",
    "hstu_jagged_attn_fwd_candidates",
    "hstu_jagged_attn_fwd_noalloc",
    "hstu_layer_workspace_bytes",
    "hstu_layer_fwd",
    "hstu_jagged_attn_valid_pairs",
    "hstu_jagged_attn_grid",
    "hstu_jagged_attn_set_fwd_kernel",
    "hstu_jagged_attn_fwd_kernel_of",
    "hstu_jagged_attn_bwd_workspace_bytes",
    "hstu_jagged_attn_bwd",
    "hstu_jagged_attn_fwd_train",
    "hstu_last_error",
)


class HstuAttnDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("ld_q", ctypes.c_int64),
        ("ld_k", ctypes.c_int64),
        ("ld_v", ctypes.c_int64),
        ("ld_u", ctypes.c_int64),
        ("ld_out", ctypes.c_int64),
        ("pos_table_len", ctypes.c_int32),
        ("time_table_len", ctypes.c_int32),
        ("ln_eps", ctypes.c_float),
        ("epilogue", ctypes.c_int32),
        ("pos_clamp", ctypes.c_int32),
    ]


class HstuLayerDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("pos_table_len", ctypes.c_int32),
        ("time_table_len", ctypes.c_int32),
        ("ln_eps", ctypes.c_float),
    ]


class HstuError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"hstu status {code}: {message}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m jagged_hstu_attention_attn_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(HstuAttnDesc)
    i32, i64, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.hstu_jagged_attn_supported.restype = ctypes.c_int
    lib.hstu_jagged_attn_supported.argtypes = [i32, i32, i32]
    lib.hstu_jagged_attn_workspace_bytes.restype = sz
    lib.hstu_jagged_attn_workspace_bytes.argtypes = [D]
    run_args = [D, P, P, P, P, P, P, P, i32, i32, f32, f32, P, P, P, P, sz, P]
    for name in ("hstu_jagged_attn_fwd", "hstu_jagged_attn_run",
                 "hstu_jagged_attn_fwd_candidates"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = run_args
    lib.hstu_jagged_attn_run_timed.restype = ctypes.c_int
    lib.hstu_jagged_attn_run_timed.argtypes = run_args + [P, P]
    for name in ("hstu_jagged_attn_plan", "hstu_jagged_attn_plan_candidates"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [D, P, P, i32, i32, P, sz, P]
    LD = ctypes.POINTER(HstuLayerDesc)
    lib.hstu_layer_workspace_bytes.restype = sz
    lib.hstu_layer_workspace_bytes.argtypes = [LD]
    lib.hstu_layer_fwd.restype = ctypes.c_int
    lib.hstu_layer_fwd.argtypes = [LD, P, P, P, P, P, P, P, i32, i32, f32, f32, P, P, P, P, sz,
                                   P]
    lib.hstu_jagged_attn_valid_pairs.restype = i64
    lib.hstu_jagged_attn_valid_pairs.argtypes = [i32, P, P, i32, i32]
    lib.hstu_jagged_attn_grid.restype = ctypes.c_int
    lib.hstu_jagged_attn_grid.argtypes = [D]
    lib.hstu_jagged_attn_fwd_noalloc.restype = ctypes.c_int
    lib.hstu_jagged_attn_fwd_noalloc.argtypes = [D, P, P, P, P, P, P, P, i32, i32, f32, f32, P,
                                                 P, P, P]
    lib.hstu_jagged_attn_set_fwd_kernel.restype = ctypes.c_int
    lib.hstu_jagged_attn_set_fwd_kernel.argtypes = [i32]
    lib.hstu_jagged_attn_fwd_kernel_of.restype = ctypes.c_int
    lib.hstu_jagged_attn_fwd_kernel_of.argtypes = [D]
    lib.hstu_jagged_attn_bwd_workspace_bytes.restype = sz
    lib.hstu_jagged_attn_bwd_workspace_bytes.argtypes = [D]
    lib.hstu_jagged_attn_bwd.restype = ctypes.c_int
    lib.hstu_jagged_attn_bwd.argtypes = [D, P, P, P, P, P, P, P, i32, i32, f32, f32, P, P, P,
                                         P, P, P, P, P, P, P, P, sz, P]
    lib.hstu_jagged_attn_fwd_train.restype = ctypes.c_int
    lib.hstu_jagged_attn_fwd_train.argtypes = [D, P, P, P, P, P, P, P, i32, i32, f32, f32, P, P,
                                               P, P, P, sz, P]
    lib.hstu_last_error.restype = ctypes.c_char_p
    lib.hstu_last_error.argtypes = []
    _lib = lib
    return lib


def last_error() -> str:
    return load().hstu_last_error().decode()


def check(code: int) -> None:
    if code != HSTU_OK:
        raise HstuError(code, last_error())
