"""ctypes loader for libmxq.so (the C ABI declared in include/mxq.h).

There is no fallback: if the library has not been built, every call raises.
"""

from __future__ import annotations

import ctypes as C
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxq.so")

MXQ_OK = 0
MXQ_ERR_NULL = 1
MXQ_ERR_SHAPE = 2
MXQ_ERR_BLOCK = 3
MXQ_ERR_DTYPE = 4
MXQ_ERR_WORKSPACE = 5
MXQ_ERR_ARCH = 6
MXQ_ERR_LAUNCH = 7
MXQ_ERR_ARG = 8
MXQ_ERR_SCRATCH = 9
MXQ_NOALLOC_SCRATCH_BYTES = 32 << 20

MXQ_DTYPE_BF16 = 0
MXQ_DTYPE_F32 = 1
MXQ_DTYPE_E4M3 = 2
MXQ_DTYPE_E2M1 = 3

MXQ_WEIGHTS_FP8_BLOCK = 0
MXQ_WEIGHTS_MXFP4 = 1

MXQ_DISPATCH_PER_BLOCK = 0
MXQ_DISPATCH_FORCED = 1
MXQ_DISPATCH_LAYER_AVERAGE = 2

MXQ_TINY_MFMA = 0
MXQ_TINY_GEMV = 1
MXQ_TINY_ROWS_AUTO = -1
MXQ_K_SPLIT_AUTO = 0
MXQ_SORT_AUTO = 0
MXQ_SORT_ALWAYS = 1
MXQ_FUSE_AUTO = 0
MXQ_FUSE_NONE = 1

MXQ_LAYOUT_PLAIN = 0
MXQ_LAYOUT_TILED = 1

# fields of mxq_fused_moe_plan, and the values of its enumerated fields
MOE_PLAN_FIELDS = ("path", "tiles", "classes", "block_m1", "block_m2", "k_split1", "k_split2", "silu", "combine")
MOE_PLAN_NAMES = {
    "path": ("sorted", "expert_stream", "self_routed"),
    "tiles": ("ring", "register", "w8a8", "w8a8_wide"),
    "silu": ("kernel", "split_sum", "stage1_epilogue", "stage2_staging", "expert_stream"),
    "combine": ("kernel", "stage2_epilogue"),
}

# byte offsets reported by mxq_fused_moe_workspace_layout
MOE_WS_FIELDS = ("sorted_ids", "expert_ids", "offsets", "num_blocks", "qx", "sx", "ic0", "ic1", "ic1_q", "ic1_s",
                 "y", "block_m", "partial")


class MoeDispatch(C.Structure):
    """struct mxq_moe_dispatch (per-call dispatch of the fused MoE)."""
    _fields_ = [("mode", C.c_int32), ("forced_class", C.c_int32), ("tiny_max_rows", C.c_int32),
                ("tiny_kernel", C.c_int32), ("k_split", C.c_int32), ("sort", C.c_int32),
                ("fuse", C.c_int32)]

_p = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64
_sz = C.c_size_t

# name -> (restype, argtypes), mirroring include/mxq.h
SIGNATURES = {
    "mxq_status_string": (C.c_char_p, [_i32]),
    "mxq_abi_version": (_i32, []),
    "mxq_init": (_i32, [_i32]),
    "mxq_per_token_group_quant_fp8": (_i32, [_p, _i64, _i64, _i64, _i32, _p, _p, _p]),
    "mxq_fp8_scaled_mm_workspace_size": (_sz, [_i64, _i64, _i64]),
    "mxq_fp8_scaled_mm": (_i32, [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i32, _p, _i64, _p, _sz, _p]),
    "mxq_fp8_scaled_bmm": (_i32, [_p, _i64, _i64, _i64, _i64, _i64, _p, _i64, _i64, _p, _i64, _p, _i32, _i64,
                                   _p, _i64, _i64, _p]),
    "mxq_block_fp8_linear_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
    "mxq_block_fp8_linear": (_i32, [_p, _i32, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _i64, _i32, _i32,
                                     _p, _i32, _p, _i32, _i64, _p, _sz, _p]),
    "mxq_block_fp8_linear_noalloc": (_i32, [_p, _i32, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _i64, _i32,
                                             _i32, _p, _i32, _p, _i32, _i64, _p]),
    "mxq_mxfp8_quant": (_i32, [_p, _i64, _i64, _i64, _p, _p, _p]),
    "mxq_mx_linear_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
    "mxq_mx_linear": (_i32, [_p, _i32, _p, _i64, _i64, _i64, _p, _i32, _i64, _p, _p, _i32, _p, _i64, _p, _sz, _p]),
    "mxq_moe_max_blocks": (_i64, [_i64, _i32, _i32, _i32]),
    "mxq_moe_align": (_i32, [_p, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _p]),
    "mxq_fused_moe_workspace_size": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32, _i32]),
    "mxq_fused_moe_fp8": (_i32, [_p, _i64, _i64, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _i32, _i32,
                                  C.POINTER(MoeDispatch), _p, _p, _sz, _p]),
    "mxq_fused_moe_mxfp4": (_i32, [_p, _i64, _i64, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _i32,
                                    C.POINTER(MoeDispatch), _p, _p, _sz, _p]),
    "mxq_fused_moe_workspace_layout": (_i32, [_i64, _i64, _i64, _i32, _i32, _i32, _i32, C.POINTER(_i64)]),
    "mxq_fused_moe_plan": (_i32, [_i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32, C.POINTER(MoeDispatch),
                                  C.POINTER(_i32)]),
    "mxq_silu_and_mul": (_i32, [_p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "mxq_moe_prepack_size": (_sz, [_i64, _i64, _i64]),
    "mxq_moe_prepack_scales_size": (_sz, [_i64, _i64, _i64]),
    "mxq_moe_prepack": (_i32, [_p, _i64, _i64, _i64, _p, _p]),
    "mxq_moe_prepack_scales": (_i32, [_p, _i64, _i64, _i64, _p, _p]),
}

_lock = threading.Lock()
_lib = None


class MxqError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


def load() -> C.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is not built; run `python -m mxfp4_block_scaled_expert_amd.build` "
                    "(there is no non-HIP fallback)")
            lib = C.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                f = getattr(lib, name)
                f.restype = res
                f.argtypes = args
            _lib = lib
    return _lib


def check(fn: str, status: int) -> None:
    if status == MXQ_OK:
        return
    text = load().mxq_status_string(status).decode()
    if status in (MXQ_ERR_SHAPE, MXQ_ERR_BLOCK, MXQ_ERR_DTYPE):
        raise ValueError(f"{fn}: {text} (status {status})")
    raise MxqError(fn, status, text)
