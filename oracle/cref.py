"""ctypes binding of the plain C++ oracle (oracle/cpp/oracle.cpp; test infrastructure only).

The same definitions as the numpy oracle, written as explicit loops over tokens, experts and
K with double accumulation; ``tests/test_oracle_cref.py`` pins the two against each other and
against closed forms.  Build with ``python -m oracle.cbuild``."""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

from .cbuild import LIB

_lib = None


def load() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run `python -m oracle.cbuild`")
        lib = C.CDLL(LIB)
        p, i64, i32, f = C.c_void_p, C.c_int64, C.c_int32, C.c_float
        lib.orc_threads.restype = C.c_int
        lib.orc_quant_1x128.argtypes = [p, i64, i64, p, p]
        lib.orc_fp8_scaled_mm_f32.argtypes = [p, p, i64, i64, i64, f, p, p]
        lib.orc_block_fp8_linear_f32.argtypes = [p, p, p, p, i64, i64, i64, i32, p, p]
        lib.orc_block_fp8_linear_bf16.argtypes = [p, p, p, i64, i64, i64, i32, p, p]
        lib.orc_fused_moe.argtypes = [p, i64, i64, i64, i32, i32, p, p, i32, p, p, p, p, p, i32, p]
        lib.orc_fused_moe.restype = C.c_int
        lib.orc_f32_to_bf16.argtypes = [p, i64, p]
        lib.orc_e4m3_table.argtypes = [p]
        _lib = lib
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _ptr(a):
    return None if a is None else a.ctypes.data


def threads() -> int:
    return int(load().orc_threads())


def e4m3_table() -> np.ndarray:
    out = np.empty(256, np.float64)
    load().orc_e4m3_table(out.ctypes.data)
    return out


def quant_1x128(x_bf16):
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 128), np.float32)
    load().orc_quant_1x128(x.ctypes.data, M, K, q.ctypes.data, s.ctypes.data)
    return q, s


def f32_to_bf16(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    load().orc_f32_to_bf16(v.ctypes.data, v.size, out.ctypes.data)
    return out


def fp8_scaled_mm_f32(a_bf16, w_e4m3, scale, bias=None):
    a, w = _c(a_bf16, np.uint16), _c(w_e4m3, np.uint8)
    b = None if bias is None else _c(bias, np.float32)
    M, K = a.shape
    N = w.shape[0]
    out = np.empty((M, N), np.float32)
    load().orc_fp8_scaled_mm_f32(a.ctypes.data, w.ctypes.data, M, N, K, float(scale), _ptr(b), out.ctypes.data)
    return out


def block_fp8_linear_f32(qa, sa, w, sw, block_n, bias=None):
    qa, sa, w, sw = _c(qa, np.uint8), _c(sa, np.float32), _c(w, np.uint8), _c(sw, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    M, K = qa.shape
    N = w.shape[0]
    out = np.empty((M, N), np.float32)
    load().orc_block_fp8_linear_f32(qa.ctypes.data, sa.ctypes.data, w.ctypes.data, sw.ctypes.data, M, N, K,
                                    int(block_n), _ptr(b), out.ctypes.data)
    return out


def block_fp8_linear_bf16(x_bf16, w, sw, block_n, bias=None):
    x, w, sw = _c(x_bf16, np.uint16), _c(w, np.uint8), _c(sw, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    M, K = x.shape
    N = w.shape[0]
    out = np.empty((M, N), np.uint16)
    load().orc_block_fp8_linear_bf16(x.ctypes.data, w.ctypes.data, sw.ctypes.data, M, N, K, int(block_n), _ptr(b),
                                     out.ctypes.data)
    return out


def _moe(x_bf16, topk_ids, topk_weights, wfmt, w1, s1, w2, s2, b1, act_quant):
    x = _c(x_bf16, np.uint16)
    ids, wts = _c(topk_ids, np.int32), _c(topk_weights, np.float32)
    M, H = x.shape
    topk = ids.shape[1]
    E, two_i = w1.shape[0], w1.shape[1]
    sdt = np.float32 if wfmt == 0 else np.uint8
    w1, w2, s1, s2 = _c(w1, np.uint8), _c(w2, np.uint8), _c(s1, sdt), _c(s2, sdt)
    b = None if b1 is None else _c(b1, np.float32)
    out = np.empty((M, H), np.uint16)
    st = load().orc_fused_moe(x.ctypes.data, M, H, two_i // 2, E, topk, ids.ctypes.data, wts.ctypes.data, wfmt,
                              w1.ctypes.data, s1.ctypes.data, w2.ctypes.data, s2.ctypes.data, _ptr(b),
                              int(bool(act_quant)), out.ctypes.data)
    if st != 0:
        raise ValueError("expert id out of range")
    return out


def fused_moe_fp8(x_bf16, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale, w1_bias=None, act_quant=False):
    return _moe(x_bf16, topk_ids, topk_weights, 0, w1, w1_scale, w2, w2_scale, w1_bias, act_quant)


def fused_moe_mxfp4(x_bf16, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale, w1_bias=None):
    return _moe(x_bf16, topk_ids, topk_weights, 1, w1, w1_scale, w2, w2_scale, w1_bias, False)
