"""Oracle dense scaled GEMMs (test infrastructure only).

Arithmetic (the plain "dequantise to fp32, multiply, apply the scales"
definition): every operand element is decoded exactly and multiplied by its
scale in fp32; the dot products are summed in float64 (numpy matmul) and the
sum is rounded once to fp32; the epilogue (per-tensor scale, bias) runs in
fp32; the output is rounded fp32 -> bf16 to nearest even.

* ``fp8_scaled_mm`` -- "SGLang PR 32618 review", implementation items 1-2 and
  the ``test_gemm.py`` listing: ``out = bf16((A @ dec(W)^T) * s + bias)`` with
  bf16 ``A [M, K]``, e4m3 ``W [N, K]``, one fp32 scale, optional fp32 bias.
  The order -- full matmul, then scale, then bias, then bf16 -- is the one the
  listing's reference computes.
* ``fp8_scaled_bmm`` -- the batched FP8 scaled GEMM that "SGLang PR 32618
  review" ("Feature and motivation") names as the existing use of the kernel
  (DeepSeek MLA): entry ``z`` is ``bf16((A[z] @ dec(W[z])^T) * s[z] + bias[z])``,
  each entry in the same order as ``fp8_scaled_mm``.  The page gives no more
  than that sentence; one fp32 scale per entry (or one shared) is the reading.
* ``block_fp8_linear`` -- "SGLang PR 35605 review", implementation item 1 and
  the ``fp8_utils.py`` listing: activations carry one scale per token per 128
  columns (``[M, K/128]``); weights carry one scale per ``block_n`` x 128 block
  (``[ceil(N/block_n), K/128]``, ``block_n`` in {1, 128}); optional bias; bf16
  output.
* ``w8a16_block_linear`` -- the same block-scaled weights against bf16
  activations: the stage GEMM of the W8A16 routed MoE ("vLLM PR 50949
  review", ``moe_fp8.cpp`` listing, where bf16 rows meet block-scaled FP8
  expert weights).
"""

import numpy as np

from .codecs import E4M3_TABLE, bf16_to_f32, f32_to_bf16
from .quant import per_token_group_quant_fp8


def dequant_e4m3_rows(codes: np.ndarray, row_scale: np.ndarray, group: int = 128) -> np.ndarray:
    """e4m3 [R, K] with per-row, per-``group``-column fp32 scales [R, K/group] -> fp32."""
    v = E4M3_TABLE[codes].astype(np.float32)
    s = np.repeat(np.asarray(row_scale, np.float32), group, axis=1)
    return (v * s).astype(np.float32)


def dequant_e4m3_blocks(codes: np.ndarray, grid: np.ndarray, block_n: int, block_k: int = 128) -> np.ndarray:
    """e4m3 [N, K] with a [ceil(N/block_n), K/block_k] fp32 scale grid -> fp32 [N, K]."""
    N, K = codes.shape
    v = E4M3_TABLE[codes].astype(np.float32)
    g = np.asarray(grid, np.float32)
    s = np.repeat(np.repeat(g, block_n, axis=0)[:N], block_k, axis=1)
    return (v * s).astype(np.float32)


def _dot_f32(a32: np.ndarray, b32: np.ndarray) -> np.ndarray:
    """sum_k a[m,k] * b[n,k] in float64, rounded once to fp32."""
    return (a32.astype(np.float64) @ b32.astype(np.float64).T).astype(np.float32)


def fp8_scaled_mm_f32(a_bf16, w_e4m3, scale, bias=None) -> np.ndarray:
    """Per-tensor W8A16 GEMM before the final bf16 rounding (fp32 [M, N])."""
    a = bf16_to_f32(a_bf16)
    w = E4M3_TABLE[w_e4m3].astype(np.float32)
    out = _dot_f32(a, w) * np.float32(scale)
    if bias is not None:
        out = out + np.asarray(bias, np.float32)
    return out.astype(np.float32)


def fp8_scaled_mm(a_bf16, w_e4m3, scale, bias=None) -> np.ndarray:
    """bf16 [M, K] x e4m3 [N, K]^T * scale (+ bias) -> bf16 [M, N] (uint16 bits)."""
    return f32_to_bf16(fp8_scaled_mm_f32(a_bf16, w_e4m3, scale, bias))


def fp8_scaled_bmm_f32(a_bf16, w_e4m3, scales, bias=None) -> np.ndarray:
    """Batched per-tensor W8A16 before the final bf16 rounding (fp32 [B, M, N]).

    ``a_bf16`` [B, M, K] bf16 bits, ``w_e4m3`` [B, N, K] codes, ``scales`` [B] fp32,
    ``bias`` None or [B, N] fp32.  Batched float64 matmul, one fp32 rounding per entry
    sum, then the scale and the bias in fp32.
    """
    a = bf16_to_f32(np.asarray(a_bf16)).astype(np.float64)
    w = E4M3_TABLE[np.asarray(w_e4m3)].astype(np.float64)
    prod = np.matmul(a, np.swapaxes(w, 1, 2)).astype(np.float32)
    out = prod * np.asarray(scales, np.float32).reshape(-1, 1, 1)
    if bias is not None:
        out = out + np.asarray(bias, np.float32)[:, None, :]
    return out.astype(np.float32)


def fp8_scaled_bmm(a_bf16, w_e4m3, scales, bias=None) -> np.ndarray:
    """bf16 [B, M, K] x e4m3 [B, N, K]^T * scale[b] (+ bias[b]) -> bf16 [B, M, N] (uint16 bits)."""
    return f32_to_bf16(fp8_scaled_bmm_f32(a_bf16, w_e4m3, scales, bias))


def block_fp8_linear_f32(qa, sa, w, sw, block_n, bias=None) -> np.ndarray:
    """W8A8 block-scaled linear before the final bf16 rounding (fp32 [M, N])."""
    if block_n not in (1, 128):
        raise ValueError("block_n must be 1 or 128")
    a = dequant_e4m3_rows(qa, sa)
    b = dequant_e4m3_blocks(w, sw, block_n)
    out = _dot_f32(a, b)
    if bias is not None:
        out = out + np.asarray(bias, np.float32)
    return out.astype(np.float32)


def block_fp8_linear(qa, sa, w, sw, block_n, bias=None) -> np.ndarray:
    """Pre-quantised e4m3 activations [M, K] + [M, K/128] scales -> bf16 [M, N]."""
    return f32_to_bf16(block_fp8_linear_f32(qa, sa, w, sw, block_n, bias))


def block_fp8_linear_bf16(x_bf16, w, sw, block_n, bias=None) -> np.ndarray:
    """bf16 activations: quantise per token per 128 columns, then the W8A8 linear."""
    qa, sa = per_token_group_quant_fp8(x_bf16, 128)
    return block_fp8_linear(qa, sa, w, sw, block_n, bias)


def w8a16_block_linear_f32(a_bf16, w, sw, block_n, bias=None) -> np.ndarray:
    """bf16 activations x block-scaled e4m3 weights, before bf16 rounding."""
    a = bf16_to_f32(a_bf16)
    b = dequant_e4m3_blocks(w, sw, block_n)
    out = _dot_f32(a, b)
    if bias is not None:
        out = out + np.asarray(bias, np.float32)
    return out.astype(np.float32)
