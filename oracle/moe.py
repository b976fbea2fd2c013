"""Oracle routed fused-MoE experts (test infrastructure only).

"vLLM PR 50949 review", implementation item 2 and the ``moe_fp8.cpp`` listing:
the routed MoE runs, for every expert block, stage 1 ``hidden @ w1`` into a
``2N``-wide intermediate (gate and up halves, with an optional per-expert
``w1`` bias), an activation, and stage 2 ``activation @ w2``; FP8 (block
scaled) and MXFP4 weights share the same structure.  Routed rows are tokens
repeated ``topk`` times (token = flat id / topk).  The pages say only
"activation"; the path computes SiLU-and-mul, and combines the ``topk``
expert outputs of a token with its routing weights.

Readings of what the pages leave open (the same readings the HIP path uses):

* ``w1`` rows ``[0, I)`` are the gate, rows ``[I, 2I)`` the up projection.
* ``ic0 = bf16(x @ w1^T + b1)``; ``ic1 = bf16(silu(gate) * up)`` with
  ``silu(g) = g / (1 + exp(-g))``; stage 2 keeps fp32 ``y = ic1 @ w2^T``;
  ``out[t] = bf16(sum_k w[t,k] * y[t*topk+k])``.  Sums in float64, rounded
  once to fp32 (the SiLU product is rounded fp64 -> fp32 -> bf16).
* W8A8 (``act_quant=True``): ``x`` is quantised per token per 128 columns
  before stage 1 and ``ic1`` likewise before stage 2 (same rule as the
  standalone quantiser).  W8A16 keeps both stage inputs in bf16.
* MXFP4 weights are W4A16: bf16 activations, e2m1 codes packed two per byte
  (low nibble = even column), one e8m0 scale per row per 32 columns.
* No ``w2`` bias.

This is written as its own loop over experts and each expert's rows in
ascending flat id; it does not call the dense oracle.  The stages are also
exposed one by one (``stage1_rows``, ``silu_mul_bf16``, ``quant_rows``,
``stage2_rows``, ``combine``) so that each stage of the GPU path can be checked
on the GPU's own input to that stage; ``_routed_moe`` is their composition.
"""

import numpy as np

from .codecs import (E4M3_TABLE, bf16_to_f32, f32_to_bf16, e2m1_decode_packed,
                     e8m0_decode)
from .quant import group_quant_f32


def dequant_fp8_expert(codes, grid, block_k=128):
    """e4m3 [N, K] with [ceil(N/128), K/128] scales -> fp32 [N, K] (128x128 blocks)."""
    N, K = codes.shape
    v = E4M3_TABLE[codes].astype(np.float32)
    s = np.repeat(np.repeat(np.asarray(grid, np.float32), 128, axis=0)[:N], block_k, axis=1)
    return (v * s).astype(np.float32)


def dequant_mxfp4_expert(packed, scales):
    """packed e2m1 [N, K/2] with e8m0 [N, K/32] -> fp32 [N, K]."""
    v = e2m1_decode_packed(packed)
    s = np.repeat(e8m0_decode(scales), 32, axis=1)
    return (v * s).astype(np.float32)


def silu_mul_bf16(ic0_f32: np.ndarray, inter: int) -> np.ndarray:
    """fp32 [rows, 2I] (the bf16 ic0 values) -> bf16 bits [rows, I] of silu(gate) * up."""
    g = ic0_f32[:, :inter].astype(np.float64)
    u = ic0_f32[:, inter:].astype(np.float64)
    with np.errstate(over="ignore"):
        act = g / (1.0 + np.exp(-g))
    return f32_to_bf16((act * u).astype(np.float32))


def stage1_rows(a_f32: np.ndarray, w1_f32: np.ndarray, b1=None) -> np.ndarray:
    """Stage 1 of routed rows of one expert: bf16 bits of ``a @ w1^T (+ b1)`` ([rows, 2I]);
    ``a`` the (dequantised) activation rows, ``w1`` the expert's dequantised weights."""
    g = (a_f32.astype(np.float64) @ w1_f32.astype(np.float64).T).astype(np.float32)
    if b1 is not None:
        g = (g + np.asarray(b1, np.float32)).astype(np.float32)
    return f32_to_bf16(g)


def quant_rows(h_bf16: np.ndarray):
    """W8A8 stage-2 input: bf16 bits [rows, I] -> (e4m3 codes, fp32 [rows, I/128] scales) and
    the fp32 values the stage multiplies (code value x group scale)."""
    q, s = group_quant_f32(bf16_to_f32(h_bf16), 128)
    return q, s, (E4M3_TABLE[q].astype(np.float32) * np.repeat(s, 128, axis=1)).astype(np.float32)


def stage2_rows(a2_f32: np.ndarray, w2_f32: np.ndarray) -> np.ndarray:
    """Stage 2 of routed rows of one expert: fp32 ``a2 @ w2^T`` ([rows, H])."""
    return (a2_f32.astype(np.float64) @ w2_f32.astype(np.float64).T).astype(np.float32)


def combine(y: np.ndarray, topk_weights: np.ndarray) -> np.ndarray:
    """fp32 y [M * topk, H] (row t * topk + k) and weights [M, topk] -> bf16 bits [M, H] of
    sum_k w[t, k] * y[t * topk + k] (float64 sum, one rounding to fp32, then bf16)."""
    w = np.asarray(topk_weights, np.float64)
    M, topk = w.shape
    acc = np.einsum("tk,tkh->th", w, np.asarray(y, np.float64).reshape(M, topk, -1))
    return f32_to_bf16(acc.astype(np.float32))


def _routed_moe(x_bf16, topk_ids, topk_weights, n_experts, inter, deq_w1, deq_w2,
                b1, act_quant):
    x_bf16 = np.asarray(x_bf16, np.uint16)
    M, H = x_bf16.shape
    ids = np.asarray(topk_ids).astype(np.int64)
    topk = ids.shape[1]
    flat = ids.reshape(-1)
    R = M * topk
    if np.any(flat < 0) or np.any(flat >= n_experts):
        raise ValueError("expert id out of range")
    if act_quant:
        qx, sx = group_quant_f32(bf16_to_f32(x_bf16), 128)
        xin = (E4M3_TABLE[qx].astype(np.float32) * np.repeat(sx, 128, axis=1)).astype(np.float32)
    else:
        xin = bf16_to_f32(x_bf16)
    y = np.zeros((R, H), dtype=np.float32)
    for e in range(n_experts):
        rows = np.nonzero(flat == e)[0]
        if rows.size == 0:
            continue  # an empty expert contributes nothing
        ic0 = bf16_to_f32(stage1_rows(xin[rows // topk], deq_w1(e), None if b1 is None else b1[e]))
        ic1 = silu_mul_bf16(ic0, inter)
        a2 = quant_rows(ic1)[2] if act_quant else bf16_to_f32(ic1)
        y[rows] = stage2_rows(a2, deq_w2(e))
    return combine(y, np.asarray(topk_weights).reshape(M, topk))


def fused_moe_fp8(x_bf16, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale,
                  w1_bias=None, act_quant=False):
    """Block-FP8 experts: w1 e4m3 [E, 2I, H] + [E, 2I/128, H/128] scales,
    w2 e4m3 [E, H, I] + [E, ceil(H/128), I/128]; bf16 out [M, H]."""
    E, two_i, _ = w1.shape
    return _routed_moe(
        x_bf16, topk_ids, topk_weights, E, two_i // 2,
        lambda e: dequant_fp8_expert(w1[e], w1_scale[e]),
        lambda e: dequant_fp8_expert(w2[e], w2_scale[e]),
        w1_bias, act_quant)


def fused_moe_mxfp4(x_bf16, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale,
                    w1_bias=None):
    """MXFP4 experts: w1 packed e2m1 [E, 2I, H/2] + e8m0 [E, 2I, H/32],
    w2 [E, H, I/2] + [E, H, I/32]; bf16 activations; bf16 out [M, H]."""
    E, two_i, _ = w1.shape
    return _routed_moe(
        x_bf16, topk_ids, topk_weights, E, two_i // 2,
        lambda e: dequant_mxfp4_expert(w1[e], w1_scale[e]),
        lambda e: dequant_mxfp4_expert(w2[e], w2_scale[e]),
        w1_bias, False)
