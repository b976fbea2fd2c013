"""Oracle per-token group quantisation (test infrastructure only).

"SGLang PR 35605 review", implementation item 1 and the ``fp8_utils.py``
listing: when the linear receives bf16 input it quantises it on the fly, one
e4m3 code per element and one fp32 scale per token per ``block_k`` = 128
consecutive columns (scale tensor ``[M, K/128]``); the weight operand is then
consumed by the block-scaled GEMM.  The pages name the routine
(``per_token_group_quant_fp8``) but do not print its body, so this is the
plainest reading of "scale = amax / 448" that the parity tests share with the
GPU side:

    amax = max_i |x_i|                  (fp32, exact)
    s    = max(amax, 1e-10) / 448       (one IEEE fp32 division)
    q_i  = e4m3_rne(clamp(x_i / s, -448, 448))   (fp32 division per element)

Both ``q`` and ``s`` are compared bit for bit with the HIP kernel.
"""

import numpy as np

from .codecs import bf16_to_f32, e4m3_encode

EPS = np.float32(1e-10)
FP8_MAX = np.float32(448.0)


def group_quant_f32(x32: np.ndarray, group: int = 128):
    """float32 [M, K] -> (uint8 codes [M, K], float32 scales [M, K/group])."""
    x32 = np.asarray(x32, dtype=np.float32)
    M, K = x32.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    xg = x32.reshape(M, K // group, group)
    amax = np.max(np.abs(xg), axis=2) if K else np.zeros((M, 0), np.float32)
    s = (np.maximum(amax, EPS) / FP8_MAX).astype(np.float32)
    with np.errstate(over="ignore"):
        y = (xg / s[:, :, None]).astype(np.float32)
    y = np.clip(y, -FP8_MAX, FP8_MAX)
    q = e4m3_encode(y).reshape(M, K)
    return q, s


def per_token_group_quant_fp8(x_bf16: np.ndarray, group: int = 128):
    """bf16 bit patterns [M, K] -> (e4m3 codes [M, K], fp32 scales [M, K/group])."""
    return group_quant_f32(bf16_to_f32(x_bf16), group)
