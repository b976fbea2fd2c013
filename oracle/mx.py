"""Oracle MX-scaled quantisation and GEMM (test infrastructure only -- see ``oracle/__init__.py``).

The spec path names gfx950's MX-scaled matrix instructions; the source pages reach
them through two formats:

* MXFP4 expert weights -- "vLLM PR 50949 review", summary and implementation item 2: e2m1
  elements with one e8m0 (power-of-two) scale per 32 consecutive elements of a row;
* the MXFP8 activation recipe -- "SGLang PR 35605 review", implementation item 1 and the
  ``fp8_utils.py`` listing: the ``[1, 32]`` block recipe (one scale per token per 32
  columns), which the page's XPU path rejects and this path supports: e4m3 elements with one
  e8m0 scale per 32 consecutive elements of a row.

The pages fix the block size (32) and the element and scale formats, not how a scale is
chosen; the reading here is the OCP Microscaling format's conversion rule (the format the
page names):

    amax = max |x_i| over the 32 elements (exact, fp32)
    shared exponent  e = floor(log2(amax)) - emax,  emax = 8 for e4m3 (its largest normal is
                     1.75 * 2^8), clamped to the e8m0 range [-127, 127]; an all-zero block
                     takes e = -127
    scale code       e + 127 (uint8, e8m0)
    element          e4m3_rne(clamp(x_i / 2^e, -448, 448))   (saturating, ties to even)

``x / 2^e`` is exact in fp32 here (a power-of-two scaling whose result stays normal or zero),
so no rounding precedes the element encoding.

The GEMM (``mx_linear``): ``out[m, n] = bf16( sum_k a[m, k] * w[n, k] + bias[n] )`` with
``a = dec(qa) * 2^(sa - 127)`` (MXFP8 activations) and ``w = dec(qw) * 2^(sw - 127)`` where
``qw`` is e4m3 (MXFP8 weights) or packed e2m1 (MXFP4 weights, element 2j in the low nibble
of byte j); operands decoded exactly to fp32, products and sums in float64, one rounding to
fp32, the bias added in fp32, then bf16 (round to nearest even) -- the same plain definition
as the other oracle GEMMs.
"""

import numpy as np

from .codecs import (E4M3_TABLE, bf16_to_f32, e2m1_decode_packed, e4m3_encode, e8m0_decode,
                     f32_to_bf16)

MX_BLOCK = 32
E4M3_EMAX = 8  # exponent of e4m3's largest normal value, 1.75 * 2^8 = 448


def _floor_log2(v: np.ndarray) -> np.ndarray:
    """floor(log2(v)) for positive finite float32 values, from the binary exponent (exact)."""
    _, ex = np.frexp(np.asarray(v, np.float64))  # v = m * 2^ex, m in [0.5, 1)
    return ex.astype(np.int64) - 1


def mxfp8_quant_f32(x32: np.ndarray):
    """float32 [M, K] (K % 32 == 0) -> (e4m3 codes uint8 [M, K], e8m0 scale codes uint8 [M, K/32])."""
    x32 = np.asarray(x32, dtype=np.float32)
    M, K = x32.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    g = x32.reshape(M, K // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(g), axis=2) if K else np.zeros((M, 0), np.float32)
    e = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)) - E4M3_EMAX, -127)
    e = np.clip(e, -127, 127)
    scaled = (g.astype(np.float64) / np.ldexp(1.0, e)[:, :, None]).astype(np.float32)
    q = e4m3_encode(np.clip(scaled, -448.0, 448.0)).reshape(M, K)
    return q, (e + 127).astype(np.uint8)


def mxfp8_quant(x_bf16: np.ndarray):
    """bf16 bit patterns [M, K] -> (e4m3 codes [M, K], e8m0 scale codes [M, K/32])."""
    return mxfp8_quant_f32(bf16_to_f32(x_bf16))


def dequant_mx(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """Row-wise MX operand -> fp32 [rows, K].  fmt "e4m3": codes uint8 [rows, K];
    fmt "e2m1": packed uint8 [rows, K/2].  scales: e8m0 uint8 [rows, K/32]."""
    if fmt == "e4m3":
        v = E4M3_TABLE[np.asarray(codes, np.uint8)]
    elif fmt == "e2m1":
        v = e2m1_decode_packed(codes)
    else:
        raise ValueError(f"unknown MX element format {fmt!r}")
    s = np.repeat(e8m0_decode(scales), MX_BLOCK, axis=1)
    return (v * s).astype(np.float32)


def mx_linear_f32(qa, sa, qw, sw, w_fmt: str, bias=None) -> np.ndarray:
    """MX-scaled linear before the final bf16 rounding (fp32 [M, N])."""
    a = dequant_mx(qa, sa, "e4m3").astype(np.float64)
    w = dequant_mx(qw, sw, w_fmt).astype(np.float64)
    out = (a @ w.T).astype(np.float32)
    if bias is not None:
        out = (out + np.asarray(bias, np.float32)).astype(np.float32)
    return out


def mx_linear(qa, sa, qw, sw, w_fmt: str, bias=None) -> np.ndarray:
    """MXFP8 activations x MXFP8 ("e4m3") or MXFP4 ("e2m1") weights -> bf16 bits [M, N]."""
    return f32_to_bf16(mx_linear_f32(qa, sa, qw, sw, w_fmt, bias))


def mx_linear_bf16(x_bf16, qw, sw, w_fmt: str, bias=None) -> np.ndarray:
    """bf16 activations: MXFP8-quantise per row per 32 columns, then the MX linear."""
    qa, sa = mxfp8_quant(x_bf16)
    return mx_linear(qa, sa, qw, sw, w_fmt, bias)
