"""Oracle codecs (test infrastructure only -- see ``oracle/__init__.py``).

Formats, as the source pages use them:

* e4m3 -- ``torch.float8_e4m3fn`` weights and activations ("SGLang PR 32618
  review", ``test_gemm.py`` listing; "SGLang PR 35605 review",
  ``test_xpu_fp8_linear.py`` listing).  OCP FP8 E4M3: 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits, no infinities, the all-ones
  exponent-and-mantissa pattern is NaN, largest finite value 448.
* e2m1 + e8m0 -- MXFP4 expert weights ("vLLM PR 50949 review", summary and
  implementation item 2).  OCP MX: e2m1 has 1 sign bit, 2 exponent bits with
  bias 1 and 1 mantissa bit; e8m0 is an unsigned power-of-two exponent with
  bias 127, 0xFF is NaN.
* bf16 -- activations and outputs on every page.

All decoders return float64 (every value of these formats is exact there).
"""

import numpy as np

__all__ = [
    "e4m3_value", "E4M3_TABLE", "e4m3_decode", "e4m3_encode", "E4M3_MAX",
    "e2m1_value", "E2M1_TABLE", "e2m1_decode_packed",
    "e8m0_decode",
    "bf16_to_f32", "f32_to_bf16",
]

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one e4m3 code, straight from the field definition."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:  # subnormal: (man / 8) * 2^(1 - 7)
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)

# codes 0x00 .. 0x7E are the finite non-negative values, in ascending order
_E4M3_POS = E4M3_TABLE[:0x7F].copy()
assert np.all(np.diff(_E4M3_POS) > 0)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32 values in [-448, 448] -> nearest e4m3 code, ties to the even code.

    The sign bit is copied from the input, so -0.0 encodes to 0x80 and a
    negative value that rounds to zero keeps its sign.  The caller clamps
    first; a value outside the range (or NaN) is an error here.
    """
    v = np.asarray(v, dtype=np.float32)
    if np.any(np.isnan(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite values within [-448, 448]")
    a = np.abs(v).astype(np.float64)
    lo = np.searchsorted(_E4M3_POS, a, side="right") - 1  # _E4M3_POS[lo] <= a
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    mid = (_E4M3_POS[lo] + _E4M3_POS[hi]) / 2.0  # exact in float64
    even = np.where(lo % 2 == 0, lo, hi)
    code = np.where(a < mid, lo, np.where(a > mid, hi, even))
    code = np.where(_E4M3_POS[lo] == a, lo, code)
    sign = np.signbit(v).astype(np.int64)
    return (code.astype(np.int64) | (sign << 7)).astype(np.uint8)


def e2m1_value(nibble: int) -> float:
    """Value of one e2m1 code (low 4 bits), from the field definition."""
    sign = -1.0 if nibble & 0x8 else 1.0
    exp = (nibble >> 1) & 0x3
    man = nibble & 0x1
    if exp == 0:  # subnormal: man * 2^(1 - 1) / 2
        return sign * man * 0.5
    return sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m1_decode_packed(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] packed e2m1 pairs -> float64 [..., K].

    Element 2j sits in the low nibble of byte j and element 2j+1 in the high
    nibble (the pages leave the packing open; this is the reading used on both
    sides of the parity tests).
    """
    p = np.asarray(packed, dtype=np.uint8)
    lo = E2M1_TABLE[p & 0xF]
    hi = E2M1_TABLE[p >> 4]
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 e8m0 exponents -> float64 2^(e-127); 0xFF -> NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = np.ldexp(1.0, c - 127)
    return np.where(c == 0xFF, np.nan, out)


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (the bf16 bits are the high half)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Keeps the high 16 bits and rounds on the discarded low 16: above half
    rounds up, below half rounds down, exactly half rounds to the even
    pattern.  Overflow goes to infinity; NaN becomes a quiet NaN.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    upper = (u >> 16).astype(np.uint32)
    lower = u & np.uint32(0xFFFF)
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    r = upper + up.astype(np.uint32)
    r = np.where(np.isnan(x), (upper & 0x8000) | 0x7FC0, r)
    return r.astype(np.uint16)
