"""Pins of the MX oracle (oracle/mx.py) against things other than itself: torch's e4m3 and
e8m0 casts (independent library routines), a brute-force search for the shared exponent,
closed forms, the rounding error bound, explicit loops, and the other oracle GEMMs on inputs
where the definitions coincide."""

import math

import numpy as np
import pytest
import torch

from oracle import codecs as C
from oracle import dense as D
from oracle import moe as OM
from oracle import mx as MX


def _bf16(x) -> np.ndarray:
    return C.f32_to_bf16(np.asarray(x, np.float32))


def _brute_shared_exp(amax: float) -> int:
    """The e with 2^(e+8) <= amax < 2^(e+9), searched (clamped to [-127, 127]); -127 for 0."""
    if amax == 0:
        return -127
    for e in range(-160, 128):
        if math.ldexp(1.0, e + 8) <= amax < math.ldexp(1.0, e + 9):
            return max(-127, min(127, e))
    raise AssertionError(amax)


def test_shared_exponent_brute_force_and_torch_e8m0():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-60, 60, (64, 1)))).astype(np.float32)
    x[0, :32] = 0.0  # a zero block
    x[1, :32] = 1e-40  # subnormal fp32 values
    q, s = MX.mxfp8_quant_f32(x)
    amax = np.abs(x.reshape(64, 8, 32)).max(axis=2)
    want = np.array([[_brute_shared_exp(float(a)) for a in row] for row in amax])
    assert np.array_equal(s.astype(np.int64) - 127, want)
    # the scale code is the e8m0 encoding of 2^e (torch's float8_e8m0fnu cast)
    pw = torch.tensor(np.ldexp(1.0, want).astype(np.float32))
    assert np.array_equal(pw.to(torch.float8_e8m0fnu).view(torch.uint8).numpy(), s)


def test_elements_match_torch_e4m3_cast_when_the_scale_is_one():
    """Blocks whose amax is 256 have shared exponent 0 (scale 1): every other element is
    encoded as itself -- all bf16 values in [-256, 256], ties included, against torch's cast."""
    pats = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    vals = pats[torch.isfinite(pats) & (pats.abs() <= 256)]
    per = 31
    n = -(-vals.numel() // per)
    vals = torch.cat([vals, torch.zeros(n * per - vals.numel())])
    grid = torch.cat([torch.full((n, 1), 256.0), vals.view(n, per)], dim=1)
    q, s = MX.mxfp8_quant(_bf16(grid.numpy()))
    assert np.all(s == 127)
    want = grid.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want)


def test_closed_forms():
    one = np.zeros((1, 32), np.float32)
    one[0, 0] = 1.0  # amax 1 -> e = -8, 1 / 2^-8 = 256 -> e4m3 0x78
    q, s = MX.mxfp8_quant_f32(one)
    assert s[0, 0] == 127 - 8 and q[0, 0] == 0x78 and np.all(q[0, 1:] == 0)
    sat = np.full((1, 32), 1.999, np.float32)  # e = -8: 1.999 * 256 = 511.7 saturates to 448
    q, s = MX.mxfp8_quant_f32(sat)
    assert s[0, 0] == 119 and np.all(q == 0x7E)
    neg = -sat
    q, _ = MX.mxfp8_quant_f32(neg)
    assert np.all(q == 0xFE)
    q, s = MX.mxfp8_quant_f32(np.zeros((2, 64), np.float32))
    assert np.all(s == 0) and np.all(q == 0)
    const = np.full((1, 32), 300.0, np.float32)  # e = 0: 300 -> nearest e4m3 is 288
    q, s = MX.mxfp8_quant_f32(const)
    assert s[0, 0] == 127 and np.all(C.e4m3_decode(q) == 288.0)


def test_rounding_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((128, 512)).astype(np.float32) * 3
    q, s = MX.mxfp8_quant_f32(x)
    X = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    v = x / X
    dec = C.e4m3_decode(q)
    sat = np.abs(v) > 448
    assert np.all(dec[sat] == np.sign(v[sat]) * 448)
    # half an e4m3 ulp at |v|: ulp = 2^(floor(log2|v|) - 3) for normals, 2^-9 below 2^-6
    av = np.abs(v[~sat])
    ulp = np.where(av >= 2.0 ** -6, np.ldexp(1.0, MX._floor_log2(np.maximum(av, 2.0 ** -6)) - 3), 2.0 ** -9)
    assert np.all(np.abs(dec[~sat] - v[~sat]) <= ulp / 2)


def test_mx_linear_brute_force_loops():
    rng = np.random.default_rng(2)
    M, N, K = 3, 5, 64
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0  # no NaN codes
    sa = rng.integers(120, 135, (M, K // 32)).astype(np.uint8)
    for fmt in ("e4m3", "e2m1"):
        if fmt == "e4m3":
            qw = rng.integers(0, 256, (N, K)).astype(np.uint8)
            qw[(qw & 0x7F) == 0x7F] = 0
        else:
            qw = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
        sw = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
        got = MX.mx_linear_f32(qa, sa, qw, sw, fmt)
        for m in range(M):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    a = C.e4m3_value(int(qa[m, k])) * math.ldexp(1.0, int(sa[m, k // 32]) - 127)
                    if fmt == "e4m3":
                        wv = C.e4m3_value(int(qw[n, k]))
                    else:
                        byte = int(qw[n, k // 2])
                        wv = C.e2m1_value(byte & 0xF if k % 2 == 0 else byte >> 4)
                    acc += a * wv * math.ldexp(1.0, int(sw[n, k // 32]) - 127)
                assert got[m, n] == np.float32(acc), (fmt, m, n)


def test_mx_linear_closed_form():
    """A = 1.0 everywhere with activation scale 2^k, W = 1.0 (e2m1 code 2, both nibbles) with
    weight scale 2^j: every output is K * 2^(k + j)."""
    M, N, K = 4, 3, 128
    for k, j in ((0, 0), (3, -5), (-20, 7)):
        qa = np.full((M, K), 0x38, np.uint8)  # e4m3 1.0
        sa = np.full((M, K // 32), 127 + k, np.uint8)
        qw = np.full((N, K // 2), 0x22, np.uint8)  # e2m1 1.0 in both nibbles
        sw = np.full((N, K // 32), 127 + j, np.uint8)
        out = C.bf16_to_f32(MX.mx_linear(qa, sa, qw, sw, "e2m1"))
        assert np.all(out == np.float32(K * 2.0 ** (k + j)))


def test_mx_linear_equals_the_other_oracle_gemms_where_they_coincide():
    rng = np.random.default_rng(3)
    M, N, K = 6, 40, 256
    x = rng.standard_normal((M, K)).astype(np.float32)
    qa, sa = MX.mxfp8_quant_f32(x)
    # e4m3 weights, every scale code 127 (1.0): the block-FP8 oracle with unit scales
    qw = (rng.standard_normal((N, K)) * 30).clip(-448, 448)
    qw = C.e4m3_encode(qw.astype(np.float32))
    ones_a = np.ones((M, K // 128), np.float32)
    ones_w = np.ones((N, K // 128), np.float32)
    unit_sa = np.full_like(sa, 127)
    got = MX.mx_linear_f32(qa, unit_sa, qw, np.full((N, K // 32), 127, np.uint8), "e4m3")
    want = D.block_fp8_linear_f32(qa, ones_a, qw, ones_w, 1)
    assert np.array_equal(got, want)
    # MXFP4 weights: the MoE oracle's MXFP4 dequantisation and stage product
    pw = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sw = rng.integers(118, 124, (N, K // 32)).astype(np.uint8)
    a32 = MX.dequant_mx(qa, sa, "e4m3")
    want = OM.stage2_rows(a32, OM.dequant_mxfp4_expert(pw, sw))
    assert np.array_equal(MX.mx_linear_f32(qa, sa, pw, sw, "e2m1"), want)
    # bf16 input path = quantise then the linear
    xb = _bf16(x)
    assert np.array_equal(MX.mx_linear_bf16(xb, pw, sw, "e2m1"),
                          MX.mx_linear(*MX.mxfp8_quant(xb), pw, sw, "e2m1"))


def test_rejects_ragged_k():
    with pytest.raises(ValueError):
        MX.mxfp8_quant_f32(np.zeros((2, 48), np.float32))
