"""Pins of the plain C++ oracle (oracle/cpp/oracle.cpp, loops with double accumulation)
against the numpy oracle (an independent implementation of the same definitions), torch's
e4m3 cast and closed forms.

The two oracles sum in different orders (sequential loops vs BLAS), both in float64, so their
fp32 results may differ by at most one fp32 unit in the last place and their bf16 outputs
agree except where such an ulp straddles a bf16 rounding midpoint."""

import numpy as np
import pytest
import torch

from oracle import codecs as OC
from oracle import cref as CR
from oracle import dense as OD
from oracle import moe as OM
from oracle.cbuild import build
from oracle.quant import per_token_group_quant_fp8


@pytest.fixture(scope="module", autouse=True)
def _built():
    build(verbose=False)


def _bf16(a) -> np.ndarray:
    return OC.f32_to_bf16(np.asarray(a, np.float32))


def _ulp_close(a, b):
    """Every pair within one fp32 unit in the last place of the larger magnitude."""
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    return bool(np.all(np.abs(a - b) <= np.spacing(np.maximum(np.abs(a), np.abs(b)))))


def test_e4m3_table_matches_torch():
    t = CR.e4m3_table()
    want = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    finite = np.isfinite(want)
    assert np.array_equal(t[finite], want[finite]) and np.all(np.isnan(t[~finite]))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(200000) * np.exp2(rng.integers(-60, 60, 200000))).astype(np.float32)
    v[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]  # exact ties
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(CR.f32_to_bf16(v), want)


def test_quant_matches_numpy_oracle_bit_for_bit():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 1024)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, (50, 8))).repeat(128, axis=1)
    x[0, :128] = 0.0
    xb = _bf16(x)
    q, s = CR.quant_1x128(xb)
    q2, s2 = per_token_group_quant_fp8(xb)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32)) and np.array_equal(q, q2)


def test_quant_every_bf16_value_with_unit_scale_matches_torch():
    pats = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    vals = pats[torch.isfinite(pats) & (pats.abs() <= 448)]
    per = 127
    n = -(-vals.numel() // per)
    vals = torch.cat([vals, torch.zeros(n * per - vals.numel())])
    grid = torch.cat([torch.full((n, 1), 448.0), vals.view(n, per)], dim=1)
    q, s = CR.quant_1x128(_bf16(grid.numpy()))
    assert np.all(s == 1.0)
    assert np.array_equal(q, grid.to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_dense_gemms_match_numpy_oracle():
    rng = np.random.default_rng(2)
    M, N, K = 33, 200, 384
    a = _bf16(rng.standard_normal((M, K)) / 10)
    w = OC.e4m3_encode(np.clip(rng.standard_normal((N, K)) * 50, -448, 448).astype(np.float32))
    bias = rng.standard_normal(N).astype(np.float32)
    got = CR.fp8_scaled_mm_f32(a, w, 0.01, bias)
    want = OD.fp8_scaled_mm_f32(a, w, 0.01, bias)
    assert _ulp_close(got, want)
    qa, sa = per_token_group_quant_fp8(_bf16(rng.standard_normal((M, K))))
    for bn in (128, 1):
        sw = (rng.random((-(-N // bn), K // 128)) + 0.1).astype(np.float32) * 1e-3
        got = CR.block_fp8_linear_f32(qa, sa, w, sw, bn, bias)
        want = OD.block_fp8_linear_f32(qa, sa, w, sw, bn, bias)
        assert _ulp_close(got, want)
        b16 = CR.f32_to_bf16(got)
        assert np.mean(b16 == OC.f32_to_bf16(want)) > 0.999


def test_dense_closed_form():
    """A = 1, W = 1.0 (0x38), per-tensor scale 2^-3: every output is K / 8 exactly."""
    M, N, K = 5, 7, 256
    a = _bf16(np.ones((M, K)))
    w = np.full((N, K), 0x38, np.uint8)
    assert np.all(CR.fp8_scaled_mm_f32(a, w, 0.125) == K / 8)


def _moe_inputs(rng, M, E, topk, H, I, mx=False):
    x = _bf16(rng.standard_normal((M, H)))
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(M)]).astype(np.int32)
    wts = rng.random((M, topk)).astype(np.float32)
    if mx:
        w1 = rng.integers(0, 256, (E, 2 * I, H // 2)).astype(np.uint8)
        w2 = rng.integers(0, 256, (E, H, I // 2)).astype(np.uint8)
        s1 = rng.integers(118, 123, (E, 2 * I, H // 32)).astype(np.uint8)
        s2 = rng.integers(118, 123, (E, H, I // 32)).astype(np.uint8)
    else:
        w1 = OC.e4m3_encode(np.clip(rng.standard_normal((E, 2 * I, H)) * 60, -448, 448).astype(np.float32))
        w2 = OC.e4m3_encode(np.clip(rng.standard_normal((E, H, I)) * 60, -448, 448).astype(np.float32))
        s1 = (rng.random((E, -(-2 * I // 128), H // 128)) * 1e-3 + 5e-4).astype(np.float32)
        s2 = (rng.random((E, -(-H // 128), I // 128)) * 1e-3 + 5e-4).astype(np.float32)
    b1 = rng.standard_normal((E, 2 * I)).astype(np.float32)
    return x, ids, wts, w1, s1, w2, s2, b1


@pytest.mark.parametrize("act_quant", [False, True])
def test_fused_moe_fp8_matches_numpy_oracle(act_quant):
    rng = np.random.default_rng(3 + act_quant)
    x, ids, wts, w1, s1, w2, s2, b1 = _moe_inputs(rng, 20, 6, 2, 256, 256)
    got = CR.fused_moe_fp8(x, ids, wts, w1, s1, w2, s2, b1, act_quant)
    want = OM.fused_moe_fp8(x, ids, wts, w1, s1, w2, s2, b1, act_quant)
    # same definition, same rounding points: identical except for rare ulp-level order effects
    assert np.mean(got == want) > 0.99
    g, w = OC.bf16_to_f32(got), OC.bf16_to_f32(want)
    assert np.all(np.abs(g - w) <= 1e-2 + 1e-2 * np.abs(w))


def test_fused_moe_mxfp4_matches_numpy_oracle():
    rng = np.random.default_rng(5)
    x, ids, wts, w1, s1, w2, s2, b1 = _moe_inputs(rng, 12, 5, 3, 320, 192, mx=True)
    got = CR.fused_moe_mxfp4(x, ids, wts, w1, s1, w2, s2, b1)
    want = OM.fused_moe_mxfp4(x, ids, wts, w1, s1, w2, s2, b1)
    assert np.mean(got == want) > 0.99
    g, w = OC.bf16_to_f32(got), OC.bf16_to_f32(want)
    assert np.all(np.abs(g - w) <= 1e-2 + 1e-2 * np.abs(w))


def test_fused_moe_single_expert_topk1_is_two_dense_gemms():
    """E = 1, top-1, weight 1, W8A8: the C MoE equals the C oracle's own block linear twice --
    quantise x, stage 1, bf16, SiLU-and-mul, bf16, quantise, stage 2, bf16 -- bit for bit."""
    rng = np.random.default_rng(6)
    x, ids, wts, w1, s1, w2, s2, _ = _moe_inputs(rng, 9, 1, 1, 256, 128)
    ids[:] = 0
    wts[:] = 1.0
    got = CR.fused_moe_fp8(x, ids, wts, w1, s1, w2, s2, None, True)
    qx, sx = CR.quant_1x128(x)
    ic0 = CR.f32_to_bf16(CR.block_fp8_linear_f32(qx, sx, w1[0], s1[0], 128))
    ic1 = OM.silu_mul_bf16(OC.bf16_to_f32(ic0), 128)
    q1, sq1 = CR.quant_1x128(ic1)
    want = CR.f32_to_bf16(CR.block_fp8_linear_f32(q1, sq1, w2[0], s2[0], 128))
    assert np.array_equal(got, want)


def test_bad_expert_id_is_refused():
    rng = np.random.default_rng(7)
    x, ids, wts, w1, s1, w2, s2, b1 = _moe_inputs(rng, 4, 3, 1, 128, 128)
    ids[0, 0] = 3
    with pytest.raises(ValueError):
        CR.fused_moe_fp8(x, ids, wts, w1, s1, w2, s2, b1)
