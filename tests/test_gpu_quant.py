"""GPU parity of per_token_group_quant_fp8 against the oracle: codes and
scales bit for bit ("SGLang PR 35605 review", implementation item 1 -- the
1x128 per-token activation quantisation)."""

import numpy as np
import pytest
import torch

from mxfp4_block_scaled_expert_amd import ops
from oracle.quant import per_token_group_quant_fp8 as oracle_quant
from tests._util import bf16_bits, u8, f32, gpu

pytestmark = pytest.mark.gpu


def _check(x: torch.Tensor):
    q, s = ops.per_token_group_quant_fp8(x)
    torch.cuda.synchronize()
    xb = bf16_bits(x.reshape(-1, x.shape[-1]))
    q_ref, s_ref = oracle_quant(xb)
    q_got = u8(q).reshape(q_ref.shape)
    s_got = f32(s).reshape(s_ref.shape)
    assert np.array_equal(s_got.view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    if not np.array_equal(q_got, q_ref):
        bad = np.argwhere(q_got != q_ref)[:8]
        raise AssertionError(f"codes differ at {bad.tolist()}: got {q_got[tuple(bad.T)]} want {q_ref[tuple(bad.T)]}")


@pytest.mark.parametrize("M,K", [(1, 128), (7, 256), (64, 2048), (333, 1024), (2048, 2048), (96, 7168)])
def test_random_shapes(M, K):
    g = torch.Generator(device="cuda").manual_seed(M * 7 + K)
    x = torch.randn(M, K, generator=g, device=gpu()).to(torch.bfloat16)
    _check(x)


def test_groups_with_wide_dynamic_range():
    g = torch.Generator(device="cuda").manual_seed(5)
    M, K = 64, 1024
    x = torch.randn(M, K, generator=g, device=gpu())
    expo = torch.randint(-30, 30, (M, K // 128, 1), generator=g, device=gpu()).float()
    x = (x.view(M, K // 128, 128) * torch.exp2(expo)).view(M, K).to(torch.bfloat16)
    _check(x)


def test_every_bf16_value_with_unit_scale():
    # groups whose amax is 448 get s == 1 exactly, so every other element is
    # encoded as itself: sweeps every bf16 value in [-448, 448], ties included
    pats = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    vals = pats[torch.isfinite(pats) & (pats.abs() <= 448)]
    per = 127
    n = -(-vals.numel() // per)
    vals = torch.cat([vals, torch.zeros(n * per - vals.numel())])
    grid = torch.cat([torch.full((n, 1), 448.0), vals.view(n, per)], dim=1)
    x = grid.to(torch.bfloat16).to(gpu())
    _check(x)


def test_every_bf16_value_with_non_power_of_two_scales():
    """Group maxima 448, 450, ..., 510 (scales 1 .. 1.138, long mantissas) against every bf16
    value in [-448, 448]: the quotients land all over the e4m3 grid, some within a few fp32
    ulps of its rounding midpoints, where the codes must still be those of the division."""
    pats = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    vals = pats[torch.isfinite(pats) & (pats.abs() <= 448)]
    per = 127
    n = -(-vals.numel() // per)
    vals = torch.cat([vals, torch.zeros(n * per - vals.numel())]).view(n, per)
    rows = []
    for amax in range(448, 512, 2):
        rows.append(torch.cat([torch.full((n, 1), float(amax)), vals], dim=1))
    x = torch.cat(rows).to(torch.bfloat16).to(gpu())
    _check(x)


def test_zero_negative_zero_and_constant_groups():
    x = torch.zeros(4, 512)
    x[0, 5] = -0.0
    x[1, :128] = 3.5
    x[1, 128:256] = -0.25
    x[2, 256:384] = 1e-30
    x[3] = -1e-39  # bf16 subnormal input
    _check(x.to(torch.bfloat16).to(gpu()))


def test_strided_rows_and_3d_input():
    g = torch.Generator(device="cuda").manual_seed(9)
    big = torch.randn(48, 1024, generator=g, device=gpu()).to(torch.bfloat16)
    _check(big[:, :512])  # row stride 1024 > K
    x3 = torch.randn(3, 5, 256, generator=g, device=gpu()).to(torch.bfloat16)
    q, s = ops.per_token_group_quant_fp8(x3)
    assert q.shape == (3, 5, 256) and s.shape == (3, 5, 2)
    _check(x3)


def test_empty_input():
    x = torch.empty(0, 256, dtype=torch.bfloat16, device=gpu())
    q, s = ops.per_token_group_quant_fp8(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)
