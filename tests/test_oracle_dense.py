"""Pins for the oracle dense GEMMs: closed forms on exact inputs, torch
float64 matmul on torch-decoded operands, and the invariants the pages state
(per-tensor scale == block scale with all blocks equal; scale layout changes
are bit-identical)."""

import numpy as np
import torch

from oracle import codecs as C
from oracle import dense as D
from oracle.quant import per_token_group_quant_fp8


def _bf16(x) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _tdec(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double()


def _ulp32(x: np.ndarray) -> np.ndarray:
    x = np.abs(np.asarray(x, np.float32))
    return np.nextafter(x, np.float32(np.inf)) - x


def test_per_tensor_closed_form():
    M, N, K = 5, 7, 576
    a = _bf16(np.ones((M, K)))
    w = np.full((N, K), 0x38, np.uint8)  # 1.0
    out = D.fp8_scaled_mm(a, w, 0.125)
    assert np.all(C.bf16_to_f32(out) == K / 8)
    bias = np.arange(N, dtype=np.float32)
    out = D.fp8_scaled_mm(a, w, 0.125, bias)
    assert np.array_equal(C.bf16_to_f32(out), np.broadcast_to(K / 8 + bias, (M, N)).astype(np.float32))


def test_per_tensor_identity_weight_returns_input():
    rng = np.random.default_rng(0)
    K = 64
    a = _bf16(rng.standard_normal((9, K)))
    w = np.zeros((K, K), np.uint8)
    np.fill_diagonal(w, 0x38)
    out = D.fp8_scaled_mm(a, w, 1.0)
    assert np.array_equal(out, a)


def test_per_tensor_vs_torch_float64():
    rng = np.random.default_rng(1)
    M, N, K = 11, 224, 576
    a = _bf16(rng.standard_normal((M, K)) / 10)
    w = torch.randn(N, K, generator=torch.Generator().manual_seed(1)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bias = rng.standard_normal(N).astype(np.float32)
    got = D.fp8_scaled_mm_f32(a, w, 0.01, bias)
    at = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).double()
    ref = ((at @ _tdec(w).T).float() * 0.01 + torch.from_numpy(bias)).numpy()
    assert np.all(np.abs(got - ref) <= 2 * _ulp32(ref))


def test_block_linear_vs_torch_float64_both_recipes():
    rng = np.random.default_rng(2)
    M, N, K = 17, 384, 512
    x = _bf16(rng.standard_normal((M, K)))
    qa, sa = per_token_group_quant_fp8(x)
    w = torch.randn(N, K, generator=torch.Generator().manual_seed(2)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for block_n in (128, 1):
        sw = (rng.random((N // block_n, K // 128)) + 0.1).astype(np.float32)
        bias = rng.standard_normal(N).astype(np.float32)
        got = D.block_fp8_linear_f32(qa, sa, w, sw, block_n, bias)
        a_t = (_tdec(qa).float() * torch.from_numpy(sa).repeat_interleave(128, 1)).double()
        swe = torch.from_numpy(sw).repeat_interleave(block_n, 0).repeat_interleave(128, 1)
        w_t = (_tdec(w).float() * swe).double()
        ref = ((a_t @ w_t.T).float() + torch.from_numpy(bias)).numpy()
        assert np.all(np.abs(got - ref) <= 2 * _ulp32(ref)), block_n


def test_block_grid_n_ceil_and_tail_rows():
    # N not a multiple of 128: the last scale-grid row covers the tail rows
    rng = np.random.default_rng(3)
    M, N, K = 4, 200, 256
    qa = rng.integers(0, 0x7F, size=(M, K)).astype(np.uint8)
    sa = np.full((M, 2), 1.0, np.float32)
    w = np.full((N, K), 0x38, np.uint8)
    sw = np.array([[1.0, 1.0], [2.0, 2.0]], np.float32)
    out = D.block_fp8_linear_f32(qa, sa, w, sw, 128)
    assert np.array_equal(out[:, 128:], 2 * out[:, :72])


def test_per_tensor_equals_block_scale_with_equal_blocks():
    rng = np.random.default_rng(4)
    M, N, K = 13, 256, 512
    a = _bf16(rng.standard_normal((M, K)) / 10)
    w = torch.randn(N, K, generator=torch.Generator().manual_seed(4)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bias = rng.standard_normal(N).astype(np.float32)
    for s in (0.0078125, 0.25):  # powers of two: both forms are exact up to the same rounding
        per_tensor = D.fp8_scaled_mm(a, w, s, bias)
        grid = np.full((N // 128, K // 128), s, np.float32)
        block = C.f32_to_bf16(D.w8a16_block_linear_f32(a, w, grid, 128, bias))
        assert np.array_equal(per_tensor, block)
    # a general scale: the block form rounds each dec(w) * s to fp32, so the two
    # agree to within 2^-24 of sum |a * w * s| plus the final fp32 roundings
    s = np.float32(0.01)
    pt = D.fp8_scaled_mm_f32(a, w, s, None)
    bl = D.w8a16_block_linear_f32(a, w, np.full((2, 4), s, np.float32), 128, None)
    at = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).double()
    mag = ((at.abs() @ _tdec(w).abs().T) * float(s)).numpy()
    assert np.all(np.abs(pt - bl) <= 2.0 ** -24 * mag + 2 * _ulp32(pt))


def test_block_n_1_with_repeated_rows_equals_128x128():
    rng = np.random.default_rng(5)
    M, N, K = 8, 256, 256
    qa = rng.integers(0, 0x7F, size=(M, K)).astype(np.uint8)
    sa = (rng.random((M, 2)) + 0.5).astype(np.float32)
    w = rng.integers(0, 0x7F, size=(N, K)).astype(np.uint8)
    sw = (rng.random((2, 2)) + 0.1).astype(np.float32)
    a = D.block_fp8_linear(qa, sa, w, sw, 128)
    b = D.block_fp8_linear(qa, sa, w, np.repeat(sw, 128, axis=0), 1)
    assert np.array_equal(a, b)
    # a transposed-storage copy of the grid (same logical values) is bit-identical
    c = D.block_fp8_linear(qa, sa, w, np.asfortranarray(sw), 128)
    assert np.array_equal(a, c)


def test_row_independence():
    rng = np.random.default_rng(6)
    x = _bf16(rng.standard_normal((9, 256)))
    w = rng.integers(0, 0x7F, size=(128, 256)).astype(np.uint8)
    sw = np.ones((1, 2), np.float32)
    full = D.block_fp8_linear_bf16(x, w, sw, 128)
    part = D.block_fp8_linear_bf16(x[4:6], w, sw, 128)
    assert np.array_equal(full[4:6], part)


# ---- batched per-tensor W8A16 (the MLA-style batched FP8 GEMM)

def test_bmm_closed_form_per_entry_scales_and_biases():
    """A = 1, W = 1.0: entry z is K * 2^-z + bias[z] exactly (small integers, exact in bf16)."""
    B, M, N, K = 4, 3, 5, 64
    a = _bf16(np.ones((B, M, K)))
    w = np.full((B, N, K), 0x38, np.uint8)
    scales = np.array([2.0 ** -z for z in range(B)], np.float32)
    bias = np.arange(B * N, dtype=np.float32).reshape(B, N)
    got = C.bf16_to_f32(D.fp8_scaled_bmm(a, w, scales, bias))
    want = (K * scales)[:, None, None] + bias[:, None, :]
    assert np.array_equal(got, np.broadcast_to(want, (B, M, N)).astype(np.float32))


def test_bmm_vs_torch_bmm_float64():
    """The batched definition against torch.bmm of torch-decoded operands (within 2 fp32 ulps
    before the bf16 rounding): catches a transposed operand or a scale applied to the wrong entry."""
    rng = np.random.default_rng(7)
    B, M, N, K = 3, 17, 96, 512
    a = _bf16(rng.standard_normal((B, M, K)) / 10)
    w = torch.randn(B, N, K, generator=torch.Generator().manual_seed(7)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scales = np.array([0.01, 0.5, 3.0], np.float32)
    bias = rng.standard_normal((B, N)).astype(np.float32)
    got = D.fp8_scaled_bmm_f32(a, w, scales, bias)
    at = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).double()
    prod = torch.bmm(at, _tdec(w).transpose(1, 2).contiguous()).float()
    ref = (prod * torch.from_numpy(scales)[:, None, None] + torch.from_numpy(bias)[:, None, :]).numpy()
    assert np.all(np.abs(got - ref) <= 2 * _ulp32(ref))


def test_bmm_entries_are_independent_and_match_the_2d_product():
    rng = np.random.default_rng(8)
    B, M, N, K = 3, 4, 32, 64
    a = _bf16(rng.standard_normal((B, M, K)))
    w = rng.integers(0, 256, (B, N, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38  # no NaN codes
    scales = np.array([0.25, 1.5, 0.03125], np.float32)
    full = D.fp8_scaled_bmm(a, w, scales)
    perm = np.array([2, 0, 1])
    assert np.array_equal(D.fp8_scaled_bmm(a[perm], w[perm], scales[perm]), full[perm])
    for z in range(B):
        assert np.array_equal(full[z], D.fp8_scaled_mm(a[z], w[z], scales[z]))
