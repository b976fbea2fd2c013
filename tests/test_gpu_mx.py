"""GPU parity of the MX-scaled path against the oracle (oracle/mx.py).

* mxq_mxfp8_quant: e4m3 codes and e8m0 scales bit for bit (the [1, 32] activation block
  recipe of "SGLang PR 35605 review", implementation item 1, with the OCP MX conversion rule).
* mxq_mx_linear: MXFP8 activations x MXFP8 or MXFP4 weights ("vLLM PR 50949 review", summary
  and implementation item 2: e2m1 + e8m0 per 32) within atol = rtol = 1e-2 of the oracle's
  bf16 result, on ragged shapes, pre-quantised and bf16 input, with bias, at the
  2048 x 2048 x 7168 workload size on sampled rows, with extreme scale codes, and with a
  canary-guarded output.
"""

import numpy as np
import pytest
import torch

from mxfp4_block_scaled_expert_amd import _lib as L
from mxfp4_block_scaled_expert_amd import ops, synth
from oracle import codecs as OC
from oracle import mx as OMX
from tests._util import assert_bf16_close, bf16_bits, bits_to_float, f32, u8, gpu

pytestmark = pytest.mark.gpu


def _check_quant(x: torch.Tensor):
    q, s = ops.mxfp8_quant(x)
    torch.cuda.synchronize()
    q_ref, s_ref = OMX.mxfp8_quant(bf16_bits(x.reshape(-1, x.shape[-1])))
    assert np.array_equal(u8(s).reshape(s_ref.shape), s_ref), "e8m0 scales differ"
    got = u8(q).reshape(q_ref.shape)
    if not np.array_equal(got, q_ref):
        bad = np.argwhere(got != q_ref)[:8]
        raise AssertionError(f"codes differ at {bad.tolist()}: got {got[tuple(bad.T)]} want {q_ref[tuple(bad.T)]}")


@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (64, 2048), (333, 1024), (2048, 2048)])
def test_mxfp8_quant_random(M, K):
    g = torch.Generator(device="cuda").manual_seed(M * 5 + K)
    _check_quant(torch.randn(M, K, generator=g, device=gpu()).to(torch.bfloat16))


def test_mxfp8_quant_wide_range_zero_and_subnormal_blocks():
    g = torch.Generator(device="cuda").manual_seed(8)
    M, K = 64, 1024
    x = torch.randn(M, K, generator=g, device=gpu())
    expo = torch.randint(-120, 120, (M, K // 32, 1), generator=g, device=gpu()).float()
    x = (x.view(M, K // 32, 32) * torch.exp2(expo)).view(M, K)
    x[0, :32] = 0.0
    x[1, :32] = 0.0
    x[1, 5] = -0.0
    x[2, :32] = 1e-39  # bf16 subnormals
    x[3, :64] = 3.0e38  # near the top of the range
    _check_quant(x.to(torch.bfloat16))


def test_mxfp8_quant_every_bf16_value_with_unit_scale():
    """Blocks with amax 256 take scale 2^0: every bf16 value in [-256, 256] is encoded as itself."""
    pats = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    vals = pats[torch.isfinite(pats) & (pats.abs() <= 256)]
    per = 31
    n = -(-vals.numel() // per)
    vals = torch.cat([vals, torch.zeros(n * per - vals.numel())])
    grid = torch.cat([torch.full((n, 1), 256.0), vals.view(n, per)], dim=1)
    _check_quant(grid.to(torch.bfloat16).to(gpu()))


def _oracle_linear(d, x=None, rows=None):
    xb = bf16_bits(d["x"] if x is None else x)
    if rows is not None:
        xb = xb[rows]
    bias = None if d["bias"] is None else f32(d["bias"].float())
    return OMX.mx_linear_bf16(xb, u8(d["w"]), u8(d["sw"]), d["w_format"], bias)


@pytest.mark.parametrize("w_format", ["e2m1", "e4m3"])
@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (17, 300, 256), (130, 520, 384), (257, 640, 512),
                                   (300, 136, 1152)])
def test_mx_linear_ragged_shapes(M, N, K, w_format):
    d = synth.mx_linear(M, N, K, seed=M + N + K, device=gpu(), w_format=w_format, bias_dtype=torch.float32)
    out = ops.mx_linear(d["x"], d["w"], d["sw"], w_format, bias=d["bias"])
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_linear(d), what=f"mx {w_format} {M}x{N}x{K}")


@pytest.mark.parametrize("seed", range(8))
def test_mx_linear_random_shapes(seed):
    """Seeded random MX linear shapes (M 1..600 on the 128-row tiles, N 8..1024, K a
    multiple of 128 up to 1536, MXFP4 or MXFP8 weights, with and without bias) against the
    oracle."""
    rng = np.random.default_rng(700 + seed)
    M = int(rng.integers(1, 601))
    N = int(rng.integers(1, 129)) * 8
    K = int(rng.integers(1, 13)) * 128
    w_format = ["e2m1", "e4m3"][seed % 2]
    d = synth.mx_linear(M, N, K, seed=seed + 21, device=gpu(), w_format=w_format,
                        bias_dtype=torch.float32 if seed % 3 else None)
    out = ops.mx_linear(d["x"], d["w"], d["sw"], w_format, bias=d["bias"])
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_linear(d), what=f"random mx {w_format} {M}x{N}x{K}")


@pytest.mark.parametrize("w_format", ["e2m1", "e4m3"])
@pytest.mark.parametrize("shape", [(300, 520, 384), (2100, 4000, 256)])
def test_mx_linear_tile_rows_from_the_grid(shape, w_format):
    """128-row tiles wherever their grid fits the GPU in one round (300 x 520: three row tiles,
    the last ragged, and an 8-column last tile), 256-row tiles otherwise (2100 x 4000: a 52-row
    last row tile and a 160-column last tile); each against the oracle."""
    M, N, K = shape
    d = synth.mx_linear(M, N, K, seed=M + N, device=gpu(), w_format=w_format, bias_dtype=torch.float32)
    out = ops.mx_linear(d["x"], d["w"], d["sw"], w_format, bias=d["bias"])
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_linear(d), what=f"mx {w_format} {M}x{N}x{K}")


@pytest.mark.parametrize("w_format", ["e2m1", "e4m3"])
@pytest.mark.parametrize("shape,split", [((300, 520, 4096), 8), ((100, 1000, 7168), 8), ((32, 4096, 3072), 4)])
def test_mx_linear_few_tiles_k_split(shape, split, w_format):
    """MX linears on few tiles with K >= 3072: each tile's K range runs as chunks writing fp32
    partial sums (the bias on the first only), added in chunk order: ragged rows and columns;
    against the oracle."""
    M, N, K = shape
    lib = L.load()
    part = lib.mxq_mx_linear_workspace_size(M, N, K, L.MXQ_DTYPE_E4M3)
    assert part == (4 * split * M * N + 255) // 256 * 256
    d = synth.mx_linear(M, N, K, seed=M + N + K, device=gpu(), w_format=w_format, bias_dtype=torch.float32)
    out = ops.mx_linear(d["x"], d["w"], d["sw"], w_format, bias=d["bias"])
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_linear(d), what=f"mx split {w_format} {M}x{N}x{K}")


@pytest.mark.parametrize("w_format", ["e2m1", "e4m3"])
def test_mx_linear_prequantised_bf16_bias_and_3d(w_format):
    d = synth.mx_linear(34, 384, 640, seed=9, device=gpu(), w_format=w_format, bias_dtype=torch.bfloat16)
    q, s = ops.mxfp8_quant(d["x"])
    out_q = ops.mx_linear(q, d["w"], d["sw"], w_format, input_scale=s, bias=d["bias"])
    out_b = ops.mx_linear(d["x"].view(2, 17, 640), d["w"], d["sw"], w_format, bias=d["bias"])
    torch.cuda.synchronize()
    assert out_b.shape == (2, 17, 384)
    assert torch.equal(out_q.view(torch.int16), out_b.view(34, 384).view(torch.int16))
    assert_bf16_close(bf16_bits(out_q), _oracle_linear(d), what=f"prequantised {w_format}")


@pytest.mark.parametrize("w_format", ["e2m1", "e4m3"])
def test_mx_linear_workload_size_sampled_rows(w_format):
    M, K, N = 2048, 2048, 7168
    d = synth.mx_linear(M, N, K, seed=1006, device=gpu(), w_format=w_format)
    out = ops.mx_linear(d["x"], d["w"], d["sw"], w_format)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 255, 256, 1000, 1023, 1024, 2046, 2047])
    assert_bf16_close(bf16_bits(out[torch.from_numpy(rows).to(gpu())]), _oracle_linear(d, rows=rows),
                      what=f"2048x2048x7168 {w_format} sampled rows")


@pytest.mark.parametrize("codes", [(1, 20), (230, 245)])
def test_mx_linear_extreme_weight_scales(codes):
    """Weight scale codes near both ends of e8m0 (2^-126 .. 2^-107, 2^103 .. 2^118; e2m1 values
    up to 6 stay finite): the output is compared at its own scale (both sides multiplied by the
    power of two that brings the reference's largest magnitude near 1, exact for these values)."""
    M, N, K = 40, 256, 512
    g = torch.Generator().manual_seed(sum(codes))
    x = (torch.randn(M, K, generator=g)).to(torch.bfloat16).to(gpu())
    w = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.int32).to(torch.uint8).to(gpu())
    sw = torch.randint(codes[0], codes[1] + 1, (N, K // 32), generator=g, dtype=torch.int32).to(torch.uint8).to(gpu())
    out = ops.mx_linear(x, w, sw, "e2m1")
    torch.cuda.synchronize()
    want = OMX.mx_linear_bf16(bf16_bits(x), u8(w), u8(sw), "e2m1")
    gv = bits_to_float(bf16_bits(out)).astype(np.float64)
    wv = bits_to_float(want).astype(np.float64)
    assert np.all(np.isfinite(gv)) and np.all(np.isfinite(wv))
    k = -int(np.floor(np.log2(np.abs(wv).max())))
    gs, ws = np.ldexp(gv, k), np.ldexp(wv, k)
    assert not np.any(np.abs(gs - ws) > 1e-2 + 1e-2 * np.abs(ws))


def test_mx_linear_writes_only_its_output_and_refuses_bad_arguments():
    lib = L.load()
    M, N, K = 130, 300, 256
    d = synth.mx_linear(M, N, K, seed=3, device=gpu(), w_format="e2m1")
    ref = ops.mx_linear(d["x"], d["w"], d["sw"], "e2m1")
    ldo = N + 20
    canary = 0x7FBF
    buf = torch.full(((M + 6) * ldo,), np.int16(np.uint16(canary).view(np.int16)), dtype=torch.int16, device=gpu())
    out = buf.view(M + 6, ldo)[3:3 + M, :N].view(torch.bfloat16)
    n = lib.mxq_mx_linear_workspace_size(M, N, K, L.MXQ_DTYPE_BF16)
    ws = torch.empty(n, dtype=torch.uint8, device=gpu())
    sh = torch.cuda.current_stream().cuda_stream
    assert lib.mxq_mx_linear(d["x"].data_ptr(), L.MXQ_DTYPE_BF16, None, M, K, K, d["w"].data_ptr(), L.MXQ_DTYPE_E2M1,
                             N, d["sw"].data_ptr(), None, 0, out.data_ptr(), ldo, ws.data_ptr(), n, sh) == 0
    torch.cuda.synchronize()
    b = buf.view(M + 6, ldo).cpu().numpy().view(np.uint16)
    mask = np.ones(b.shape, bool)
    mask[3:3 + M, :N] = False
    assert np.all(b[mask] == canary), "canary overwritten"
    assert torch.equal(out.contiguous().view(torch.int16), ref.view(torch.int16))
    # K % 128, unknown weight format, small workspace
    assert lib.mxq_mx_linear(d["x"].data_ptr(), L.MXQ_DTYPE_BF16, None, M, 96, 96, d["w"].data_ptr(),
                             L.MXQ_DTYPE_E2M1, N, d["sw"].data_ptr(), None, 0, out.data_ptr(), ldo, ws.data_ptr(), n,
                             sh) == L.MXQ_ERR_SHAPE
    assert lib.mxq_mx_linear(d["x"].data_ptr(), L.MXQ_DTYPE_BF16, None, M, K, K, d["w"].data_ptr(), L.MXQ_DTYPE_F32,
                             N, d["sw"].data_ptr(), None, 0, out.data_ptr(), ldo, ws.data_ptr(), n, sh) == L.MXQ_ERR_DTYPE
    assert lib.mxq_mx_linear(d["x"].data_ptr(), L.MXQ_DTYPE_BF16, None, M, K, K, d["w"].data_ptr(), L.MXQ_DTYPE_E2M1,
                             N, d["sw"].data_ptr(), None, 0, out.data_ptr(), ldo, ws.data_ptr(), n - 1,
                             sh) == L.MXQ_ERR_WORKSPACE
