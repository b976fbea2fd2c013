"""GPU parity of the dense linears against the oracle.

* fp8_scaled_mm: the test grid of "SGLang PR 32618 review" (test_gemm.py
  listing: M in {1, 11, 97}, N in {128, 224}, K in {512, 576}, 0-d or [1]
  scale, with and without bias).
* block_fp8_linear: the cases of "SGLang PR 35605 review" (implementation
  item 4 and the test_xpu_fp8_linear.py listing: M = 1/8/16/17, 2-D and 3-D,
  non-contiguous input, pre-quantised input, both weight recipes, a non-square
  scale grid, and the transposed scale storage giving identical bits), plus the
  2048 x 2048 x 7168 workload on sampled rows.
"""

import json
import os

import numpy as np
import pytest
import torch

from mxfp4_block_scaled_expert_amd import _lib as L
from mxfp4_block_scaled_expert_amd import ops, synth
from oracle import dense as OD
from oracle.quant import per_token_group_quant_fp8 as oracle_quant
from tests._util import assert_bf16_close, bf16_bits, f32, u8, gpu

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_recipes.json")
RECIPES = json.load(open(GOLDEN))
G = RECIPES["per_tensor_w8a16_grid"]


@pytest.mark.parametrize("M", G["M"])
@pytest.mark.parametrize("N", G["N"])
@pytest.mark.parametrize("K", G["K"])
@pytest.mark.parametrize("scale_as_vector", G["scale_as_vector"])
@pytest.mark.parametrize("has_bias", G["has_bias"])
def test_fp8_scaled_mm_page_grid(M, N, K, scale_as_vector, has_bias):
    d = synth.dense_w8a16(M, N, K, seed=M * 1000 + N + K, device=gpu(), has_bias=has_bias, scale=G["scale"])
    scale = d["scale"] if scale_as_vector else d["scale"].reshape(())
    out = ops.fp8_scaled_mm(d["a"], d["w"], scale, d["bias"])
    torch.cuda.synchronize()
    want = OD.fp8_scaled_mm(bf16_bits(d["a"]), u8(d["w"]), float(f32(d["scale"])[0]),
                            None if d["bias"] is None else f32(d["bias"]))
    assert_bf16_close(bf16_bits(out), want, what=f"fp8_scaled_mm {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,stream", [(1, 2048, 7168, True), (5, 998, 4096, True), (16, 2048, 7168, True),
                                          (3, 1024, 16384, True), (9, 4096, 4096, True), (16, 2048, 2048, False),
                                          (32, 1024, 7168, False)])
def test_fp8_scaled_mm_few_rows(M, N, K, stream):
    """Few-row per-tensor W8A16 products with long K run on the weight-streaming kernel (the
    scale applied to each 128-wide K block's partial sum, K split into chunks summed in chunk
    order): one row, ragged rows and a column count that is not a multiple of 4, two row
    tiles, K = 16384 staged a chunk at a time, 128-column tiles; and two neighbours that stay
    on the tiles; each with a bias against the oracle."""
    if stream:
        assert L.load().mxq_fp8_scaled_mm_workspace_size(M, N, K) > 0
    d = synth.dense_w8a16(M, N, K, seed=M + N + K, device=gpu())
    out = ops.fp8_scaled_mm(d["a"], d["w"], d["scale"], d["bias"])
    torch.cuda.synchronize()
    want = OD.fp8_scaled_mm(bf16_bits(d["a"]), u8(d["w"]), float(f32(d["scale"])[0]), f32(d["bias"]))
    assert_bf16_close(bf16_bits(out), want, what=f"fp8_scaled_mm few rows {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,split", [(64, 2048, 7168, 4), (300, 520, 7168, 2), (1, 2048, 7136, 8), (128, 2048, 7168, 2),
                                         (33, 2048, 6144, 4)])
def test_fp8_scaled_mm_ring_k_split(M, N, K, split):
    """Per-tensor products whose ring-fed tiles leave the GPU mostly idle, K >= 6144: each
    tile's K range runs as 2, 4 or 8 chunks writing fp32 partial sums (each scaled), added in
    chunk order by the split-sum kernel: ragged rows and columns, a K that is not a multiple of
    128 (not streamed), a bias on the first chunk only; each against the oracle."""
    part = L.load().mxq_fp8_scaled_mm_workspace_size(M, N, K)
    assert part == (4 * split * M * N + 255) // 256 * 256
    d = synth.dense_w8a16(M, N, K, seed=M + N + K + 1, device=gpu())
    out = ops.fp8_scaled_mm(d["a"], d["w"], d["scale"], d["bias"])
    torch.cuda.synchronize()
    want = OD.fp8_scaled_mm(bf16_bits(d["a"]), u8(d["w"]), float(f32(d["scale"])[0]), f32(d["bias"]))
    assert_bf16_close(bf16_bits(out), want, what=f"fp8_scaled_mm ring split {M}x{N}x{K}")


def test_fp8_scaled_mm_workload_and_bf16_bias_and_3d():
    d = synth.dense_w8a16(97, 224, 576, seed=1, device=gpu())
    x3 = d["a"].view(1, 97, 576)
    out = ops.fp8_scaled_mm(x3, d["w"], d["scale"], d["bias"].to(torch.bfloat16))
    assert out.shape == (1, 97, 224)
    torch.cuda.synchronize()
    bias_b = f32(d["bias"].to(torch.bfloat16))
    want = OD.fp8_scaled_mm(bf16_bits(d["a"]), u8(d["w"]), 0.01, bias_b)
    assert_bf16_close(bf16_bits(out.view(97, 224)), want, what="fp8_scaled_mm bf16 bias")


# ---- batched per-tensor W8A16 (MLA-style per-head products)

def _mm_runs_tiles(M, K):
    """A 2-D per-tensor call of few rows with K a multiple of 128 may run the weight-streaming
    kernel, and one with K >= 4096 may split K on the ring-fed tiles, both grouping the K sums
    differently; otherwise it runs the tiles the batched call uses, bit for bit."""
    return (K % 128 != 0 or M > 64) and K < 4096


def _assert_entry(out_z, ref, d, z, scale_z, bias_z, what):
    """Entry z of a batched call against the 2-D call: bit for bit where both run the tiles,
    else both against the oracle."""
    M, K = ref.shape[0], d["a"].shape[-1]
    if _mm_runs_tiles(M, K):
        assert torch.equal(out_z.view(torch.int16), ref.view(torch.int16)), what
        return
    want = OD.fp8_scaled_mm(bf16_bits(d["a"][z] if d["a"].dim() == 3 else d["a"]), u8(d["w"][z] if d["w"].dim() == 3 else d["w"]),
                            float(f32(scale_z)[0]), None if bias_z is None else f32(bias_z))
    assert_bf16_close(bf16_bits(ref), want, what=what + " (2-D)")
    assert_bf16_close(bf16_bits(out_z), want, what=what + " (batched)")


def _oracle_bmm(d, bias=None):
    B = d["a"].shape[0]
    sc = f32(d["scale"])
    scales = np.broadcast_to(sc, (B,)) if sc.size == 1 else sc
    return OD.fp8_scaled_bmm(bf16_bits(d["a"]), u8(d["w"]), scales, None if bias is None else bias)


# (24, 97, 224, 576): the batch's grid exceeds one workgroup per compute unit, so the batched
# call runs the register-staged tiles while each 2-D reference call runs the ring-fed tiles --
# the two kernels must agree bit for bit
@pytest.mark.parametrize("B,M,N,K", [(4, 97, 224, 576), (16, 1, 128, 512), (3, 130, 200, 512), (2, 33, 128, 96),
                                     (24, 97, 224, 576)])
@pytest.mark.parametrize("per_entry_scale", [True, False])
def test_fp8_scaled_bmm_matches_per_entry_products_and_oracle(B, M, N, K, per_entry_scale):
    d = synth.batched_w8a16(B, M, N, K, seed=B * 7 + M + N + K, device=gpu(), per_entry_scale=per_entry_scale)
    out = ops.fp8_scaled_bmm(d["a"], d["w"], d["scale"], d["bias"])
    torch.cuda.synchronize()
    assert out.shape == (B, M, N)
    for z in range(B):  # every entry is the 2-D product (bit for bit where both run the tiles)
        sz = d["scale"][z if per_entry_scale else 0].reshape(1)
        ref = ops.fp8_scaled_mm(d["a"][z], d["w"][z], sz, d["bias"][z])
        _assert_entry(out[z], ref, d, z, sz, d["bias"][z], f"entry {z}")
    assert_bf16_close(bf16_bits(out), _oracle_bmm(d, f32(d["bias"])), what=f"bmm {B}x{M}x{N}x{K}")


def test_fp8_scaled_bmm_shared_bias_bf16_and_no_bias():
    d = synth.batched_w8a16(5, 40, 256, 512, seed=31, device=gpu())
    shared = d["bias"][0].to(torch.bfloat16)
    out = ops.fp8_scaled_bmm(d["a"], d["w"], d["scale"], shared)
    out0 = ops.fp8_scaled_bmm(d["a"], d["w"], d["scale"])
    torch.cuda.synchronize()
    bias = np.broadcast_to(f32(shared), (5, 256))
    assert_bf16_close(bf16_bits(out), _oracle_bmm(d, bias), what="bmm shared bf16 bias")
    assert_bf16_close(bf16_bits(out0), _oracle_bmm(d), what="bmm no bias")


def test_fp8_scaled_bmm_mla_head_shapes_sampled():
    """DeepSeek MLA-shaped per-head products at full size (128 heads, 64 tokens): the
    absorbed key projection [T, 128] x [512, 128]^T and the value projection [T, 512] x
    [128, 512]^T; every head checked against the oracle on its first and last rows."""
    for (N, K) in [(512, 128), (128, 512)]:
        d = synth.batched_w8a16(128, 64, N, K, seed=N + K, device=gpu(), has_bias=False)
        out = ops.fp8_scaled_bmm(d["a"], d["w"], d["scale"])
        torch.cuda.synchronize()
        rows = [0, 31, 63]
        sub = {"a": d["a"][:, rows], "w": d["w"], "scale": d["scale"]}
        assert_bf16_close(bf16_bits(out[:, rows]), _oracle_bmm(sub), what=f"MLA heads N={N} K={K}")


def test_fp8_scaled_bmm_shared_inputs_through_the_c_abi():
    """Batch stride 0 on A and on W: every entry reads the same operand (documented sharing)."""
    from mxfp4_block_scaled_expert_amd import _lib as L
    lib = L.load()
    d = synth.batched_w8a16(4, 24, 128, 256, seed=51, device=gpu(), has_bias=False)
    B, M, N, K = 4, 24, 128, 256
    out = torch.empty(B, M, N, dtype=torch.bfloat16, device=gpu())
    st = torch.cuda.current_stream().cuda_stream
    # shared A (entry 0), per-entry W
    assert lib.mxq_fp8_scaled_bmm(d["a"].data_ptr(), B, M, K, K, 0, d["w"].data_ptr(), N, N * K, d["scale"].data_ptr(),
                                  1, None, 0, 0, out.data_ptr(), N, M * N, st) == 0
    torch.cuda.synchronize()
    for z in range(B):
        ref = ops.fp8_scaled_mm(d["a"][0], d["w"][z], d["scale"][z].reshape(1))
        _assert_entry(out[z], ref, {"a": d["a"][0], "w": d["w"][z]}, z, d["scale"][z].reshape(1), None,
                      f"shared A, entry {z}")
    # per-entry A, shared W (entry 0) and shared scale
    assert lib.mxq_fp8_scaled_bmm(d["a"].data_ptr(), B, M, K, K, M * K, d["w"].data_ptr(), N, 0, d["scale"].data_ptr(),
                                  0, None, 0, 0, out.data_ptr(), N, M * N, st) == 0
    torch.cuda.synchronize()
    for z in range(B):
        ref = ops.fp8_scaled_mm(d["a"][z], d["w"][0], d["scale"][0].reshape(1))
        _assert_entry(out[z], ref, {"a": d["a"][z], "w": d["w"][0]}, z, d["scale"][0].reshape(1), None,
                      f"shared W, entry {z}")
    # overlapping outputs are refused before any launch
    assert lib.mxq_fp8_scaled_bmm(d["a"].data_ptr(), B, M, K, K, M * K, d["w"].data_ptr(), N, N * K,
                                  d["scale"].data_ptr(), 1, None, 0, 0, out.data_ptr(), N, N, st) == L.MXQ_ERR_SHAPE


def test_fp8_scaled_bmm_empty_and_strided_input():
    d = synth.batched_w8a16(3, 20, 128, 256, seed=41, device=gpu())
    empty = ops.fp8_scaled_bmm(d["a"][:, :0], d["w"], d["scale"], d["bias"])
    assert empty.shape == (3, 0, 128)
    # row stride 320 elements and a batch stride with a gap: strided entries, same results
    big = torch.zeros(3, 24, 320, dtype=torch.bfloat16, device=gpu())
    big[:, :20, :256] = d["a"]
    view = big[:, :20, :256]
    got = ops.fp8_scaled_bmm(view, d["w"], d["scale"], d["bias"])
    ref = ops.fp8_scaled_bmm(d["a"], d["w"], d["scale"], d["bias"])
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def _block_case(M, N, K, block_n, seed, bias_dtype=None, scale_recipe="synth"):
    d = synth.block_linear(M, N, K, seed=seed, device=gpu(), block_n=block_n, bias_dtype=bias_dtype)
    if scale_recipe == "page":  # rand(N/bn, K/128) + 0.1 as in the page's accuracy test
        g = torch.Generator(device="cuda").manual_seed(seed + 1)
        d["sw"] = torch.rand(d["sw"].shape, generator=g, device=gpu()) + 0.1
        d["w"] = torch.randn(N, K, generator=g, device=gpu()).to(torch.bfloat16).to(torch.float8_e4m3fn).view(torch.uint8)
    return d


def _oracle_block(d, x2=None):
    x = d["x"] if x2 is None else x2
    bias = None if d["bias"] is None else f32(d["bias"].float())
    return OD.block_fp8_linear_bf16(bf16_bits(x.reshape(-1, x.shape[-1])), u8(d["w"]), f32(d["sw"]), d["block_n"],
                                    bias)


@pytest.mark.parametrize("M", [1, 8, 16, 17])
@pytest.mark.parametrize("block_n", [128, 1])
def test_block_linear_page_recipe(M, block_n):
    d = _block_case(M, 256, 256, block_n, seed=M + block_n, bias_dtype=torch.bfloat16, scale_recipe="page")
    out = ops.block_fp8_linear(d["x"], d["w"], [block_n, 128], d["sw"], bias=d["bias"])
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_block(d), what=f"block linear M={M} bn={block_n}")
    # the load-time relayout of the scale grid (stored transposed) gives the same bits
    sw_t = torch.empty_strided(d["sw"].shape, (1, d["sw"].shape[0]), dtype=torch.float32, device=gpu())
    sw_t.copy_(d["sw"])
    out_t = ops.block_fp8_linear(d["x"], d["w"], [block_n, 128], sw_t, bias=d["bias"])
    torch.cuda.synchronize()
    assert torch.equal(out_t, out)


@pytest.mark.parametrize("block_n", [128, 1])
@pytest.mark.parametrize("M,N,K", [(200, 384, 512), (130, 200, 256), (64, 1152, 1024), (257, 640, 384)])
def test_block_linear_ragged_tiles(M, N, K, block_n):
    """M > 128 takes the large direct-to-LDS tile, for 128x128 and (per-column scales) 1x128
    weight blocks alike; the scale grid stored transposed gives the same bits."""
    d = _block_case(M, N, K, block_n, seed=M + N + K + block_n, bias_dtype=torch.float32)
    out = ops.block_fp8_linear(d["x"], d["w"], [block_n, 128], d["sw"], bias=d["bias"])
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_block(d), what=f"block linear {M}x{N}x{K} bn={block_n}")
    sw_t = torch.empty_strided(d["sw"].shape, (1, d["sw"].shape[0]), dtype=torch.float32, device=gpu())
    sw_t.copy_(d["sw"])
    out_t = ops.block_fp8_linear(d["x"], d["w"], [block_n, 128], sw_t, bias=d["bias"])
    torch.cuda.synchronize()
    assert torch.equal(out_t, out)


def test_block_linear_prequantised_3d_and_noncontiguous():
    d = _block_case(34, 256, 384, 128, seed=77)
    q, s = ops.per_token_group_quant_fp8(d["x"])
    out_q = ops.block_fp8_linear(q, d["w"], [128, 128], d["sw"], input_scale=s)
    out_b = ops.block_fp8_linear(d["x"], d["w"], [128, 128], d["sw"])
    torch.cuda.synchronize()
    assert torch.equal(out_q, out_b)
    x3 = d["x"].view(2, 17, 384)
    out3 = ops.block_fp8_linear(x3, d["w"], [128, 128], d["sw"])
    assert out3.shape == (2, 17, 256)
    assert torch.equal(out3.view(34, 256), out_b)
    # non-contiguous 3-D view (last dim strided)
    big = torch.zeros(2, 17, 384, 2, dtype=torch.bfloat16, device=gpu())
    big[..., 0] = x3
    xs = big[..., 0]
    assert xs.stride(-1) != 1
    outs = ops.block_fp8_linear(xs, d["w"], [128, 128], d["sw"])
    torch.cuda.synchronize()
    assert torch.equal(outs.view(34, 256), out_b)
    assert_bf16_close(bf16_bits(out_b), _oracle_block(d), what="prequantised")


def test_block_linear_non_square_scale_grid():
    d = _block_case(9, 384, 1024, 128, seed=5)  # grid [3, 8]
    out = ops.block_fp8_linear(d["x"], d["w"], (128, 128), d["sw"])
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_block(d), what="non-square grid")


def test_block_linear_rejects_bad_block_sizes():
    d = _block_case(4, 256, 256, 128, seed=3)
    for bs in RECIPES["block_fp8_shapes"]["rejected_block_sizes"]:
        with pytest.raises(ValueError):
            ops.block_fp8_linear(d["x"], d["w"], bs, d["sw"])


@pytest.mark.parametrize("block_n", [128, 1])
def test_block_linear_workload_sampled_rows(block_n):
    M, K, N = 2048, 2048, 7168
    d = _block_case(M, N, K, block_n, seed=1002)
    out = ops.block_fp8_linear(d["x"], d["w"], [block_n, 128], d["sw"])
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 129, 1000, 1023, 1024, 2046, 2047])
    want = OD.block_fp8_linear_bf16(bf16_bits(d["x"][rows]), u8(d["w"]), f32(d["sw"]), block_n)
    assert_bf16_close(bf16_bits(out[rows]), want, what=f"2048x2048x7168 sampled rows bn={block_n}")
    if block_n != 128:
        return
    # the quantised activations of the workload are bit-exact too
    q, s = ops.per_token_group_quant_fp8(d["x"])
    torch.cuda.synchronize()
    q_ref, s_ref = oracle_quant(bf16_bits(d["x"][rows]))
    assert np.array_equal(u8(q)[rows], q_ref) and np.array_equal(f32(s)[rows], s_ref)


def test_block_linear_zero_rows():
    d = _block_case(1, 256, 256, 128, seed=4)
    out = ops.block_fp8_linear(d["x"][:0], d["w"], [128, 128], d["sw"])
    assert out.shape == (0, 256)


@pytest.mark.parametrize("seed", range(8))
def test_random_per_tensor_shapes_both_kernels_and_oracle(seed):
    """Seeded random per-tensor W8A16 shapes (M 1..300, N 16..700, K a multiple of 32 up to
    1024, with and without bias): a batched call large enough to run the register-staged
    kernel equals, entry by entry, the 2-D calls (the ring-fed kernel where the grid fits the
    GPU and K > 128; few rows with K a multiple of 128 may stream instead, checked against the
    oracle), and both match the oracle."""
    rng = np.random.default_rng(500 + seed)
    M = int(rng.integers(1, 301))
    N = int(rng.integers(1, 44)) * 16
    K = int(rng.integers(1, 33)) * 32
    B = 40
    d = synth.batched_w8a16(B, M, N, K, seed=seed + 3, device=gpu(), has_bias=bool(seed % 2))
    out = ops.fp8_scaled_bmm(d["a"], d["w"], d["scale"], d["bias"])
    torch.cuda.synchronize()
    for z in (0, B // 2, B - 1):
        ref = ops.fp8_scaled_mm(d["a"][z], d["w"][z], d["scale"][z].reshape(1),
                                None if d["bias"] is None else d["bias"][z])
        torch.cuda.synchronize()
        _assert_entry(out[z], ref, d, z, d["scale"][z].reshape(1), None if d["bias"] is None else d["bias"][z],
                      f"M={M} N={N} K={K} entry {z}")
    want = _oracle_bmm(dict(d, a=d["a"][:2], w=d["w"][:2], scale=d["scale"][:2]),
                       None if d["bias"] is None else f32(d["bias"][:2]))
    assert_bf16_close(bf16_bits(out[:2]), want, what=f"random bmm M={M} N={N} K={K}")


@pytest.mark.parametrize("seed", range(8))
def test_random_block_linear_shapes(seed):
    """Seeded random block-FP8 W8A8 shapes (M 1..600 across the 128-row switch to the large
    tile, N 16..1024 including partial 256- and 128-wide column tiles, K a multiple of 128 up
    to 1024, 128x128 or 1x128 weight blocks, with and without bias) against the oracle."""
    rng = np.random.default_rng(900 + seed)
    M = int(rng.integers(1, 601))
    N = int(rng.integers(1, 65)) * 16
    K = int(rng.integers(1, 9)) * 128
    block_n = [128, 1][seed % 2]
    bias = torch.float32 if seed % 3 else None
    d = _block_case(M, N, K, block_n, seed=seed + 11, bias_dtype=bias)
    out = ops.block_fp8_linear(d["x"], d["w"], [block_n, 128], d["sw"], bias=d["bias"])
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_block(d), what=f"random block linear {M}x{N}x{K} bn={block_n}")


@pytest.mark.parametrize("block_n", [128, 1])
@pytest.mark.parametrize("shape", [(300, 520, 384), (1100, 3900, 256), (2100, 4000, 128), (130, 256, 16512)])
def test_block_linear_grid_picked_tiles(shape, block_n):
    """The dense W8A8 GEMM picks its tile from the grid: 300 x 520 fits one round of 128 x 128
    tiles (ragged rows and an 8-column last tile); 1100 x 3900 one round of 128 x 256 tiles
    (ragged rows, the 60-column tail on the 128-wide register-staged tile); 2100 x 4000 takes
    the 256 x 256 tile (ragged rows and a 160-column last tile); K = 16512, past the
    direct-to-LDS tiles' range, runs on the register-staged tiles.  Each against the oracle."""
    M, N, K = shape
    d = _block_case(M, N, K, block_n, seed=M + block_n, bias_dtype=torch.float32)
    out = ops.block_fp8_linear(d["x"], d["w"], [block_n, 128], d["sw"], bias=d["bias"])
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_block(d), what=f"block linear {M}x{N}x{K} bn={block_n}")


@pytest.mark.parametrize("M,N,K,prequant,split", [(1, 2048, 7168, False, 8), (5, 998, 7168, False, 8),
                                                  (13, 2048, 4096, True, 8), (40, 1024, 7168, False, 4),
                                                  (8, 12288, 1536, True, 2), (3, 300, 256, False, 1),
                                                  (64, 256, 4096, True, 8), (1, 7168, 16384, False, 8),
                                                  (4, 16384, 4096, True, 4)])
@pytest.mark.parametrize("block_n", [128, 1])
def test_block_linear_few_rows(M, N, K, prequant, split, block_n):
    """Few-row block linears (128 x 128 or 1 x 128 weight blocks; the latter with each K chunk's
    column scales in LDS) run on the weight-streaming kernel in
    tiles of 4 or 8 rows, K cut into `split` chunks whose fp32 partial sums a second kernel adds
    in chunk order: ragged row tiles, a column count that is not a multiple of 4 (the scalar
    sum), 64- and 128-column tiles, bf16 input quantised in the call (the partial sums after
    the codes in the workspace) and pre-quantised input (bit-equal to it), a bias, and one
    unsplit case writing bf16 directly, K = 16384, where only a K chunk of each row fits the
    workgroup's LDS, and a long-K call whose row tiles would fill the GPU (4 x 16384 x 4096);
    each against the oracle."""
    lib = L.load()
    part = lib.mxq_block_fp8_linear_workspace_size(M, N, K, L.MXQ_DTYPE_E4M3)
    assert part == (0 if split == 1 else (4 * split * M * N + 255) // 256 * 256)
    d = _block_case(M, N, K, block_n, seed=M * 7 + N, bias_dtype=torch.float32)
    out = ops.block_fp8_linear(d["x"], d["w"], [block_n, 128], d["sw"], bias=d["bias"])
    if prequant:
        q, s = ops.per_token_group_quant_fp8(d["x"])
        out_q = ops.block_fp8_linear(q, d["w"], [block_n, 128], d["sw"], input_scale=s, bias=d["bias"])
        torch.cuda.synchronize()
        assert torch.equal(out_q.view(torch.int16), out.view(torch.int16))
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_block(d), what=f"few-row block linear {M}x{N}x{K} bn={block_n}")


@pytest.mark.parametrize("M,N,K,block_n", [(128, 2048, 7168, 128), (300, 520, 4096, 128), (1000, 1024, 4096, 128),
                                           (96, 998, 7168, 1), (65, 256, 8192, 128)])
def test_block_linear_few_tiles_k_split(M, N, K, block_n):
    """65 to 1024 rows whose 128 x 128 tiles leave the GPU mostly idle: each tile's K range runs
    as 2, 4 or 8 chunks (workgroups of their own) writing fp32 partial sums, added in chunk
    order by the split-sum kernel: ragged rows and columns, a column count that is not a
    multiple of 4, per-column (1 x 128) weight scales, a bias added once, and one row past
    the 64-row tiles; each against the oracle."""
    lib = L.load()
    part = lib.mxq_block_fp8_linear_workspace_size(M, N, K, L.MXQ_DTYPE_E4M3)
    assert part > 0 and part % (4 * M * N) in (0, 256 - (4 * M * N) % 256) and part // (4 * M * N) in (2, 4, 8)
    d = _block_case(M, N, K, block_n, seed=M + N + K, bias_dtype=torch.float32)
    out = ops.block_fp8_linear(d["x"], d["w"], [block_n, 128], d["sw"], bias=d["bias"])
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _oracle_block(d), what=f"few-tile split {M}x{N}x{K} bn={block_n}")
