"""The allocation-free block linear (mxq_block_fp8_linear_noalloc) against the allocating
entry point (mxq_block_fp8_linear), through the C ABI: two calls in a row on one stream, the
second with a smaller input, each bit-identical to the allocating call on the same inputs;
plus the size limit, refused before anything is enqueued."""

import pytest
import torch

from mxfp4_block_scaled_expert_amd import _lib as L
from mxfp4_block_scaled_expert_amd import synth


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _call(lib, d, M, N, K, out, noalloc, bias=None, x=None, a_dtype=None, a_scale=None):
    x = d["x"] if x is None else x
    a_dtype = L.MXQ_DTYPE_BF16 if a_dtype is None else a_dtype
    sw = d["sw"]
    b = None if bias is None else bias.data_ptr()
    sp = None if a_scale is None else a_scale.data_ptr()
    common = (x.data_ptr(), a_dtype, sp, M, K, K, d["w"].data_ptr(), N, sw.data_ptr(), sw.stride(0),
              sw.stride(1), d["block_n"], 128, b, L.MXQ_DTYPE_F32, out.data_ptr(), L.MXQ_DTYPE_BF16, N)
    if noalloc:
        return lib.mxq_block_fp8_linear_noalloc(*common, _stream())
    n = lib.mxq_block_fp8_linear_workspace_size(M, N, K, a_dtype)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    st = lib.mxq_block_fp8_linear(*common, ws.data_ptr(), n, _stream())
    torch.cuda.synchronize()
    return st


def test_size_limit_is_refused_before_any_launch():
    lib = L.load()
    # 4096 x 8192 needs 32 MiB of codes plus 1 MiB of scales: beyond the 32 MiB scratch
    st = lib.mxq_block_fp8_linear_noalloc(None, L.MXQ_DTYPE_BF16, None, 4096, 8192, 8192, None, 256, None, 64, 1,
                                          128, 128, None, 0, None, L.MXQ_DTYPE_BF16, 256, None)
    assert st == L.MXQ_ERR_SCRATCH
    # shape and block errors are reported as such
    assert lib.mxq_block_fp8_linear_noalloc(None, L.MXQ_DTYPE_BF16, None, 4, 200, 200, None, 256, None, 2, 1, 128,
                                            128, None, 0, None, L.MXQ_DTYPE_BF16, 256, None) == L.MXQ_ERR_SHAPE
    assert lib.mxq_block_fp8_linear_noalloc(None, L.MXQ_DTYPE_BF16, None, 4, 256, 256, None, 256, None, 2, 1, 64,
                                            128, None, 0, None, L.MXQ_DTYPE_BF16, 256, None) == L.MXQ_ERR_BLOCK
    assert lib.mxq_block_fp8_linear_noalloc(None, L.MXQ_DTYPE_BF16, None, 4, 256, 256, None, 256, None, 2, 1, 128,
                                            128, None, 0, None, L.MXQ_DTYPE_BF16, 256, None) == L.MXQ_ERR_NULL


@pytest.mark.gpu
def test_noalloc_matches_the_allocating_entry_point_on_two_calls():
    lib = L.load()
    dev = torch.device("cuda", 0)
    # first call: close to the limit (4096 x 7168 -> 30.3 MB of the 32 MiB), second: smaller and ragged
    cases = [(4096, 512, 7168, 128, False), (300, 1000, 384, 1, True)]
    outs = []
    for M, N, K, bn, with_bias in cases:
        d = synth.block_linear(M, N, K, seed=M + N + K, device=dev, block_n=bn,
                               bias_dtype=torch.float32 if with_bias else None)
        got = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        assert _call(lib, d, M, N, K, got, True, d["bias"]) == L.MXQ_OK
        outs.append((d, got, M, N, K))
    torch.cuda.synchronize()
    for d, got, M, N, K in outs:
        want = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        assert _call(lib, d, M, N, K, want, False, d["bias"]) == L.MXQ_OK
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{M}x{N}x{K}"


@pytest.mark.gpu
def test_noalloc_prequantised_input_needs_no_scratch():
    lib = L.load()
    dev = torch.device("cuda", 0)
    M, N, K = 256, 384, 512
    d = synth.block_linear(M, N, K, seed=5, device=dev)
    q = torch.empty(M, K, dtype=torch.uint8, device=dev)
    s = torch.empty(M, K // 128, dtype=torch.float32, device=dev)
    assert lib.mxq_per_token_group_quant_fp8(d["x"].data_ptr(), M, K, K, 128, q.data_ptr(), s.data_ptr(),
                                             _stream()) == 0
    got = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    assert _call(lib, d, M, N, K, got, True, x=q, a_dtype=L.MXQ_DTYPE_E4M3, a_scale=s) == L.MXQ_OK
    want = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    assert _call(lib, d, M, N, K, want, False, x=q, a_dtype=L.MXQ_DTYPE_E4M3, a_scale=s) == L.MXQ_OK
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


@pytest.mark.gpu
def test_noalloc_few_rows_split_matches_on_two_calls():
    """Few rows: the K split's fp32 partial sums go to the static array as well.  Two calls in a
    row on one stream (the second smaller, with a ragged column count and pre-quantised input),
    each bit-identical to the allocating entry point on the same inputs."""
    lib = L.load()
    dev = torch.device("cuda", 0)
    outs = []
    for M, N, K, preq in [(8, 2048, 7168, False), (3, 998, 4096, True)]:
        assert lib.mxq_block_fp8_linear_workspace_size(M, N, K, L.MXQ_DTYPE_E4M3) > 0  # the split runs
        d = synth.block_linear(M, N, K, seed=M + N + K, device=dev, bias_dtype=torch.float32)
        kw = {}
        if preq:
            q = torch.empty(M, K, dtype=torch.uint8, device=dev)
            s = torch.empty(M, K // 128, dtype=torch.float32, device=dev)
            assert lib.mxq_per_token_group_quant_fp8(d["x"].data_ptr(), M, K, K, 128, q.data_ptr(), s.data_ptr(),
                                                     _stream()) == 0
            kw = dict(x=q, a_dtype=L.MXQ_DTYPE_E4M3, a_scale=s)
        got = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        assert _call(lib, d, M, N, K, got, True, d["bias"], **kw) == L.MXQ_OK
        outs.append((d, got, M, N, K, kw))
    torch.cuda.synchronize()
    for d, got, M, N, K, kw in outs:
        want = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        assert _call(lib, d, M, N, K, want, False, d["bias"], **kw) == L.MXQ_OK
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{M}x{N}x{K}"


@pytest.mark.gpu
def test_noalloc_few_tiles_split_matches_on_two_calls():
    """65..1024 rows on few tiles with long K: the K split's partial sums go to the static array.
    Two calls in a row on one stream (the second smaller and ragged), each bit-identical to the
    allocating entry point on the same inputs."""
    lib = L.load()
    dev = torch.device("cuda", 0)
    outs = []
    for M, N, K in [(128, 2048, 7168), (300, 520, 4096)]:
        assert lib.mxq_block_fp8_linear_workspace_size(M, N, K, L.MXQ_DTYPE_E4M3) > 0  # the split runs
        d = synth.block_linear(M, N, K, seed=M + N + K, device=dev, bias_dtype=torch.float32)
        got = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        assert _call(lib, d, M, N, K, got, True, d["bias"]) == L.MXQ_OK
        outs.append((d, got, M, N, K))
    torch.cuda.synchronize()
    for d, got, M, N, K in outs:
        want = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        assert _call(lib, d, M, N, K, want, False, d["bias"]) == L.MXQ_OK
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{M}x{N}x{K}"
