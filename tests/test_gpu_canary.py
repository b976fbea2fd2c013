"""Canary-guarded outputs: every entry point writes exactly its output elements.

Each output lives inside a larger buffer filled with a canary pattern: guard
rows before and after it, and (where the entry point takes a row stride) guard
columns past each row.  After the call the canaries must be untouched and the
output must equal, bit for bit, the same call made through the binding into a
plain buffer.  Shapes are ragged in every dimension (partial row tiles, partial
column tiles, reductions that end mid-tile, single rows), so every tail path of
the kernels is exercised.
"""

import ctypes as C

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_expert_amd as mx
from mxfp4_block_scaled_expert_amd import _lib as L
from mxfp4_block_scaled_expert_amd import ops, synth
from tests._util import gpu

pytestmark = pytest.mark.gpu

CANARY16 = 0x7FBF  # a bf16 NaN pattern no kernel produces from finite inputs
CANARY8 = 0xA5
GUARD_ROWS = 3


def _guarded(rows, cols, ld, dtype, canary):
    """A [GUARD_ROWS + rows + GUARD_ROWS, ld] buffer of canaries and the [rows, cols] window."""
    itemsize = torch.empty((), dtype=dtype).element_size()
    raw = torch.empty((2 * GUARD_ROWS + rows) * ld * itemsize, dtype=torch.uint8, device=gpu())
    if itemsize == 1:
        raw.fill_(canary)
    elif itemsize == 2:
        raw.view(torch.int16).fill_(np.int16(np.uint16(canary).view(np.int16)))
    else:
        raw.view(torch.int32).fill_(int(np.uint32(canary).view(np.int32)))
    full = raw.view(dtype).view(2 * GUARD_ROWS + rows, ld)
    return full, full[GUARD_ROWS:GUARD_ROWS + rows, :cols]


def _assert_canaries(full, rows, cols, canary):
    itemsize = full.element_size()
    bits = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[itemsize]
    b = full.view(bits).cpu().numpy().astype(np.int64) & ((1 << (8 * itemsize)) - 1)
    mask = np.ones(b.shape, bool)
    mask[GUARD_ROWS:GUARD_ROWS + rows, :cols] = False
    bad = (b != canary) & mask
    assert not bad.any(), f"{int(bad.sum())} canary elements overwritten, first at {np.argwhere(bad)[:4].tolist()}"


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("M,N,K,block_n", [(300, 200, 384, 128), (17, 1000, 256, 128), (257, 640, 384, 1),
                                           (1, 130, 128, 128), (129, 264, 256, 1), (64, 136, 1152, 128),
                                           (5, 998, 4096, 128)])
def test_block_linear_writes_only_its_output(M, N, K, block_n):
    lib = L.load()
    d = synth.block_linear(M, N, K, seed=M + N + K, device=gpu(), block_n=block_n, bias_dtype=torch.float32)
    ref = ops.block_fp8_linear(d["x"], d["w"], [block_n, 128], d["sw"], bias=d["bias"])
    ldo = N + 40
    full, out = _guarded(M, N, ldo, torch.bfloat16, CANARY16)
    ws_n = lib.mxq_block_fp8_linear_workspace_size(M, N, K, L.MXQ_DTYPE_BF16)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=gpu())
    st = lib.mxq_block_fp8_linear(d["x"].data_ptr(), L.MXQ_DTYPE_BF16, None, M, K, K, d["w"].data_ptr(), N,
                                  d["sw"].data_ptr(), d["sw"].stride(0), d["sw"].stride(1), block_n, 128,
                                  d["bias"].data_ptr(), L.MXQ_DTYPE_F32, out.data_ptr(), L.MXQ_DTYPE_BF16, ldo,
                                  ws.data_ptr(), ws_n, _stream())
    assert st == 0
    torch.cuda.synchronize()
    _assert_canaries(full, M, N, CANARY16)
    assert torch.equal(out.contiguous().view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(97, 224, 576), (130, 200, 512), (1, 128, 32), (33, 136, 96), (5, 998, 4096)])
def test_per_tensor_mm_writes_only_its_output(M, N, K):
    lib = L.load()
    d = synth.dense_w8a16(M, N, K, seed=M * 3 + N + K, device=gpu())
    ref = ops.fp8_scaled_mm(d["a"], d["w"], d["scale"], d["bias"])
    ldo = N + 24
    full, out = _guarded(M, N, ldo, torch.bfloat16, CANARY16)
    ws_n = lib.mxq_fp8_scaled_mm_workspace_size(M, N, K)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=gpu())
    st = lib.mxq_fp8_scaled_mm(d["a"].data_ptr(), M, K, K, d["w"].data_ptr(), N, d["scale"].data_ptr(),
                               d["bias"].data_ptr(), L.MXQ_DTYPE_F32, out.data_ptr(), ldo, ws.data_ptr(), ws_n,
                               _stream())
    assert st == 0
    torch.cuda.synchronize()
    _assert_canaries(full, M, N, CANARY16)
    assert torch.equal(out.contiguous().view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("M,K", [(1, 128), (37, 384), (300, 2048)])
def test_quant_writes_only_its_outputs(M, K):
    lib = L.load()
    g = torch.Generator(device="cuda").manual_seed(M + K)
    x = torch.randn(M, K, generator=g, device=gpu()).to(torch.bfloat16)
    q_ref, s_ref = ops.per_token_group_quant_fp8(x)
    qf, q = _guarded(M, K, K, torch.uint8, CANARY8)
    sf, s = _guarded(M, K // 128, K // 128, torch.float32, 0x7FC00001)
    assert lib.mxq_per_token_group_quant_fp8(x.data_ptr(), M, K, K, 128, q.data_ptr(), s.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    _assert_canaries(qf, M, K, CANARY8)
    _assert_canaries(sf, M, K // 128, 0x7FC00001)
    assert torch.equal(q, q_ref.view(torch.uint8)) and torch.equal(s.view(torch.int32), s_ref.view(torch.int32))


@pytest.mark.parametrize("quant", [False, True])
def test_silu_and_mul_writes_only_its_outputs(quant):
    lib = L.load()
    rows, I = 45, 384
    g = torch.Generator(device="cuda").manual_seed(9)
    ic0 = (torch.randn(rows, 2 * I, generator=g, device=gpu()) * 2).to(torch.bfloat16)
    if quant:
        q_ref, s_ref = ops.silu_and_mul(ic0, quant=True)
        qf, q = _guarded(rows, I, I, torch.uint8, CANARY8)
        sf, s = _guarded(rows, I // 128, I // 128, torch.float32, 0x7FC00001)
        assert lib.mxq_silu_and_mul(ic0.data_ptr(), rows, I, 2 * I, None, q.data_ptr(), s.data_ptr(), _stream()) == 0
        torch.cuda.synchronize()
        _assert_canaries(qf, rows, I, CANARY8)
        _assert_canaries(sf, rows, I // 128, 0x7FC00001)
        assert torch.equal(q, q_ref.view(torch.uint8)) and torch.equal(s, s_ref)
    else:
        ref = ops.silu_and_mul(ic0)
        hf, h = _guarded(rows, I, I, torch.bfloat16, CANARY16)
        assert lib.mxq_silu_and_mul(ic0.data_ptr(), rows, I, 2 * I, h.data_ptr(), None, None, _stream()) == 0
        torch.cuda.synchronize()
        _assert_canaries(hf, rows, I, CANARY16)
        assert torch.equal(h.view(torch.int16), ref.view(torch.int16))


MOE_CASES = {
    # W8A8 with ragged blocks in every class; H = 384: a partial 256-wide column tile
    "w8a8": (dict(kind="fused_moe_fp8", M=150, E=12, topk=3, H=384, I=256, zipf=1.1, act_quant=True), None),
    # W8A16 small blocks (counts straddling the class bounds), tile classes forced
    "w8a16_forced_16": ("moe_block_fp8_w8a16_e8_h2048_i1024", 1),
    # MXFP4 with H = I = 2880 (a partial 64-column tile, a ragged last K step)
    "mxfp4": (dict(kind="fused_moe_mxfp4", M=40, E=8, topk=4, H=2880, I=2880), None),
    "mxfp4_128": (dict(kind="fused_moe_mxfp4", M=40, E=8, topk=4, H=2880, I=2880), 4),
    # decode-sized: the expert-streaming path
    "mxfp4_stream": (dict(kind="fused_moe_mxfp4", M=12, E=16, topk=4, H=96, I=96), None),
}


@pytest.mark.parametrize("case", sorted(MOE_CASES))
def test_fused_moe_writes_only_its_output(case):
    spec, forced = MOE_CASES[case]
    inp = synth.moe_inputs(spec, seed=61, device=gpu())
    d = None if forced is None else ops.Dispatch(mx.MXQ_DISPATCH_FORCED, forced)
    M, H = inp["x"].shape
    full, out = _guarded(M, H, H, torch.bfloat16, CANARY16)
    if inp["kind"] == "fused_moe_mxfp4":
        ref = ops.fused_moe_mxfp4(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"],
                                  inp["w2"], inp["w2_scale"], inp["w1_bias"], dispatch=d)
        ops.fused_moe_mxfp4(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"], inp["w2"],
                            inp["w2_scale"], inp["w1_bias"], dispatch=d, out=out)
    else:
        ref = ops.fused_moe_fp8(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"], inp["w2"],
                                inp["w2_scale"], None, act_quant=inp["act_quant"], dispatch=d)
        ops.fused_moe_fp8(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"], inp["w2"],
                          inp["w2_scale"], None, act_quant=inp["act_quant"], dispatch=d, out=out)
    torch.cuda.synchronize()
    _assert_canaries(full, M, H, CANARY16)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
