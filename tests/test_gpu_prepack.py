"""GPU checks of the load-time weight relayout.

* mxq_moe_prepack / mxq_moe_prepack_scales produce exactly the tiled layout the
  header defines (compared byte for byte with a numpy re-layout written from that
  definition, ragged row lengths included).
* The fused MoE gives bit-identical outputs from plain and tiled weights, for every
  weight format and every tile class (the load-time relayout changes no arithmetic;
  "SGLang PR 32618 review": packed and unpacked weights are tested against the same
  reference; "SGLang PR 35605 review": the load-time layout must match exactly).
* The tiled decode workload also matches the oracle on sampled tokens.
"""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_expert_amd as mx
from mxfp4_block_scaled_expert_amd import ops, synth
from tests._util import assert_bf16_close, bf16_bits, gpu
from tests.test_gpu_moe import SMALL_BLOCKS, _run_oracle, _small_spec

pytestmark = pytest.mark.gpu


def _tiled_ref(w: np.ndarray) -> np.ndarray:
    E, N, RB = w.shape
    S = -(-RB // 128)
    wp = np.zeros((E, N, S * 128), np.uint8)
    wp[:, :, :RB] = w
    # row step bytes = 32 q + 16 h + b;  tile bytes = 1024 h + 16 (16 q + l16) + b
    t = wp.reshape(E, N // 16, 16, S, 4, 2, 16).transpose(0, 1, 3, 5, 4, 2, 6)
    return np.ascontiguousarray(t).reshape(E, N, S * 128)


def _tiled_scales_ref(s: np.ndarray) -> np.ndarray:
    E, N, G = s.shape
    S = -(-G // 8)
    sp = np.zeros((E, N, S * 8), np.uint8)
    sp[:, :, :G] = s
    # step groups = 2 q + j;  tile bytes = 2 (16 q + l16) + j
    t = sp.reshape(E, N // 16, 16, S, 4, 2).transpose(0, 1, 3, 4, 2, 5)
    return np.ascontiguousarray(t).reshape(E, N, S * 8)


@pytest.mark.parametrize("shape", [(3, 48, 1440), (2, 32, 256), (1, 16, 16), (2, 64, 2048)])
def test_prepack_weight_layout(shape):
    g = torch.Generator().manual_seed(sum(shape))
    w = torch.randint(0, 256, shape, dtype=torch.uint8, generator=g)
    got = ops.moe_prepack(w.to(gpu()))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), _tiled_ref(w.numpy()))


@pytest.mark.parametrize("shape", [(3, 48, 90), (2, 32, 64), (1, 16, 3), (2, 64, 224)])
def test_prepack_scale_layout(shape):
    g = torch.Generator().manual_seed(7 + sum(shape))
    s = torch.randint(0, 256, shape, dtype=torch.uint8, generator=g)
    got = ops.moe_prepack_scales(s.to(gpu()))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), _tiled_scales_ref(s.numpy()))


def _tiled(inp):
    t = dict(inp)
    t["w1"] = ops.moe_prepack(inp["w1"])
    t["w2"] = ops.moe_prepack(inp["w2"])
    if inp["kind"] == "fused_moe_mxfp4":
        t["w1_scale"] = ops.moe_prepack_scales(inp["w1_scale"])
        t["w2_scale"] = ops.moe_prepack_scales(inp["w2_scale"])
    return t


def _run(inp, layout, dispatch=None):
    if inp["kind"] == "fused_moe_mxfp4":
        return ops.fused_moe_mxfp4(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"],
                                   inp["w2"], inp["w2_scale"], inp["w1_bias"], weight_layout=layout,
                                   dispatch=dispatch)
    return ops.fused_moe_fp8(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"],
                             inp["w2"], inp["w2_scale"], inp.get("w1_bias"), act_quant=inp["act_quant"],
                             weight_layout=layout, dispatch=dispatch)


CASES = {
    "w8a16": lambda: synth.moe_inputs(SMALL_BLOCKS, seed=1003, device=gpu()),
    "w8a8": lambda: synth.moe_inputs(_small_spec("fused_moe_fp8", 300, 16, 4, 512, 256, zipf=1.1, act_quant=True),
                                     seed=31, device=gpu()),
    "mxfp4": lambda: synth.moe_inputs(_small_spec("fused_moe_mxfp4", 40, 8, 4, 2880, 2880), seed=32, device=gpu()),
}


@pytest.mark.parametrize("forced", [None, 0, 1, 2, 3, 4])
@pytest.mark.parametrize("kind", ["w8a16", "w8a8", "mxfp4"])
def test_tiled_equals_plain_bit_for_bit(kind, forced):
    inp = CASES[kind]()
    tin = _tiled(inp)
    d = None if forced is None else ops.Dispatch(mx.MXQ_DISPATCH_FORCED, forced)
    a = _run(inp, "plain", d)
    b = _run(tin, "tiled", d)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{kind} forced={forced}"


def test_tiled_tiny_rows_and_gemv_request():
    """Tiny-class bounds 4 and 16, and the GEMV request (plain only) with tiled weights."""
    inp = CASES["mxfp4"]()
    tin = _tiled(inp)
    want = _run_oracle(inp)
    for rows, tiny in ((4, mx.MXQ_TINY_MFMA), (16, mx.MXQ_TINY_MFMA), (8, mx.MXQ_TINY_GEMV)):
        # the plain-layout reference runs the same kernels: the MFMA tiny kernel, same class bound
        ref = _run(inp, "plain", ops.Dispatch(mx.MXQ_DISPATCH_PER_BLOCK, 0, rows, mx.MXQ_TINY_MFMA))
        got = _run(tin, "tiled", ops.Dispatch(mx.MXQ_DISPATCH_PER_BLOCK, 0, rows, tiny))
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), f"rows={rows} kernel={tiny}"
        assert_bf16_close(bf16_bits(got), want, what=f"tiny rows={rows} kernel={tiny}")


def test_gptoss_decode_tiled_against_oracle():
    inp = synth.moe_inputs("moe_mxfp4_gptoss_decode_m32", seed=1004, device=gpu())
    out = _run(_tiled(inp), "tiled")
    torch.cuda.synchronize()
    tokens = np.array([1, 17, 30])
    want = _run_oracle(inp, tokens)
    assert_bf16_close(bf16_bits(out[torch.from_numpy(tokens).to(gpu())]), want, what="gpt-oss decode tiled")


def test_binding_rejects_wrong_layout_shapes():
    inp = CASES["mxfp4"]()
    with pytest.raises(ValueError):
        _run(inp, "tiled")  # plain tensors passed as tiled
    with pytest.raises(ValueError):
        _run(inp, "swizzled")
