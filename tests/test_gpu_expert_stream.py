"""GPU parity of the expert-streaming path: routings made only of tiny expert blocks with bf16
activations, the path the fused MoE takes by default for decode-sized batches.

Every case runs twice: with the default dispatch (the streaming kernels group the routed rows
by expert inside each workgroup and end stage 1 in the SiLU-and-mul) and with every block forced
through the tiny-block class (sorted block tables, gate / up rows stored, standalone
SiLU-and-mul).  Both evaluate the same per-row arithmetic and rounding points ("vLLM PR 50949
review", implementation items 1-2), so the outputs must agree bit for bit; both must match the
oracle within atol = rtol = 1e-2.  The shapes cover partial column tiles, reduction lengths that
are not a whole number of ring turns (and a single step), experts holding more rows than one
pass, 512 experts, expert ids outside [0, E), both weight layouts, and the GPT-OSS decode shape.
"""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_expert_amd as mx
from mxfp4_block_scaled_expert_amd import ops, synth
from tests._util import assert_bf16_close, bf16_bits, gpu
from tests.test_gpu_moe import _run_oracle, _small_spec

pytestmark = pytest.mark.gpu


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
                             inp["w2"], inp["w2_scale"], inp.get("w1_bias"), act_quant=False, weight_layout=layout,
                             dispatch=dispatch)


def _stream_vs_tiny_class(inp, layout, what):
    """Default dispatch (streaming path) and forced tiny class without a K split: bit-identical
    outputs."""
    src = _tiled(inp) if layout == "tiled" else inp
    got = _run(src, layout)
    ref = _run(src, layout, ops.Dispatch(mx.MXQ_DISPATCH_FORCED, 0, k_split=1))
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), what
    return got


CASES = {
    # partial 64-column tiles in both stages, a reduction of one (ragged) step
    "mxfp4_h96_i96": ("fused_moe_mxfp4", 16, 8, 4, 96, 96),
    # up to 16 rows per expert (four passes); 4 and 2 steps: padded to whole ring turns
    "mxfp4_multipass": ("fused_moe_mxfp4", 32, 4, 2, 1024, 512),
    # e4m3 weights with block scales; 4 and 2 steps
    "w8a16_h512_i256": ("fused_moe_fp8", 24, 8, 2, 512, 256),
    # many experts, a few rows each
    "mxfp4_e512": ("fused_moe_mxfp4", 8, 512, 8, 256, 128),
    "w8a16_e512": ("fused_moe_fp8", 8, 512, 8, 256, 128),
}


@pytest.mark.parametrize("layout", ["plain", "tiled"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_stream_path_matches_tiny_class_and_oracle(case, layout):
    kind, M, E, topk, H, I = CASES[case]
    inp = synth.moe_inputs(_small_spec(kind, M, E, topk, H, I), seed=501 + len(case), device=gpu())
    got = _stream_vs_tiny_class(inp, layout, f"{case} {layout}")
    assert_bf16_close(bf16_bits(got), _run_oracle(inp), what=f"{case} {layout}")


def test_stream_path_with_bias_on_e4m3_weights():
    inp = synth.moe_inputs(_small_spec("fused_moe_fp8", 12, 8, 2, 512, 256), seed=77, device=gpu())
    g = torch.Generator().manual_seed(78)
    inp["w1_bias"] = torch.randn(8, 512, generator=g).to(gpu())
    got = _stream_vs_tiny_class(inp, "plain", "e4m3 + bias")
    assert_bf16_close(bf16_bits(got), _run_oracle(inp), what="e4m3 + bias")


def test_stream_path_one_expert_takes_every_row():
    """All 32 tokens pick experts 0 and 1: two experts with 32 rows each (eight passes)."""
    inp = synth.moe_inputs(_small_spec("fused_moe_mxfp4", 32, 8, 2, 512, 256), seed=91, device=gpu())
    ids = torch.tensor([[0, 1]] * 32, dtype=torch.int32)
    ids[::2] = torch.tensor([1, 0], dtype=torch.int32)
    inp["topk_ids"] = ids.to(gpu())
    got = _stream_vs_tiny_class(inp, "tiled", "two hot experts")
    assert_bf16_close(bf16_bits(got), _run_oracle(inp), what="two hot experts")


def test_stream_path_drops_ids_outside_the_expert_range():
    """Ids -1 and E name no expert: both paths drop those routed rows (the oracle rejects them,
    so the check is against the tiny-block class, and against the oracle on the remaining
    routing with the dropped rows' weights set to zero)."""
    inp = synth.moe_inputs(_small_spec("fused_moe_mxfp4", 16, 8, 2, 256, 128), seed=93, device=gpu())
    ids = inp["topk_ids"].cpu().clone()
    ids[3, 1] = -1
    ids[7, 0] = 8
    ids[11, 1] = 1 << 20
    inp["topk_ids"] = ids.to(gpu())
    got = _stream_vs_tiny_class(inp, "plain", "ids outside [0, E)")
    ok = inp["topk_ids"].cpu().numpy()
    bad = (ok < 0) | (ok >= 8)
    ref = dict(inp)
    ref["topk_ids"] = torch.from_numpy(np.where(bad, 0, ok).astype(np.int32))
    ref["topk_weights"] = torch.from_numpy(np.where(bad, 0.0, inp["topk_weights"].cpu().numpy()).astype(np.float32))
    assert_bf16_close(bf16_bits(got), _run_oracle(ref), what="ids outside [0, E)")


def test_stream_path_gptoss_decode_shape_matches_tiny_class():
    inp = synth.moe_inputs("moe_mxfp4_gptoss_decode_m32", seed=1004, device=gpu())
    _stream_vs_tiny_class(inp, "tiled", "GPT-OSS decode, tiled")
