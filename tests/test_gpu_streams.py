"""The library keeps no per-call state on the device: calls on different streams with their
own workspaces run side by side, and a captured graph of calls replays them.

* two fused-MoE calls (the self-routed bf16 path and the sorted W8A8 path) and a block-FP8
  linear issued on three streams at once give the bits of the same calls issued one by one;
* a graph capturing a fused-MoE call (inputs, output and workspace allocated beforehand) and
  a block-FP8 linear (its output and workspace from the graph's pool) -- the library records
  no memset, allocation or synchronisation -- replayed three times with new input values
  written eagerly between the replays, matches an eager call on each replay's inputs bit for
  bit.
"""

import pytest
import torch

from mxfp4_block_scaled_expert_amd import _lib as L
from mxfp4_block_scaled_expert_amd import ops, synth
from tests._util import gpu

pytestmark = pytest.mark.gpu

SELF_ROUTED = "moe_block_fp8_w8a16_e8_h2048_i1024"
W8A8 = dict(kind="fused_moe_fp8", M=150, E=12, topk=3, H=384, I=256, zipf=1.1, act_quant=True)


def _moe(inp, ws, out):
    return ops.fused_moe_fp8(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"], inp["w2"],
                             inp["w2_scale"], inp.get("w1_bias"), act_quant=inp["act_quant"], workspace=ws, out=out)


def _moe_buffers(inp):
    M, H = inp["x"].shape
    ws = ops.fused_moe_workspace(M, H, inp["I"], inp["E"], inp["topk"], L.MXQ_WEIGHTS_FP8_BLOCK, inp["act_quant"],
                                 gpu())
    return ws, torch.empty(M, H, dtype=torch.bfloat16, device=gpu())


def _linear_inputs():
    return synth.block_linear(256, 768, 512, seed=5, device=gpu())


def _linear(d):
    return ops.block_fp8_linear(d["x"], d["w"], [128, 128], d["sw"])


def test_calls_on_three_streams_match_serial_calls():
    a = synth.moe_inputs(SELF_ROUTED, seed=31, device=gpu())
    b = synth.moe_inputs(W8A8, seed=32, device=gpu())
    d = _linear_inputs()
    wa, oa = _moe_buffers(a)
    wb, ob = _moe_buffers(b)
    ref_a = _moe(a, wa, oa).clone()
    ref_b = _moe(b, wb, ob).clone()
    ref_l = _linear(d).clone()
    torch.cuda.synchronize()
    for t in (oa, ob):
        t.zero_()
    streams = [torch.cuda.Stream() for _ in range(3)]
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(streams[0]):
            _moe(a, wa, oa)
        with torch.cuda.stream(streams[1]):
            _moe(b, wb, ob)
        with torch.cuda.stream(streams[2]):
            ol = _linear(d)
        torch.cuda.synchronize()
        assert torch.equal(oa.view(torch.int16), ref_a.view(torch.int16))
        assert torch.equal(ob.view(torch.int16), ref_b.view(torch.int16))
        assert torch.equal(ol.view(torch.int16), ref_l.view(torch.int16))


def test_captured_graph_replays_match_eager_calls():
    a = synth.moe_inputs(SELF_ROUTED, seed=41, device=gpu())
    d = _linear_inputs()
    wa, oa = _moe_buffers(a)
    # warm the library and the allocator outside the capture
    _moe(a, wa, oa)
    _linear(d)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _moe(a, wa, oa)
        ol = _linear(d)  # output (and the call's workspace) in the graph's memory pool
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(7)
    for rep in range(3):
        # new input values in place (eager work between the replays)
        a["x"].copy_(torch.randn(a["x"].shape, generator=gen, device=gpu()).to(torch.bfloat16))
        d["x"].copy_(torch.randn(d["x"].shape, generator=gen, device=gpu()).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_a, got_l = oa.clone(), ol.clone()
        wa2, oa2 = _moe_buffers(a)
        want_a = _moe(a, wa2, oa2)
        want_l = _linear(d)
        torch.cuda.synchronize()
        assert torch.equal(got_a.view(torch.int16), want_a.view(torch.int16)), f"replay {rep}: MoE"
        assert torch.equal(got_l.view(torch.int16), want_l.view(torch.int16)), f"replay {rep}: linear"
