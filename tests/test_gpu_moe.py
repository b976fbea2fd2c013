"""GPU parity of the routed-MoE path against the oracle.

* moe_align: the integer block tables, bit for bit ("vLLM PR 50949 review",
  moe_fp8.cpp listing: expert_ids / offsets / sorted_ids walk).
* fused_moe_fp8 / fused_moe_mxfp4: bf16 outputs within atol = rtol = 1e-2 of
  the oracle, on the deterministic small-block routing (counts 4, 5, 33, 0, 0,
  12, 1, 73 straddle every tile-class bound; "vLLM PR 50949 review",
  implementation item 4), with every block forced through every tile class,
  with the per-layer average rule, W8A8 and MXFP4 variants, and the GPT-OSS- and
  DeepSeek-shaped workloads on sampled tokens.
"""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_expert_amd as mx
from mxfp4_block_scaled_expert_amd import _lib as L
from mxfp4_block_scaled_expert_amd import ops, synth
from oracle import moe as OM
from oracle.align import moe_align as oracle_align
from tests._util import assert_bf16_close, assert_bf16_close_requant, bf16_bits, f32, u8, gpu

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ align

def _check_align(ids: torch.Tensor, E: int, block_m: int):
    s, e, o, nb = ops.moe_align(ids.to(gpu()), E, block_m)
    torch.cuda.synchronize()
    rs, re, ro, rnb = oracle_align(ids.cpu().numpy(), E, block_m)
    assert int(nb.item()) == rnb
    assert np.array_equal(e.cpu().numpy(), re)
    assert np.array_equal(o.cpu().numpy(), ro)
    assert np.array_equal(s.cpu().numpy(), rs)


@pytest.mark.parametrize("seed", range(6))
def test_align_random(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 3000))
    E = int(rng.choice([1, 3, 8, 64, 256, 512]))
    topk = int(rng.integers(1, min(E, 8) + 1))
    block_m = int(rng.choice([1, 4, 16, 64, 128]))
    ids = torch.from_numpy(np.stack([rng.choice(E, size=topk, replace=False) for _ in range(M)]).astype(np.int32))
    _check_align(ids, E, block_m)


def test_align_small_block_counts_and_skewed_prefill():
    ids, _ = synth.route_counts((4, 5, 33, 0, 0, 12, 1, 73))
    for bm in (4, 16, 32, 128):
        _check_align(ids, 8, bm)
    ids, _ = synth.route_zipf(4096, 256, 8, 1.1, seed=7)
    _check_align(ids, 256, 128)
    ids, _ = synth.route_softmax_topk(32, 128, 4, seed=3)
    _check_align(ids, 128, 128)


# ------------------------------------------------------------------ fused MoE helpers

def _to_np(inp):
    out = {}
    for k in ("w1", "w2", "w1_scale", "w2_scale"):
        t = inp[k]
        out[k] = t.cpu().numpy()
    out["w1_bias"] = None if inp.get("w1_bias") is None else inp["w1_bias"].cpu().numpy()
    return out


def _run_gpu(inp, dispatch=None, **kw):
    if inp["kind"] == "fused_moe_mxfp4":
        return ops.fused_moe_mxfp4(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"],
                                   inp["w2"], inp["w2_scale"], inp["w1_bias"], dispatch=dispatch, **kw)
    return ops.fused_moe_fp8(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"],
                             inp["w2"], inp["w2_scale"], inp.get("w1_bias"), act_quant=inp["act_quant"],
                             dispatch=dispatch, **kw)


def _run_oracle(inp, tokens=None):
    x = bf16_bits(inp["x"])
    ids = inp["topk_ids"].cpu().numpy()
    w = inp["topk_weights"].cpu().numpy()
    if tokens is not None:
        x, ids, w = x[tokens], ids[tokens], w[tokens]
        used = np.unique(ids)
        # only the experts these tokens reach are copied to the host
        remap = {int(e): i for i, e in enumerate(used)}
        ids = np.vectorize(lambda v: remap[int(v)])(ids).astype(np.int32)
        sel = torch.from_numpy(used.astype(np.int64)).to(inp["w1"].device)
        host = {k: inp[k].index_select(0, sel).cpu().numpy() for k in ("w1", "w2", "w1_scale", "w2_scale")}
        host["w1_bias"] = None if inp.get("w1_bias") is None else inp["w1_bias"].index_select(0, sel).cpu().numpy()
    else:
        host = _to_np(inp)
    if inp["kind"] == "fused_moe_mxfp4":
        return OM.fused_moe_mxfp4(x, ids, w, host["w1"], host["w1_scale"], host["w2"], host["w2_scale"],
                                  host["w1_bias"])
    return OM.fused_moe_fp8(x, ids, w, host["w1"], host["w1_scale"], host["w2"], host["w2_scale"],
                            host["w1_bias"], act_quant=inp["act_quant"])


SMALL_BLOCKS = "moe_block_fp8_w8a16_e8_h2048_i1024"


def test_small_expert_blocks_w8a16_per_block_dispatch():
    inp = synth.moe_inputs(SMALL_BLOCKS, seed=1003, device=gpu())
    out = _run_gpu(inp)
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _run_oracle(inp), what="w8a16 counts (4,5,33,0,0,12,1,73)")


@pytest.mark.parametrize("forced", [0, 1, 2, 3, 4])
def test_small_expert_blocks_every_class(forced):
    inp = synth.moe_inputs(SMALL_BLOCKS, seed=1003, device=gpu())
    want = _run_oracle(inp)
    out = _run_gpu(inp, ops.Dispatch(mx.MXQ_DISPATCH_FORCED, forced, 4))
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), want, what=f"forced class {forced}")


@pytest.mark.parametrize("tiny", [mx.MXQ_TINY_MFMA, mx.MXQ_TINY_GEMV])
@pytest.mark.parametrize("kind", ["w8a16", "w8a8", "mxfp4"])
def test_tiny_block_kernels(kind, tiny):
    """Both tiny-block kernels, every block forced through them, each weight format."""
    if kind == "w8a16":
        inp = synth.moe_inputs(SMALL_BLOCKS, seed=1003, device=gpu())
        check = assert_bf16_close
    elif kind == "w8a8":
        inp = synth.moe_inputs(_small_spec("fused_moe_fp8", 300, 16, 4, 512, 256, zipf=1.1, act_quant=True),
                               seed=21, device=gpu())
        check = assert_bf16_close_requant
    else:
        inp = synth.moe_inputs(_small_spec("fused_moe_mxfp4", 40, 8, 4, 2880, 2880), seed=22, device=gpu())
        check = assert_bf16_close
    want = _run_oracle(inp)
    out = _run_gpu(inp, ops.Dispatch(mx.MXQ_DISPATCH_FORCED, 0, 4, tiny))
    torch.cuda.synchronize()
    check(bf16_bits(out), want, what=f"{kind} tiny={tiny}")


def test_layer_average_rule_matches_too():
    inp = synth.moe_inputs(SMALL_BLOCKS, seed=1003, device=gpu())
    out = _run_gpu(inp, ops.Dispatch(mx.MXQ_DISPATCH_LAYER_AVERAGE, 0, 4))
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _run_oracle(inp), what="layer-average dispatch")


def _small_spec(kind, M, E, topk, H, I, zipf=None, act_quant=False):
    spec = dict(kind=kind, M=M, E=E, topk=topk, H=H, I=I, act_quant=act_quant)
    if zipf:
        spec["zipf"] = zipf
    return spec


@pytest.mark.parametrize("forced", [None, 0, 1, 2, 3, 4])
def test_w8a8_skewed_small(forced):
    spec = _small_spec("fused_moe_fp8", 300, 16, 4, 512, 256, zipf=1.1, act_quant=True)
    inp = synth.moe_inputs(spec, seed=11, device=gpu())
    want = _run_oracle(inp)
    out = _run_gpu(inp, None if forced is None else ops.Dispatch(mx.MXQ_DISPATCH_FORCED, forced, 4))
    torch.cuda.synchronize()
    assert_bf16_close_requant(bf16_bits(out), want, what=f"w8a8 forced={forced}")


def test_w8a16_with_bias_and_topk():
    spec = _small_spec("fused_moe_fp8", 77, 12, 3, 384, 256, zipf=0.8)
    inp = synth.moe_inputs(spec, seed=12, device=gpu())
    g = torch.Generator(device="cuda").manual_seed(3)
    inp["w1_bias"] = torch.randn(12, 512, generator=g, device=gpu())
    out = _run_gpu(inp)
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), _run_oracle(inp), what="w8a16 bias topk3")


@pytest.mark.parametrize("forced", [None, 0, 1, 4])
def test_mxfp4_ragged_k(forced):
    spec = _small_spec("fused_moe_mxfp4", 40, 8, 4, 2880, 2880)
    inp = synth.moe_inputs(spec, seed=13, device=gpu())
    want = _run_oracle(inp)
    out = _run_gpu(inp, None if forced is None else ops.Dispatch(mx.MXQ_DISPATCH_FORCED, forced, 4))
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), want, what=f"mxfp4 forced={forced}")


def test_gptoss_decode_workload_sampled_tokens():
    inp = synth.moe_inputs("moe_mxfp4_gptoss_decode_m32", seed=1004, device=gpu())
    out = _run_gpu(inp)
    torch.cuda.synchronize()
    tokens = np.array([0, 13, 31])
    want = _run_oracle(inp, tokens)
    assert_bf16_close(bf16_bits(out[torch.from_numpy(tokens).to(gpu())]), want, what="gpt-oss decode")


def test_zero_tokens():
    spec = _small_spec("fused_moe_fp8", 4, 4, 2, 256, 128)
    inp = synth.moe_inputs(spec, seed=1, device=gpu())
    out = ops.fused_moe_fp8(inp["x"][:0], inp["topk_ids"][:0], inp["topk_weights"][:0], inp["w1"], inp["w1_scale"],
                            inp["w2"], inp["w2_scale"])
    assert out.shape == (0, 256)


@pytest.mark.parametrize("kind", ["w8a16", "mxfp4"])
def test_small_batch_fused_silu_matches_unfused_and_oracle(kind):
    """M <= 32: every block takes the tiny-block kernel and stage 2 computes the SiLU-and-mul while
    staging its rows.  Forcing the tiny class (without a K split) keeps the same kernels with the
    standalone SiLU-and-mul pass, so the two must agree bit for bit; both must match the oracle."""
    if kind == "w8a16":
        spec = _small_spec("fused_moe_fp8", 24, 8, 2, 512, 256)
    else:
        spec = _small_spec("fused_moe_mxfp4", 16, 8, 4, 2880, 2880)
    inp = synth.moe_inputs(spec, seed=41, device=gpu())
    fused = _run_gpu(inp)
    plain = _run_gpu(inp, ops.Dispatch(mx.MXQ_DISPATCH_FORCED, 0, k_split=1))
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), plain.view(torch.int16))
    assert_bf16_close(bf16_bits(fused), _run_oracle(inp), what=f"{kind} fused SiLU")


# ------------------------------------------------------------------ K split (bf16 activations)

@pytest.mark.parametrize("k_split", [1, 2, 8])
@pytest.mark.parametrize("forced", [None, 0, 1, 2, 3, 4])
def test_k_split_small_blocks_every_class(forced, k_split):
    """The small-block W8A16 routing with each tile's K cut into 2 or 8 chunks (fp32 partial
    slices summed after each stage), per block and with every class forced."""
    inp = synth.moe_inputs(SMALL_BLOCKS, seed=1003, device=gpu())
    want = _run_oracle(inp)
    mode = mx.MXQ_DISPATCH_PER_BLOCK if forced is None else mx.MXQ_DISPATCH_FORCED
    out = _run_gpu(inp, ops.Dispatch(mode, forced or 0, k_split=k_split))
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), want, what=f"forced={forced} k_split={k_split}")


@pytest.mark.parametrize("k_split", [2, 4, 8])
@pytest.mark.parametrize("forced", [0, 1, 4])
def test_k_split_mxfp4_ragged_chunks(forced, k_split):
    """MXFP4, K = 2880 in both stages: chunks of 1536 / 768 / 512 columns, the last one ragged
    (a partial 128-wide tile step, a partial 256-wide tiny-kernel step)."""
    spec = _small_spec("fused_moe_mxfp4", 40, 8, 4, 2880, 2880)
    inp = synth.moe_inputs(spec, seed=13, device=gpu())
    want = _run_oracle(inp)
    out = _run_gpu(inp, ops.Dispatch(mx.MXQ_DISPATCH_FORCED, forced, 4, k_split=k_split))
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), want, what=f"mxfp4 forced={forced} k_split={k_split}")


@pytest.mark.parametrize("k_split", [2, 8])
def test_k_split_bias_topk_and_dropped_ids(k_split):
    """The stage-1 bias is added once (by the first chunk); rows with expert ids outside [0, E)
    are dropped as without a split."""
    spec = _small_spec("fused_moe_fp8", 77, 12, 3, 384, 256, zipf=0.8)
    inp = synth.moe_inputs(spec, seed=12, device=gpu())
    g = torch.Generator(device="cuda").manual_seed(3)
    inp["w1_bias"] = torch.randn(12, 512, generator=g, device=gpu())
    inp["topk_ids"][5, 1] = -1
    inp["topk_ids"][9, 0] = 12
    out = _run_gpu(inp, ops.Dispatch(k_split=k_split))
    torch.cuda.synchronize()
    ids = inp["topk_ids"].cpu().numpy()
    keep = ids.copy()
    keep[(ids < 0) | (ids >= 12)] = 0
    w = inp["topk_weights"].clone()
    w[torch.from_numpy((ids < 0) | (ids >= 12)).to(gpu())] = 0.0
    ref_inp = dict(inp, topk_ids=torch.from_numpy(keep).to(gpu()), topk_weights=w)
    assert_bf16_close(bf16_bits(out), _run_oracle(ref_inp), what=f"bias/dropped k_split={k_split}")


@pytest.mark.parametrize("forced", [None, 1, 2, 3, 4])
def test_mxfp4_plain_k_multiple_of_128(forced):
    """MXFP4 with K % 128 == 0 in both stages on the plain layout: the ring-fed tiles copy one
    aligned e8m0 dword per weight row per K step (the tiled layout and K = 2880 take other
    copy paths); bias, top-3, every tile class."""
    spec = _small_spec("fused_moe_mxfp4", 70, 6, 3, 1024, 384)
    inp = synth.moe_inputs(spec, seed=71, device=gpu())
    want = _run_oracle(inp)
    d = None if forced is None else ops.Dispatch(mx.MXQ_DISPATCH_FORCED, forced, 4)
    out = _run_gpu(inp, d)
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(out), want, what=f"mxfp4 plain K%128 forced={forced}")


@pytest.mark.parametrize("kind,H,I", [("fused_moe_fp8", 128, 128), ("fused_moe_fp8", 640, 384),
                                      ("fused_moe_mxfp4", 96, 160)])
def test_ring_tiles_narrow_and_ragged_shapes(kind, H, I):
    """Single-step and ragged K ranges, weight-row counts that end inside a 16-row group of the
    last 128-column tile, a single expert holding every row, every class forced."""
    for forced in (1, 2, 3, 4):
        spec = _small_spec(kind, 50, 1, 1, H, I)
        inp = synth.moe_inputs(spec, seed=H + I + forced, device=gpu())
        want = _run_oracle(inp)
        out = _run_gpu(inp, ops.Dispatch(mx.MXQ_DISPATCH_FORCED, forced, 4))
        torch.cuda.synchronize()
        assert_bf16_close(bf16_bits(out), want, what=f"{kind} H={H} I={I} forced={forced}")


# ------------------------------------------------------------------ self-routed tiles

def _auto_and_sorted(inp, layout="plain", **d):
    outs = []
    for srt in (mx.MXQ_SORT_AUTO, mx.MXQ_SORT_ALWAYS):
        dd = ops.Dispatch(sort=srt, **d)
        if inp["kind"] == "fused_moe_mxfp4":
            outs.append(ops.fused_moe_mxfp4(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"],
                                            inp["w1_scale"], inp["w2"], inp["w2_scale"], inp["w1_bias"],
                                            weight_layout=layout, dispatch=dd))
        else:
            outs.append(_run_gpu(inp, dd))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("case", ["small_blocks", "multi_block_expert", "r1024", "e512_forced", "r2048_e512",
                                  "r2048_mxfp4", "mxfp4"])
def test_self_routed_tiles_match_sorted(case):
    """Small bf16 routings without a tiny class skip the sort: each tile finds its rows from the
    routing ids (the sort's expert order, cut into 64-row blocks).  Every row's products are the
    sorted path's, so the outputs equal it bit for bit (and the oracle's within tolerance): the
    small-block routing (empty experts, blocks in several classes), an expert holding several
    128-row blocks, 1024 routed rows, E = 512 with forced classes, the largest self-routed
    routing (2048 routed rows over 512 experts), 2048 MXFP4 routed rows, and MXFP4 on both
    weight layouts."""
    runs = [{}]
    if case == "small_blocks":
        inp = synth.moe_inputs(SMALL_BLOCKS, seed=1003, device=gpu())
        runs = [{}, dict(k_split=1), dict(k_split=8)]
    elif case == "multi_block_expert":
        inp = synth.moe_inputs(_small_spec("fused_moe_fp8", 300, 4, 2, 256, 128, zipf=1.5), seed=61, device=gpu())
        assert np.bincount(inp["topk_ids"].cpu().numpy().ravel(), minlength=4).max() > 256
    elif case == "r1024":
        inp = synth.moe_inputs(_small_spec("fused_moe_fp8", 256, 64, 4, 256, 256, zipf=0.9), seed=62, device=gpu())
    elif case == "e512_forced":
        inp = synth.moe_inputs(_small_spec("fused_moe_fp8", 300, 512, 2, 128, 128), seed=63, device=gpu())
        runs = [dict(tiny_max_rows=0)] + [dict(mode=mx.MXQ_DISPATCH_FORCED, forced_class=c) for c in (1, 2, 3, 4)]
    elif case == "r2048_e512":
        # the largest self-routed routing: 2048 routed rows over 512 experts (its routing ids and
        # counts fill the most LDS)
        inp = synth.moe_inputs(_small_spec("fused_moe_fp8", 1024, 512, 2, 128, 128, zipf=1.0), seed=64, device=gpu())
        runs = [dict(tiny_max_rows=0), dict(mode=mx.MXQ_DISPATCH_FORCED, forced_class=4)]
    elif case == "r2048_mxfp4":
        inp = synth.moe_inputs(_small_spec("fused_moe_mxfp4", 512, 32, 4, 256, 256), seed=65, device=gpu())
    else:
        inp = synth.moe_inputs(_small_spec("fused_moe_mxfp4", 40, 8, 4, 2880, 2880), seed=13, device=gpu())
        runs = [{}, dict(mode=mx.MXQ_DISPATCH_FORCED, forced_class=1), dict(k_split=1)]
    want = _run_oracle(inp)
    M, H = inp["x"].shape
    wts = L.MXQ_WEIGHTS_MXFP4 if inp["kind"] == "fused_moe_mxfp4" else L.MXQ_WEIGHTS_FP8_BLOCK
    for d in runs:
        # (MXFP4 with K = 2880 self-routes on the tiled layout only)
        plan = ops.fused_moe_plan(M, H, inp["I"], inp["E"], inp["topk"], wts, dispatch=ops.Dispatch(**d),
                                  weight_layout="tiled" if case == "mxfp4" else "plain")
        assert plan["path"] == "self_routed", (case, d, plan)
        auto, srt = _auto_and_sorted(inp, **d)
        assert torch.equal(auto.view(torch.int16), srt.view(torch.int16)), (case, d)
        assert_bf16_close(bf16_bits(auto), want, what=f"self-routed {case} {d}")
        if case == "mxfp4":
            tin = dict(inp, w1=ops.moe_prepack(inp["w1"]), w2=ops.moe_prepack(inp["w2"]),
                       w1_scale=ops.moe_prepack_scales(inp["w1_scale"]),
                       w2_scale=ops.moe_prepack_scales(inp["w2_scale"]))
            for t in _auto_and_sorted(tin, "tiled", **d):
                assert torch.equal(t.view(torch.int16), auto.view(torch.int16)), (case, "tiled", d)


# ------------------------------------------------------------------ SiLU-and-mul in the stage-1 epilogue

@pytest.mark.parametrize("case", ["small_blocks", "top1_dropped", "bias_top3_dropped", "m256", "mxfp4", "mxfp4_top1",
                                  "forced"])
def test_fused_silu_stage1_matches_unfused(case):
    """With bf16 activations, stage 1 wholly on the direct-to-LDS tiles and whole K ranges, each
    stage-1 tile pairs 64 gate with the matching 64 up weight rows and writes ic1 itself.  The
    same call with MXQ_FUSE_NONE (ic0 written, then the standalone SiLU-and-mul) gives the same
    bits; both match the oracle.  Self-routed and sorted tiles, plain and tiled weights, a bias
    on both halves, dropped ids, and every tile class forced.  With top-1 routing the self-routed
    stage 2 also folds the combine into its epilogue (zeroing the rows of dropped tokens)."""
    extra = [{}]
    if case == "small_blocks":
        inp = synth.moe_inputs(SMALL_BLOCKS, seed=1003, device=gpu())
        runs = [{}, dict(k_split=1), dict(k_split=1, sort=mx.MXQ_SORT_ALWAYS)]
    elif case == "top1_dropped":
        inp = synth.moe_inputs(SMALL_BLOCKS, seed=1003, device=gpu())
        inp["topk_ids"][3, 0] = -1
        inp["topk_ids"][40, 0] = 8
        inp["topk_ids"][127, 0] = -7
        runs = [{}, dict(k_split=1), dict(sort=mx.MXQ_SORT_ALWAYS)]
    elif case == "bias_top3_dropped":
        inp = synth.moe_inputs(_small_spec("fused_moe_fp8", 77, 12, 3, 384, 256, zipf=0.8), seed=12, device=gpu())
        g = torch.Generator(device="cuda").manual_seed(3)
        inp["w1_bias"] = torch.randn(12, 512, generator=g, device=gpu())
        inp["topk_ids"][5, 1] = -1
        inp["topk_ids"][9, 0] = 12
        runs = [dict(k_split=1), dict(k_split=1, sort=mx.MXQ_SORT_ALWAYS)]
    elif case == "m256":
        inp = synth.moe_inputs(_small_spec("fused_moe_fp8", 256, 8, 2, 512, 256, zipf=1.2), seed=81, device=gpu())
        runs = [{}, dict(sort=mx.MXQ_SORT_ALWAYS)]
    elif case == "mxfp4":
        inp = synth.moe_inputs(_small_spec("fused_moe_mxfp4", 40, 8, 4, 2880, 2880), seed=13, device=gpu())
        runs = [dict(k_split=1)]
        extra = [{}, {"tiled": True}]
    elif case == "mxfp4_top1":
        # top-1 MXFP4 with a w1 bias and a ragged K (I = H = 2880): both epilogue folds
        inp = synth.moe_inputs(_small_spec("fused_moe_mxfp4", 96, 8, 1, 2880, 2880), seed=14, device=gpu())
        runs = [{}, dict(sort=mx.MXQ_SORT_ALWAYS)]
        extra = [{}, {"tiled": True}]
    else:
        inp = synth.moe_inputs(_small_spec("fused_moe_fp8", 70, 6, 3, 1024, 384), seed=71, device=gpu())
        runs = [dict(mode=mx.MXQ_DISPATCH_FORCED, forced_class=c, k_split=1) for c in (1, 2, 3, 4)]
    ids = inp["topk_ids"].cpu().numpy()
    E = inp["E"]
    ref = inp
    if case in ("bias_top3_dropped", "top1_dropped"):
        keep = ids.copy()
        keep[(ids < 0) | (ids >= E)] = 0
        w = inp["topk_weights"].clone()
        w[torch.from_numpy((ids < 0) | (ids >= E)).to(gpu())] = 0.0
        ref = dict(inp, topk_ids=torch.from_numpy(keep).to(gpu()), topk_weights=w)
    want = _run_oracle(ref)
    for ex in extra:
        src = inp
        layout = "plain"
        if ex.get("tiled"):
            src = dict(inp, w1=ops.moe_prepack(inp["w1"]), w2=ops.moe_prepack(inp["w2"]),
                       w1_scale=ops.moe_prepack_scales(inp["w1_scale"]),
                       w2_scale=ops.moe_prepack_scales(inp["w2_scale"]))
            layout = "tiled"
        for d in runs:
            outs = []
            for fuse in (mx.MXQ_FUSE_AUTO, mx.MXQ_FUSE_NONE):
                dd = ops.Dispatch(fuse=fuse, **d)
                if src["kind"] == "fused_moe_mxfp4":
                    outs.append(ops.fused_moe_mxfp4(src["x"], src["topk_ids"], src["topk_weights"], src["w1"],
                                                    src["w1_scale"], src["w2"], src["w2_scale"], src["w1_bias"],
                                                    weight_layout=layout, dispatch=dd))
                else:
                    outs.append(_run_gpu(src, dd))
            torch.cuda.synchronize()
            assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), (case, layout, d)
            assert_bf16_close(bf16_bits(outs[0]), want, what=f"fused SiLU {case} {layout} {d}")


def test_output_buffer_in_a_larger_allocation():
    """The top-1 combine folded into stage 2 writes exactly the output rows: an output window
    inside a zeroed larger buffer (16-byte aligned, as every pointer must be) gets the same bits
    as a fresh output and the bytes around it stay zero; an output 8 bytes off that alignment
    is refused before anything runs."""
    inp = synth.moe_inputs(SMALL_BLOCKS, seed=1003, device=gpu())
    M, H = inp["x"].shape
    ref = _run_gpu(inp)
    buf = torch.zeros(M * H + 16, dtype=torch.bfloat16, device=gpu())
    out = buf[8:8 + M * H].view(M, H)
    got = _run_gpu(inp, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.all(buf[:8] == 0) and torch.all(buf[8 + M * H:] == 0)
    with pytest.raises(ValueError):
        _run_gpu(inp, out=buf[4:4 + M * H].view(M, H))


@pytest.mark.parametrize("seed", range(24))
def test_random_small_routings_all_paths_agree(seed):
    """Seeded random small bf16 routings (tokens, experts, top-k, sizes, Zipf skew, a few dropped
    ids, FP8 or MXFP4 weights, per-block / forced-class / layer-average dispatch): the default
    call (self-routed where it applies, with its epilogue folds), the call with the sort kept and
    the call with no fusion give the same bits, and all match the oracle."""
    rng = np.random.default_rng(1000 + seed)
    kind = "fused_moe_mxfp4" if seed % 3 == 2 else "fused_moe_fp8"
    E = int(rng.choice([1, 2, 5, 8, 16, 40]))
    topk = int(rng.integers(1, min(E, 4) + 1))
    M = int(rng.integers(1, 200))
    if kind == "fused_moe_mxfp4":  # ragged K steps (multiples of 32)
        H = int(rng.choice([96, 160, 256, 352]))
        I = int(rng.choice([96, 160, 256, 352]))
    else:
        H = int(rng.choice([128, 256, 384]))
        I = int(rng.choice([128, 256, 512]))
    spec = _small_spec(kind, M, E, topk, H, I, zipf=float(rng.choice([0.0, 0.8, 1.3])) or None)
    inp = synth.moe_inputs(spec, seed=seed + 7, device=gpu())
    ids = inp["topk_ids"].cpu().numpy()
    drop = rng.random(ids.shape) < 0.03
    if drop.any():
        bad = np.where(rng.random(ids.shape) < 0.5, -1, E)
        ids = np.where(drop, bad, ids).astype(np.int32)
        inp["topk_ids"] = torch.from_numpy(ids).to(gpu())
    keep = np.where((ids < 0) | (ids >= E), 0, ids).astype(np.int32)
    w = inp["topk_weights"].clone()
    w[torch.from_numpy((ids < 0) | (ids >= E)).to(gpu())] = 0.0
    want = _run_oracle(dict(inp, topk_ids=torch.from_numpy(keep).to(gpu()), topk_weights=w))
    mode = [{}, {}, dict(mode=mx.MXQ_DISPATCH_FORCED, forced_class=int(rng.integers(0, 5))),
            dict(mode=mx.MXQ_DISPATCH_LAYER_AVERAGE)][seed % 4]
    outs = [_run_gpu(inp, ops.Dispatch(sort=so, fuse=fu, **mode))
            for so, fu in ((mx.MXQ_SORT_AUTO, mx.MXQ_FUSE_AUTO), (mx.MXQ_SORT_ALWAYS, mx.MXQ_FUSE_AUTO),
                           (mx.MXQ_SORT_AUTO, mx.MXQ_FUSE_NONE))]
    torch.cuda.synchronize()
    what = f"seed {seed}: {kind} M={M} E={E} topk={topk} H={H} I={I} {mode}"
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16)), what
    assert_bf16_close(bf16_bits(outs[0]), want, what=what)


@pytest.mark.parametrize("seed", range(8))
def test_random_w8a8_routings(seed):
    """Seeded random W8A8 routings (tokens 1..600 so that blocks fill every class and the
    128-row tile, 2..64 experts, top-1..top-8, Zipf skew) against the oracle (the requantised
    end-to-end bar; the stages are held to the strict bar in the stage-by-stage tests)."""
    rng = np.random.default_rng(3000 + seed)
    E = int(rng.choice([2, 6, 16, 64]))
    topk = int(rng.integers(1, min(E, 8) + 1))
    M = int(rng.integers(1, 601))
    H = int(rng.choice([128, 256, 512]))
    I = int(rng.choice([128, 256, 384]))
    spec = _small_spec("fused_moe_fp8", M, E, topk, H, I, zipf=float(rng.choice([0.0, 1.1])) or None, act_quant=True)
    inp = synth.moe_inputs(spec, seed=seed + 17, device=gpu())
    out = _run_gpu(inp)
    torch.cuda.synchronize()
    assert_bf16_close_requant(bf16_bits(out), _run_oracle(inp), what=f"w8a8 seed {seed}: M={M} E={E} topk={topk} H={H} I={I}")
