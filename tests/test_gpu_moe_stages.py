"""Stage-by-stage GPU parity of the routed MoE against the oracle.

Every intermediate of a fused-MoE call is read back from the caller-owned
workspace (``mxq_fused_moe_workspace_layout`` names where each lives) and held
to its own bar, each stage computed by the oracle from the GPU's own input to
that stage:

* the align tables and the 1x128 quantisation of x: bit for bit;
* stage 1 (``ic0``, bf16): within atol = rtol = 1e-2 of the oracle's stage 1;
* the SiLU-and-mul (``mxq_silu_and_mul``, bf16): within 1e-2 of the oracle's
  (its exponential is the one unpinned piece); its W8A8 re-quantisation
  (``ic1`` codes and scales): bit for bit against the oracle's quantiser applied
  to the GPU's own bf16 product;
* stage 2 (``y``, fp32) and the top-k combine (bf16 out): within 1e-2 of the
  oracle's stage 2 and combine computed from the GPU's own ``ic1``.

Sources: "vLLM PR 50949 review", implementation items 2 and 4 and the
moe_fp8.cpp listing (stage 1 into the 2N-wide intermediate, the activation,
stage 2; the 1e-2 bar against the float reference); "SGLang PR 35605 review",
implementation item 1 (activations quantised per token per 128 columns).
"""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_expert_amd as mx
from mxfp4_block_scaled_expert_amd import _lib as L
from mxfp4_block_scaled_expert_amd import ops, synth
from oracle import codecs as OC
from oracle import moe as OM
from oracle.align import moe_align as oracle_align
from oracle.quant import group_quant_f32, per_token_group_quant_fp8 as oracle_quant
from tests._util import assert_bf16_close, assert_bf16_close_requant, bf16_bits, bits_to_float, f32, u8, gpu

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ SiLU-and-mul

@pytest.mark.parametrize("rows,I,pad", [(300, 256, 0), (17, 2048, 64), (1, 128, 8)])
def test_silu_and_mul_and_requant(rows, I, pad):
    g = torch.Generator(device="cuda").manual_seed(rows + I)
    ic0 = torch.randn(rows, 2 * I + pad, generator=g, device=gpu()) * 3
    ic0[0, :128] = 0.0  # a zero gate group: h = 0, codes 0, scale 1e-10 / 448
    ic0[-1, I:I + 128] *= 1e4  # a wide-range group
    ic0 = ic0.to(torch.bfloat16)[:, :2 * I]  # row stride 2I + pad when pad > 0
    h = ops.silu_and_mul(ic0)
    q, s = ops.silu_and_mul(ic0, quant=True)
    torch.cuda.synchronize()
    want = OM.silu_mul_bf16(bits_to_float(bf16_bits(ic0)), I)
    assert_bf16_close(bf16_bits(h), want, what="silu_and_mul")
    # the re-quantisation of the GPU's own bf16 product: bit for bit
    q_ref, s_ref = oracle_quant(bf16_bits(h))
    assert np.array_equal(f32(s).view(np.uint32), s_ref.view(np.uint32)), "ic1 scales differ"
    assert np.array_equal(u8(q), q_ref), "ic1 codes differ"


# ------------------------------------------------------------------ workspace readers

def _region(ws: torch.Tensor, off: int, n: int, dtype) -> torch.Tensor:
    assert off >= 0
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype)


class Stages:
    """The W8A8 intermediates a fused-MoE call left in its workspace."""

    def __init__(self, ws, M, H, I, E, topk):
        lay = ops.fused_moe_workspace_layout(M, H, I, E, topk, L.MXQ_WEIGHTS_FP8_BLOCK, True)
        R = M * topk
        self.bm = bm = lay["block_m"]
        mb = ops.moe_max_blocks(M, topk, E, bm)
        self.nb = int(_region(ws, lay["num_blocks"], 1, torch.int32).item())
        self.expert_ids = _region(ws, lay["expert_ids"], mb, torch.int32).cpu().numpy()
        self.offsets = _region(ws, lay["offsets"], mb + 1, torch.int32).cpu().numpy()
        self.sorted_ids = _region(ws, lay["sorted_ids"], mb * bm, torch.int32).cpu().numpy()
        self.ws, self.lay, self.R, self.H, self.I, self.M = ws, lay, R, H, I, M
        # compact row -> flat routed id, and -> expert
        self.flat_of = np.full(R, -1, np.int64)
        self.expert_of = np.full(R, -1, np.int64)
        for b in range(self.nb):
            o0, o1 = int(self.offsets[b]), int(self.offsets[b + 1])
            self.flat_of[o0:o1] = self.sorted_ids[b * bm: b * bm + (o1 - o0)]
            self.expert_of[o0:o1] = self.expert_ids[b]
        self.compact_of = np.full(R, -1, np.int64)
        self.compact_of[self.flat_of[self.flat_of >= 0]] = np.nonzero(self.flat_of >= 0)[0]

    def qx(self):
        return (u8(_region(self.ws, self.lay["qx"], self.M * self.H, torch.uint8)).reshape(self.M, self.H),
                f32(_region(self.ws, self.lay["sx"], self.M * (self.H // 128), torch.float32)).reshape(self.M, -1))

    def ic0_rows(self, compact):
        t = _region(self.ws, self.lay["ic0"], self.R * 2 * self.I, torch.bfloat16).view(self.R, 2 * self.I)
        return t[torch.from_numpy(np.asarray(compact)).to(gpu())]

    def ic1_rows(self, compact):
        q = _region(self.ws, self.lay["ic1_q"], self.R * self.I, torch.uint8).view(self.R, self.I)
        s = _region(self.ws, self.lay["ic1_s"], self.R * (self.I // 128), torch.float32).view(self.R, -1)
        idx = torch.from_numpy(np.asarray(compact)).to(gpu())
        return u8(q[idx]), f32(s[idx])

    def y_rows(self, flat):
        t = _region(self.ws, self.lay["y"], self.R * self.H, torch.float32).view(self.R, self.H)
        return f32(t[torch.from_numpy(np.asarray(flat)).to(gpu())])


def _host_weights(inp, which, e):
    """Dequantised fp32 weights `which` ("w1" / "w2") of expert e (plain-layout tensors)."""
    return OM.dequant_fp8_expert(u8(inp[which][e]), f32(inp[which + "_scale"][e]))


def _check_tables(st: Stages, ids: np.ndarray, E: int):
    rs, re, ro, rnb = oracle_align(ids, E, st.bm)
    assert st.nb == rnb
    assert np.array_equal(st.expert_ids[:rnb], re[:rnb])
    assert np.array_equal(st.offsets[:rnb + 1], ro[:rnb + 1])
    for b in range(rnb):  # real slots only (the fused path writes no pad slots)
        n = int(ro[b + 1] - ro[b])
        assert np.array_equal(st.sorted_ids[b * st.bm: b * st.bm + n], rs[b * st.bm: b * st.bm + n]), f"block {b}"


def _check_stages(inp, st: Stages, out: torch.Tensor, stage1_experts, tokens):
    """The stage checks described in the module docstring.  Stage 1 on every row of
    `stage1_experts`; the SiLU re-quantisation, stage 2 and the combine on the routed rows of
    `tokens`."""
    M, H, I, topk = st.M, st.H, st.I, inp["topk"]
    ids = inp["topk_ids"].cpu().numpy()
    wts = inp["topk_weights"].cpu().numpy()
    xb = bf16_bits(inp["x"])
    # x quantised: bit for bit (whole tensor)
    qx, sx = st.qx()
    q_ref, s_ref = oracle_quant(xb)
    assert np.array_equal(sx.view(np.uint32), s_ref.view(np.uint32)), "x scales differ"
    assert np.array_equal(qx, q_ref), "x codes differ"
    x_deq = (OC.E4M3_TABLE[q_ref].astype(np.float32) * np.repeat(s_ref, 128, axis=1)).astype(np.float32)


    # stage 1, whole experts
    for e in stage1_experts:
        compact = np.nonzero(st.expert_of == e)[0]
        if compact.size == 0:
            continue
        toks = st.flat_of[compact] // topk
        want = OM.stage1_rows(x_deq[toks], _host_weights(inp, "w1", e))
        got = bf16_bits(st.ic0_rows(compact))
        assert_bf16_close(got, want, what=f"stage 1 expert {e} ({compact.size} rows)")

    # routed rows of the sampled tokens
    flat = (np.asarray(tokens)[:, None] * topk + np.arange(topk)[None, :]).reshape(-1)
    compact = st.compact_of[flat]
    assert np.all(compact >= 0)
    ic0 = st.ic0_rows(compact)
    h = ops.silu_and_mul(ic0)
    torch.cuda.synchronize()
    assert_bf16_close(bf16_bits(h), OM.silu_mul_bf16(bits_to_float(bf16_bits(ic0)), I), what="silu(ic0)")
    q1, s1 = st.ic1_rows(compact)
    q1_ref, s1_ref, a2 = OM.quant_rows(bf16_bits(h))
    assert np.array_equal(s1.view(np.uint32), s1_ref.view(np.uint32)), "ic1 scales differ"
    assert np.array_equal(q1, q1_ref), "ic1 codes differ"
    # stage 2 from the GPU's ic1, then the combine
    y_ref = np.zeros((flat.size, H), np.float32)
    fl_e = ids.reshape(-1)[flat]
    for e in np.unique(fl_e):
        sel = np.nonzero(fl_e == e)[0]
        y_ref[sel] = OM.stage2_rows(a2[sel], _host_weights(inp, "w2", int(e)))
    y_got = st.y_rows(flat)
    assert_bf16_close(OC.f32_to_bf16(y_got), OC.f32_to_bf16(y_ref), what="stage 2 (y)")
    out_ref = OM.combine(y_ref, wts[tokens])
    assert_bf16_close(bf16_bits(out[torch.from_numpy(np.asarray(tokens)).to(gpu())]), out_ref,
                      what="combine (out)")


def _run_fp8(inp, ws, layout="plain", dispatch=None):
    src = inp
    if layout == "tiled":
        src = dict(inp)
        src["w1"] = ops.moe_prepack(inp["w1"])
        src["w2"] = ops.moe_prepack(inp["w2"])
    out = ops.fused_moe_fp8(src["x"], src["topk_ids"], src["topk_weights"], src["w1"], src["w1_scale"], src["w2"],
                            src["w2_scale"], None, act_quant=True, workspace=ws, weight_layout=layout,
                            dispatch=dispatch)
    torch.cuda.synchronize()
    return out


def _spec(M, E, topk, H, I, zipf=1.1):
    return dict(kind="fused_moe_fp8", M=M, E=E, topk=topk, H=H, I=I, zipf=zipf, act_quant=True)


@pytest.mark.parametrize("forced", [None, 0, 1, 2, 3, 4])
@pytest.mark.parametrize("layout", ["plain", "tiled"])
@pytest.mark.parametrize("H", [512, 640])
def test_w8a8_moe_stage_by_stage(forced, layout, H):
    """A skewed routing whose blocks straddle every class bound, every class forced.  H = 640:
    stage 2's last column tile is 128 wide, which the column-width rule sends to the 128-wide
    tile while the other column tiles of the same blocks take the 256-wide one."""
    M, I, E, topk = 300, 256, 16, 4
    inp = synth.moe_inputs(_spec(M, E, topk, H, I), seed=11, device=gpu())
    ws = ops.fused_moe_workspace(M, H, I, E, topk, L.MXQ_WEIGHTS_FP8_BLOCK, True, gpu())
    d = None if forced is None else ops.Dispatch(mx.MXQ_DISPATCH_FORCED, forced, 4)
    out = _run_fp8(inp, ws, layout, d)
    st = Stages(ws, M, H, I, E, topk)
    _check_tables(st, inp["topk_ids"].cpu().numpy(), E)
    _check_stages(inp, st, out, stage1_experts=range(E), tokens=np.arange(M))
    # the end-to-end comparison with the oracle's own chain (re-quantisation of its own ic1)
    from tests.test_gpu_moe import _run_oracle
    assert_bf16_close_requant(bf16_bits(out), _run_oracle(inp), what="end to end")


def test_deepseek_prefill_stage_by_stage_sampled():
    """The DeepSeek-shaped W8A8 prefill (E = 256, top-8, H = 7168, I = 2048, 4096 tokens, Zipf
    1.1) on the tiled layout the benchmark times.  Stage 1 on every row of the hottest expert
    (its first, middle and last blocks included) and of experts owning a <= 16-row and a
    17-64-row block; the re-quantisation, stage 2 and the combine on 64 tokens: rows of those
    blocks plus tokens whose experts are mostly among the popular ones."""
    name = "moe_block_fp8_w8a8_deepseek_prefill_m4096"
    inp = synth.moe_inputs(name, seed=1005, device=gpu())
    M, H, I, E, topk = 4096, 7168, 2048, 256, 8
    ws = ops.fused_moe_workspace(M, H, I, E, topk, L.MXQ_WEIGHTS_FP8_BLOCK, True, gpu())
    out = _run_fp8(inp, ws, "tiled")
    st = Stages(ws, M, H, I, E, topk)
    ids = inp["topk_ids"].cpu().numpy()
    _check_tables(st, ids, E)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    hot = int(np.argmax(counts))
    last = counts - (np.ceil(counts / st.bm).astype(int) - 1) * st.bm  # rows of each expert's last block
    small = int(np.nonzero((counts > 0) & (last <= 16))[0][0])
    mid = int(np.nonzero((last > 16) & (last <= 64))[0][0])
    stage1 = [hot, small, mid]
    tok = set()
    for e in stage1:
        rows = np.nonzero(st.expert_of == e)[0]
        for c in (rows[0], rows[len(rows) // 2], rows[-1], rows[min(len(rows) - 1, st.bm)]):
            tok.add(int(st.flat_of[c] // topk))
    # fill up to 64 tokens with those whose experts are the most popular (bounded host work)
    rank = np.argsort(np.argsort(-counts))
    score = rank[ids].max(axis=1)
    for t in np.argsort(score, kind="stable"):
        if len(tok) >= 64:
            break
        tok.add(int(t))
    _check_stages(inp, st, out, stage1_experts=stage1, tokens=np.array(sorted(tok)))
    # run-to-run determinism (no float atomics anywhere on the path)
    out2 = _run_fp8(inp, ws, "tiled")
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("M,E,topk", [(1100, 40, 4), (1025, 9, 8), (4096, 512, 2)])
def test_many_rows_multi_workgroup_sort(M, E, topk):
    """More than 4096 routed rows: the sort runs as a histogram pass, the tables in one workgroup
    and a scatter pass.  Its tables (a ragged last chunk, few and many experts) equal the
    oracle's bit for bit."""
    H, I = 256, 128
    inp = synth.moe_inputs(_spec(M, E, topk, H, I), seed=M + E, device=gpu())
    ws = ops.fused_moe_workspace(M, H, I, E, topk, L.MXQ_WEIGHTS_FP8_BLOCK, True, gpu())
    _run_fp8(inp, ws, "plain")
    st = Stages(ws, M, H, I, E, topk)
    _check_tables(st, inp["topk_ids"].cpu().numpy(), E)


def test_many_rows_sort_drops_ids_outside_the_expert_range():
    """Ids -1 and E drop their rows in the multi-workgroup sort as in the one-workgroup sort of
    mxq_moe_align (the oracle rejects such ids; the one-workgroup sort is pinned to it on valid
    routings): same block tables, same real slots."""
    M, E, topk, H, I = 1100, 40, 4, 256, 128
    inp = synth.moe_inputs(_spec(M, E, topk, H, I), seed=77, device=gpu())
    ids = inp["topk_ids"].clone()
    ids[3, 0] = -1
    ids[M - 1, topk - 1] = E
    ids[600, 2] = 1 << 20
    inp["topk_ids"] = ids
    ws = ops.fused_moe_workspace(M, H, I, E, topk, L.MXQ_WEIGHTS_FP8_BLOCK, True, gpu())
    _run_fp8(inp, ws, "plain")
    st = Stages(ws, M, H, I, E, topk)
    s, e, o, nb = ops.moe_align(ids, E, st.bm)
    torch.cuda.synchronize()
    nb = int(nb.item())
    s, e, o = s.cpu().numpy(), e.cpu().numpy(), o.cpu().numpy()
    assert st.nb == nb and o[nb] == M * topk - 3
    assert np.array_equal(st.expert_ids[:nb], e[:nb]) and np.array_equal(st.offsets[:nb + 1], o[:nb + 1])
    for b in range(nb):
        n = int(o[b + 1] - o[b])
        assert np.array_equal(st.sorted_ids[b * st.bm: b * st.bm + n], s[b * st.bm: b * st.bm + n]), f"block {b}"


# ------------------------------------------------------------------ GPT-OSS decode, every token

def test_gptoss_decode_every_token_both_layouts():
    from tests.test_gpu_moe import _run_oracle
    inp = synth.moe_inputs("moe_mxfp4_gptoss_decode_m32", seed=1004, device=gpu())
    plain = ops.fused_moe_mxfp4(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"],
                                inp["w2"], inp["w2_scale"], inp["w1_bias"])
    tiled = ops.fused_moe_mxfp4(inp["x"], inp["topk_ids"], inp["topk_weights"], ops.moe_prepack(inp["w1"]),
                                ops.moe_prepack_scales(inp["w1_scale"]), ops.moe_prepack(inp["w2"]),
                                ops.moe_prepack_scales(inp["w2_scale"]), inp["w1_bias"], weight_layout="tiled")
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), tiled.view(torch.int16))
    assert_bf16_close(bf16_bits(tiled), _run_oracle(inp), what="gpt-oss decode, all 32 tokens")


# ------------------------------------------------------------------ extreme e8m0 scales

def _extreme_mx_inputs(E, H, I, M, topk, w1_codes, w2_codes, x_exp, seed, device=None):
    """MXFP4 experts whose e8m0 scale codes are drawn from the given ranges; x scaled by 2^x_exp
    (magnitudes at least 2^x_exp, so no activation is a bf16 subnormal)."""
    g = torch.Generator().manual_seed(seed)
    ids, w = synth.route_softmax_topk(M, E, topk, seed + 1)
    mag = (1.0 + torch.rand(M, H, generator=g)) * torch.where(torch.rand(M, H, generator=g) < 0.5, -1.0, 1.0)
    x = (mag * 2.0 ** x_exp).to(torch.bfloat16)
    w1 = torch.randint(0, 256, (E, 2 * I, H // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    w2 = torch.randint(0, 256, (E, H, I // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    s1 = torch.randint(w1_codes[0], w1_codes[1] + 1, (E, 2 * I, H // 32), generator=g, dtype=torch.int32)
    s2 = torch.randint(w2_codes[0], w2_codes[1] + 1, (E, H, I // 32), generator=g, dtype=torch.int32)
    # above 2^125 only element magnitudes up to 1.5 stay finite in fp32 (6 * 2^127 overflows)
    for wq, sq in ((w1, s1), (w2, s2)):
        big = (sq > 252).repeat_interleave(16, dim=2)
        wq[big] &= 0xBB
    dev = device if device is not None else gpu()
    return {"x": x.to(dev), "topk_ids": ids.to(dev), "topk_weights": w.to(dev), "w1": w1.to(dev),
            "w1_scale": s1.to(torch.uint8).to(dev), "w2": w2.to(dev), "w2_scale": s2.to(torch.uint8).to(dev),
            "w1_bias": None, "E": E, "topk": topk, "H": H, "I": I, "act_quant": False, "kind": "fused_moe_mxfp4"}


def _assert_close_at_scale(got_bits, want_bits, what):
    """The 1e-2 bar applied at the output's own scale: both sides multiplied by the power of two
    that brings the reference's largest magnitude to about 1 (exact for these values)."""
    g = bits_to_float(got_bits).astype(np.float64)
    w = bits_to_float(want_bits).astype(np.float64)
    assert np.all(np.isfinite(w)) and np.all(np.isfinite(g)), what
    k = -int(np.floor(np.log2(np.abs(w).max())))
    gs, ws = np.ldexp(g, k), np.ldexp(w, k)
    bad = np.abs(gs - ws) > 1e-2 + 1e-2 * np.abs(ws)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside the band at scale 2^{-k}"


CASES_E8M0 = {
    # w1 scales 2^103..2^127 against activations ~2^-120; w2 scales 2^-126..2^-107
    "high_w1_low_w2": ((230, 254), (1, 20), -120),
    # w1 scales 2^-126..2^-107 against activations ~2^100; w2 scales 2^103..2^107
    "low_w1_high_w2": ((1, 20), (230, 234), 100),
}


@pytest.mark.parametrize("case", sorted(CASES_E8M0))
@pytest.mark.parametrize("forced", [None, 0, 1, 4, "gemv"])
def test_mxfp4_extreme_scale_codes(case, forced):
    """e8m0 codes near both ends of the range (2^-126 .. 2^127) decode exactly in every
    kernel that reads MX scales: the expert-streaming path (default at this size), the tiny
    MFMA kernel, the vector-ALU GEMV, and the 16- and 128-row tiles."""
    from tests.test_gpu_moe import _run_oracle
    c1, c2, xe = CASES_E8M0[case]
    inp = _extreme_mx_inputs(8, 256, 256, 24, 2, c1, c2, xe, seed=sum(c1) + sum(c2))
    want = _run_oracle(inp)
    if forced == "gemv":
        d = ops.Dispatch(mx.MXQ_DISPATCH_FORCED, 0, 16, mx.MXQ_TINY_GEMV)
    else:
        d = None if forced is None else ops.Dispatch(mx.MXQ_DISPATCH_FORCED, forced, 16)
    out = ops.fused_moe_mxfp4(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"],
                              inp["w2"], inp["w2_scale"], None, dispatch=d)
    torch.cuda.synchronize()
    _assert_close_at_scale(bf16_bits(out), want, f"{case} forced={forced}")
