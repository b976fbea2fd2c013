"""Pins for the oracle routed fused-MoE.

(i)   one expert, topk=1 equals the dense oracle GEMMs chained with torch's
      SiLU -- bit for bit, W8A16 and W8A8;
(ii)  a per-token loop with no expert sorting gives the same bits;
(iii) permuting tokens permutes the output; relabelling experts (weights and
      ids together) leaves it unchanged;
(iv)  experts that receive no rows have no effect, even when their weights are
      NaN codes ("vLLM PR 50949 review", implementation item 3: empty expert
      blocks are skipped);
(v)   identical experts with routing weights summing to one reproduce the
      dense MLP;
(vi)  MXFP4 weights whose values are also e4m3 values give exactly the FP8
      W8A16 result -- pins the e2m1 unpacking order, the e8m0 scale indexing
      and the bias path against the torch-pinned FP8 path.
"""

import numpy as np
import pytest
import torch

from oracle import codecs as C
from oracle import dense as D
from oracle import moe as MOE
from oracle.quant import per_token_group_quant_fp8


def _bf16(x) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _silu_mul_torch(ic0_bf16: np.ndarray, inter: int) -> np.ndarray:
    t = torch.from_numpy(C.bf16_to_f32(ic0_bf16).astype(np.float64))
    act = torch.nn.functional.silu(t[:, :inter]) * t[:, inter:]
    return _bf16(act.float().numpy())


def _fp8_experts(E, H, I, seed):
    g = torch.Generator().manual_seed(seed)
    w1 = (torch.randn(E, 2 * I, H, generator=g) * 100).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    w2 = (torch.randn(E, H, I, generator=g) * 100).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    s1 = (torch.rand(E, 2 * I // 128, H // 128, generator=g) * 4e-4 + 3e-4).numpy()
    s2 = (torch.rand(E, H // 128, I // 128, generator=g) * 4e-4 + 3e-4).numpy()
    return w1, s1, w2, s2


def _routing(M, E, topk, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(M)]).astype(np.int32)
    w = rng.random((M, topk)).astype(np.float32)
    return ids, w


H, I = 256, 128


@pytest.mark.parametrize("act_quant,with_bias", [(False, False), (True, False), (False, True), (True, True)])
def test_single_expert_equals_dense_chain(act_quant, with_bias):
    M = 21
    rng = np.random.default_rng(0)
    x = _bf16(rng.standard_normal((M, H)))
    w1, s1, w2, s2 = _fp8_experts(1, H, I, 1)
    b1 = rng.standard_normal((1, 2 * I)).astype(np.float32) if with_bias else None
    ids = np.zeros((M, 1), np.int32)
    wts = np.ones((M, 1), np.float32)
    got = MOE.fused_moe_fp8(x, ids, wts, w1, s1, w2, s2, b1, act_quant=act_quant)
    bias0 = None if b1 is None else b1[0]
    if act_quant:
        ic0 = D.block_fp8_linear_bf16(x, w1[0], s1[0], 128, bias0)
        ic1 = _silu_mul_torch(ic0, I)
        ref = D.block_fp8_linear_bf16(ic1, w2[0], s2[0], 128)
    else:
        ic0 = C.f32_to_bf16(D.w8a16_block_linear_f32(x, w1[0], s1[0], 128, bias0))
        ic1 = _silu_mul_torch(ic0, I)
        ref = C.f32_to_bf16(D.w8a16_block_linear_f32(ic1, w2[0], s2[0], 128))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("act_quant", [False, True])
def test_per_token_loop_equals_expert_sorted(act_quant):
    M, E, topk = 19, 6, 3
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal((M, H)))
    w1, s1, w2, s2 = _fp8_experts(E, H, I, 3)
    ids, wts = _routing(M, E, topk, 4)
    got = MOE.fused_moe_fp8(x, ids, wts, w1, s1, w2, s2, act_quant=act_quant)
    out = np.zeros((M, H), np.float64)
    for t in range(M):
        for k in range(topk):
            e = ids[t, k]
            if act_quant:
                q, s = per_token_group_quant_fp8(x[t:t + 1])
                ic0 = D.block_fp8_linear(q, s, w1[e], s1[e], 128)
                ic1 = _silu_mul_torch(ic0, I)
                q2, s2_ = per_token_group_quant_fp8(ic1)
                y = D.block_fp8_linear_f32(q2, s2_, w2[e], s2[e], 128)
            else:
                ic0 = C.f32_to_bf16(D.w8a16_block_linear_f32(x[t:t + 1], w1[e], s1[e], 128))
                ic1 = _silu_mul_torch(ic0, I)
                y = D.w8a16_block_linear_f32(ic1, w2[e], s2[e], 128)
            out[t] += np.float64(wts[t, k]) * y[0].astype(np.float64)
    assert np.array_equal(got, C.f32_to_bf16(out.astype(np.float32)))


def test_token_permutation_and_expert_relabelling():
    M, E, topk = 16, 5, 2
    rng = np.random.default_rng(5)
    x = _bf16(rng.standard_normal((M, H)))
    w1, s1, w2, s2 = _fp8_experts(E, H, I, 6)
    ids, wts = _routing(M, E, topk, 7)
    base = MOE.fused_moe_fp8(x, ids, wts, w1, s1, w2, s2)
    perm = rng.permutation(M)
    permuted = MOE.fused_moe_fp8(x[perm], ids[perm], wts[perm], w1, s1, w2, s2)
    assert np.array_equal(permuted, base[perm])
    lab = rng.permutation(E)  # expert e becomes lab[e]
    inv = np.argsort(lab)
    relab = MOE.fused_moe_fp8(x, lab[ids].astype(np.int32), wts, w1[inv], s1[inv], w2[inv], s2[inv])
    assert np.array_equal(relab, base)
    # swapping the order of a token's top-k entries changes nothing either
    sw = MOE.fused_moe_fp8(x, ids[:, ::-1].copy(), wts[:, ::-1].copy(), w1, s1, w2, s2)
    assert np.array_equal(sw, base)


def test_empty_experts_have_no_effect():
    M, E, topk = 12, 6, 2
    rng = np.random.default_rng(8)
    x = _bf16(rng.standard_normal((M, H)))
    w1, s1, w2, s2 = _fp8_experts(E, H, I, 9)
    ids = rng.choice([0, 2, 3], size=(M, 1)).astype(np.int32)
    ids = np.concatenate([ids, np.where(ids == 0, 3, 0).astype(np.int32)], axis=1)
    wts = rng.random((M, topk)).astype(np.float32)
    base = MOE.fused_moe_fp8(x, ids, wts, w1, s1, w2, s2)
    for e in (1, 4, 5):
        w1[e] = 0x7F
        w2[e] = 0xFF
        s1[e] = np.nan
    assert np.array_equal(MOE.fused_moe_fp8(x, ids, wts, w1, s1, w2, s2), base)


def test_identical_experts_reproduce_dense_mlp():
    M, E, topk = 10, 4, 3
    rng = np.random.default_rng(10)
    x = _bf16(rng.standard_normal((M, H)))
    w1, s1, w2, s2 = _fp8_experts(1, H, I, 11)
    W1, S1, W2, S2 = (np.repeat(a, E, axis=0) for a in (w1, s1, w2, s2))
    ids, _ = _routing(M, E, topk, 12)
    wts = np.full((M, topk), 1.0 / 4, np.float32)
    wts[:, 0] = 0.5  # 0.5 + 0.25 + 0.25 = 1, all exact
    got = MOE.fused_moe_fp8(x, ids, wts, W1, S1, W2, S2)
    ic0 = C.f32_to_bf16(D.w8a16_block_linear_f32(x, w1[0], s1[0], 128))
    ref = C.f32_to_bf16(D.w8a16_block_linear_f32(_silu_mul_torch(ic0, I), w2[0], s2[0], 128))
    assert np.array_equal(got, ref)


def test_mxfp4_equals_fp8_when_values_coincide():
    M, E, topk = 14, 4, 2
    Hm, Im = 128, 128
    rng = np.random.default_rng(13)
    x = _bf16(rng.standard_normal((M, Hm)))
    ids, wts = _routing(M, E, topk, 14)
    bias = rng.standard_normal((E, 2 * Im)).astype(np.float32)
    p1 = rng.integers(0, 256, size=(E, 2 * Im, Hm // 2)).astype(np.uint8)
    p2 = rng.integers(0, 256, size=(E, Hm, Im // 2)).astype(np.uint8)
    e1 = rng.integers(124, 131, size=(E, 2 * Im, Hm // 32)).astype(np.uint8)
    e2 = rng.integers(124, 131, size=(E, Hm, Im // 32)).astype(np.uint8)

    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

    def values(packed, sc):  # written out from the format: low nibble first
        lo, hi = packed & 0xF, packed >> 4
        v = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,))
        v[..., 0::2] = np.where(lo & 8, -1, 1) * mags[lo & 7]
        v[..., 1::2] = np.where(hi & 8, -1, 1) * mags[hi & 7]
        return v * np.repeat(2.0 ** (sc.astype(np.int64) - 127), 32, axis=-1)

    def to_e4m3(v):
        return torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    f1, f2 = to_e4m3(values(p1, e1)), to_e4m3(values(p2, e2))
    assert np.array_equal(C.E4M3_TABLE[f1], values(p1, e1))  # exactly representable
    g1 = np.ones((E, 2 * Im // 128, Hm // 128), np.float32)
    g2 = np.ones((E, Hm // 128, Im // 128), np.float32)
    got = MOE.fused_moe_mxfp4(x, ids, wts, p1, e1, p2, e2, bias)
    ref = MOE.fused_moe_fp8(x, ids, wts, f1, g1, f2, g2, bias, act_quant=False)
    assert np.array_equal(got, ref)
