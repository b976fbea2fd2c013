"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws numbers and prepares weights the way a checkpoint would hold
them; it holds none of the path's arithmetic (no activation quantiser, no
GEMM, no routing-to-blocks logic) and neither the HIP library nor the oracle
calls it.  The weight preparation below (block FP8 and MXFP4 weights from
Gaussian draws) is offline work of a model's weight conversion, not a step of
the path: the path receives its output, codes plus scales, as inputs.

Recipes (shapes and distributions follow the source pages' tests and the
DeepSeek- / GPT-OSS-shaped workloads the path is measured on):

* per-tensor W8A16 ("SGLang PR 32618 review", ``test_gemm.py`` listing):
  ``A = bf16(randn/10)``, ``W = e4m3(randn)``, scale 0.01, fp32 ``randn`` bias.
* block FP8 weights: ``w = 0.05 * randn`` quantised per 128x128 block (or per
  row per 128 columns for 1x128 blocks): ``scale_inv = amax / 448``,
  ``codes = e4m3(clamp(w / scale_inv, +-448))`` with torch's own e4m3 cast
  (round to nearest even), so every block's largest element lands on +-448.
* MXFP4 weights: ``w = 0.05 * randn`` quantised per row per 32 columns by the
  OCP MX rule: shared exponent ``floor(log2(amax)) - 2`` (2 = the largest
  e2m1 exponent), stored as e8m0 ``exponent + 127``; elements ``w / 2^exp``
  rounded to the nearest e2m1 value, ties to the even code, saturating at 6.
* the "page" FP8 recipe (``fp8_codes`` / ``fp8_block_scales``) of "SGLang PR
  35605 review" (``test_xpu_fp8_linear.py`` listing: codes cast from randn,
  scales ``rand + 0.1``) for its accuracy cases.
* activations ``bf16(randn)``; MXFP4 ``w1`` bias fp32 ``randn``.
* routing: deterministic per-expert counts over consecutive tokens (weight
  1.0); softmax-then-top-k of ``randn`` logits (weights not renormalised);
  Zipf(s) popularity over a seeded permutation of the experts, ``topk``
  distinct experts per token, weights = softmax of ``randn`` logits.

Generation runs on any torch device; big expert stacks are drawn one expert at
a time (seed + expert id) so host memory stays bounded.
"""

from __future__ import annotations

from typing import Dict, Optional, Sequence

import torch

FP8_CODE_STD = 100.0
WEIGHT_STD = 0.05


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def fp8_codes(shape, g: torch.Generator, device, std: float = FP8_CODE_STD) -> torch.Tensor:
    """uint8 e4m3 codes of ``clamp(std * randn, +-448)`` (torch's own cast)."""
    v = torch.randn(*shape, generator=g, device=device) * std
    return v.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def fp8_block_scales(shape, g: torch.Generator, device) -> torch.Tensor:
    u = torch.rand(*shape, generator=g, device=device)
    return ((0.8 + 0.4 * u) * (WEIGHT_STD / FP8_CODE_STD)).float()


def bf16_randn(shape, g, device, std: float = 1.0) -> torch.Tensor:
    return (torch.randn(*shape, generator=g, device=device) * std).to(torch.bfloat16)


def fp8_block_quantize(w: torch.Tensor, block_n: int = 128, block_k: int = 128):
    """fp32 [N, K] -> (uint8 e4m3 codes [N, K], fp32 scale_inv [ceil(N/block_n), K/block_k]).

    Per block: ``scale_inv = amax / 448``; ``codes = e4m3(clamp(w / scale_inv, +-448))``
    (torch's cast, round to nearest even).  A zero block gets scale 1 and zero codes."""
    N, K = w.shape
    nb = -(-N // block_n)
    wp = torch.zeros(nb * block_n, K, dtype=torch.float32, device=w.device)
    wp[:N] = w
    blocks = wp.view(nb, block_n, K // block_k, block_k)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).float()
    q = (blocks / scale[:, None, :, None]).clamp_(-448.0, 448.0)
    codes = q.reshape(nb * block_n, K)[:N].to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


# e2m1 magnitudes by code (bits 0-2) and the midpoints between neighbours
_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def mxfp4_quantize(w: torch.Tensor):
    """fp32 [N, K] (K % 32 == 0) -> (packed e2m1 uint8 [N, K/2], e8m0 uint8 [N, K/32]) by the OCP
    MX rule: shared exponent floor(log2(amax)) - 2 per 32 elements (an all-zero group takes the
    smallest exponent, -127), elements rounded to the nearest e2m1 value with ties to the even
    code and saturated at 6; element 2j in the low nibble of byte j."""
    N, K = w.shape
    g = w.reshape(N, K // 32, 32).float()
    amax = g.abs().amax(dim=2)
    _, ex = torch.frexp(amax)  # amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
    shared = torch.where(amax > 0, ex - 1 - 2, torch.full_like(ex, -127)).clamp_(-127, 127)
    v = g / torch.ldexp(torch.ones_like(amax), shared)[:, :, None]
    mag = v.abs()
    mids = torch.tensor(_E2M1_MIDS, dtype=torch.float32, device=w.device)
    below = (mag[..., None] > mids).sum(dim=-1)  # code when no tie
    tie = (mag[..., None] == mids).any(dim=-1)
    code = below + (tie & (below % 2 == 1)).to(below.dtype)  # a tie goes to the even code
    code = code | (v < 0).to(code.dtype) * 8
    code = code.to(torch.uint8).reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    scales = (shared + 127).to(torch.uint8).contiguous()
    return packed, scales


# --------------------------------------------------------------------------- dense

def dense_w8a16(M: int, N: int, K: int, seed: int, device="cpu", has_bias=True,
                scale: float = 0.01) -> Dict[str, torch.Tensor]:
    g = _gen(seed, device)
    a = (torch.randn(M, K, generator=g, device=device) / 10).to(torch.bfloat16)
    w = torch.randn(N, K, generator=g, device=device).to(torch.float8_e4m3fn).view(torch.uint8)
    bias = torch.randn(N, generator=g, device=device) if has_bias else None
    return {"a": a, "w": w, "scale": torch.tensor([scale], dtype=torch.float32, device=device),
            "bias": bias}


def batched_w8a16(B: int, M: int, N: int, K: int, seed: int, device="cpu", has_bias=True,
                  per_entry_scale=True) -> Dict[str, torch.Tensor]:
    """Batched per-tensor W8A16 operands (per-head products of an MLA-style layer): the
    per-tensor recipe above for each of B entries; scales rand + 0.005 per entry (or one)."""
    g = _gen(seed, device)
    a = (torch.randn(B, M, K, generator=g, device=device) / 10).to(torch.bfloat16)
    w = torch.randn(B, N, K, generator=g, device=device).to(torch.float8_e4m3fn).view(torch.uint8)
    scale = torch.rand(B if per_entry_scale else 1, generator=g, device=device) * 0.02 + 0.005
    bias = torch.randn(B, N, generator=g, device=device) if has_bias else None
    return {"a": a, "w": w, "scale": scale, "bias": bias}


def block_linear(M: int, N: int, K: int, seed: int, device="cpu", block_n: int = 128,
                 bias_dtype: Optional[torch.dtype] = None) -> Dict[str, torch.Tensor]:
    """bf16 ``randn`` activations and ``0.05 * randn`` weights quantised per block_n x 128."""
    g = _gen(seed, device)
    x = bf16_randn((M, K), g, device)
    w, sw = fp8_block_quantize(torch.randn(N, K, generator=g, device=device) * WEIGHT_STD, block_n)
    bias = None
    if bias_dtype is not None:
        bias = torch.randn(N, generator=g, device=device).to(bias_dtype)
    return {"x": x, "w": w, "sw": sw, "bias": bias, "block_n": block_n}


def mx_linear(M: int, N: int, K: int, seed: int, device="cpu", w_format: str = "e2m1",
              bias_dtype: Optional[torch.dtype] = None) -> Dict[str, torch.Tensor]:
    """bf16 ``randn`` activations and MX weights: MXFP4 (``"e2m1"``) from ``0.05 * randn`` by the
    OCP rule, or MXFP8 (``"e4m3"``) drawn as codes ``e4m3(clamp(100 * randn, +-448))`` with e8m0
    scale codes uniform in [110, 114] (2^-17 .. 2^-13, decoded weights ~0.05 * randn)."""
    g = _gen(seed, device)
    x = bf16_randn((M, K), g, device)
    if w_format == "e2m1":
        w, sw = mxfp4_quantize(torch.randn(N, K, generator=g, device=device) * WEIGHT_STD)
    else:
        w = fp8_codes((N, K), g, device)
        sw = torch.randint(110, 115, (N, K // 32), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    bias = None
    if bias_dtype is not None:
        bias = torch.randn(N, generator=g, device=device).to(bias_dtype)
    return {"x": x, "w": w, "sw": sw, "bias": bias, "w_format": w_format}


# --------------------------------------------------------------------------- routing

def route_counts(counts: Sequence[int], device="cpu"):
    """topk=1: expert e gets ``counts[e]`` consecutive tokens, weight 1.0."""
    ids = torch.cat([torch.full((c,), e, dtype=torch.int32) for e, c in enumerate(counts)])
    w = torch.ones(ids.numel(), 1, dtype=torch.float32)
    return ids.view(-1, 1).to(device), w.to(device)


def route_softmax_topk(M: int, E: int, topk: int, seed: int, device="cpu"):
    g = _gen(seed, "cpu")
    logits = torch.randn(M, E, generator=g)
    probs = torch.softmax(logits.float(), dim=-1)
    w, ids = torch.topk(probs, topk, dim=-1)
    return ids.to(torch.int32).to(device), w.float().to(device)


def route_zipf(M: int, E: int, topk: int, s: float, seed: int, device="cpu"):
    g = _gen(seed, "cpu")
    perm = torch.randperm(E, generator=g)
    pop = torch.empty(E, dtype=torch.float64)
    pop[perm] = torch.arange(1, E + 1, dtype=torch.float64) ** (-s)
    ids = torch.multinomial(pop.expand(M, E), topk, replacement=False, generator=g)
    w = torch.softmax(torch.randn(M, topk, generator=g), dim=-1)
    return ids.to(torch.int32).to(device), w.float().to(device)


# --------------------------------------------------------------------------- experts

def moe_fp8_weights(E: int, H: int, I: int, seed: int, device="cpu"):
    """w1 [E, 2I, H], w2 [E, H, I]: ``0.05 * randn`` quantised per 128x128 block."""
    w1 = torch.empty(E, 2 * I, H, dtype=torch.uint8, device=device)
    w2 = torch.empty(E, H, I, dtype=torch.uint8, device=device)
    s1 = torch.empty(E, -(-2 * I // 128), H // 128, dtype=torch.float32, device=device)
    s2 = torch.empty(E, -(-H // 128), I // 128, dtype=torch.float32, device=device)
    for e in range(E):
        g = _gen(seed + 7919 * (e + 1), device)
        w1[e], s1[e] = fp8_block_quantize(torch.randn(2 * I, H, generator=g, device=device) * WEIGHT_STD)
        w2[e], s2[e] = fp8_block_quantize(torch.randn(H, I, generator=g, device=device) * WEIGHT_STD)
    return {"w1": w1, "w1_scale": s1, "w2": w2, "w2_scale": s2}


def moe_mxfp4_weights(E: int, H: int, I: int, seed: int, device="cpu", with_bias=True):
    """w1 [E, 2I, H/2], w2 [E, H, I/2] packed e2m1 with e8m0 scales per 32 columns: ``0.05 * randn``
    quantised by the OCP MX rule."""
    w1 = torch.empty(E, 2 * I, H // 2, dtype=torch.uint8, device=device)
    w2 = torch.empty(E, H, I // 2, dtype=torch.uint8, device=device)
    s1 = torch.empty(E, 2 * I, H // 32, dtype=torch.uint8, device=device)
    s2 = torch.empty(E, H, I // 32, dtype=torch.uint8, device=device)
    b1 = torch.empty(E, 2 * I, dtype=torch.float32, device=device) if with_bias else None
    for e in range(E):
        g = _gen(seed + 7919 * (e + 1), device)
        w1[e], s1[e] = mxfp4_quantize(torch.randn(2 * I, H, generator=g, device=device) * WEIGHT_STD)
        w2[e], s2[e] = mxfp4_quantize(torch.randn(H, I, generator=g, device=device) * WEIGHT_STD)
        if b1 is not None:
            b1[e] = torch.randn(2 * I, generator=g, device=device)
    return {"w1": w1, "w1_scale": s1, "w2": w2, "w2_scale": s2, "w1_bias": b1}


# --------------------------------------------------------------------------- workloads

WORKLOADS = {
    "per_tensor_w8a16_97x576x224": dict(kind="fp8_scaled_mm", M=97, K=576, N=224),
    "block_w8a8_linear_2048x2048x7168": dict(kind="block_fp8_linear", M=2048, K=2048, N=7168),
    "moe_block_fp8_w8a16_e8_h2048_i1024": dict(
        kind="fused_moe_fp8", E=8, topk=1, H=2048, I=1024,
        counts=(4, 5, 33, 0, 0, 12, 1, 73), act_quant=False),
    "moe_mxfp4_gptoss_decode_m32": dict(
        kind="fused_moe_mxfp4", M=32, E=128, topk=4, H=2880, I=2880),
    "moe_block_fp8_w8a8_deepseek_prefill_m4096": dict(
        kind="fused_moe_fp8", M=4096, E=256, topk=8, H=7168, I=2048, zipf=1.1, act_quant=True),
}


def moe_inputs(name_or_spec, seed: int, device="cpu", M: Optional[int] = None) -> Dict:
    """All inputs of one routed-MoE workload (``M`` overrides the token count)."""
    spec = dict(WORKLOADS[name_or_spec]) if isinstance(name_or_spec, str) else dict(name_or_spec)
    E, topk, H, I = spec["E"], spec["topk"], spec["H"], spec["I"]
    if "counts" in spec:
        ids, w = route_counts(spec["counts"], device)
        M = ids.shape[0]
    else:
        M = spec["M"] if M is None else M
        if "zipf" in spec:
            ids, w = route_zipf(M, E, topk, spec["zipf"], seed + 1, device)
        else:
            ids, w = route_softmax_topk(M, E, topk, seed + 1, device)
    g = _gen(seed, device)
    x = bf16_randn((M, H), g, device)
    if spec["kind"] == "fused_moe_mxfp4":
        wts = moe_mxfp4_weights(E, H, I, seed + 2, device)
    else:
        wts = moe_fp8_weights(E, H, I, seed + 2, device)
        wts["w1_bias"] = None
    out = {"x": x, "topk_ids": ids, "topk_weights": w, "E": E, "topk": topk, "H": H, "I": I,
           "act_quant": bool(spec.get("act_quant", False)), "kind": spec["kind"]}
    out.update(wts)
    return out


def moe_flops(M: int, topk: int, H: int, I: int) -> float:
    R = M * topk
    return 2.0 * R * (2 * I * H + H * I)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)

