"""Thin torch binding of libmxq: argument marshalling only.

Each function validates dtypes and shapes, flattens leading dimensions, takes
``data_ptr()``s and the current HIP stream, allocates outputs and workspaces
with torch's caching allocator, and calls the C entry point of the same name
(``mxq_<name>``).  Every step of the computation runs in the HIP kernels.

Semantics carried over from the source pages:

* N-D inputs are flattened to 2-D and the result is viewed back ("SGLang PR
  32618 review", fp8.py listing; "SGLang PR 35605 review", fp8_utils.py
  listing).
* An input whose last dimension is not unit-stride is copied; other strides
  are passed through (fp8_utils.py listing).
* ``block_size`` must be ``[1, 128]`` or ``[128, 128]``, anything else raises
  ``ValueError`` (fp8_utils.py listing).
* The per-tensor scale may be a 0-d or a 1-element tensor ("SGLang PR 32618
  review", test_gemm.py listing).
"""

from __future__ import annotations

from typing import Dict, NamedTuple, Optional, Sequence, Tuple

import ctypes

import torch

from . import _lib as L

C_i64 = ctypes.c_int64

_E4M3 = torch.float8_e4m3fn


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _as_u8(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == _E4M3:
        return t.view(torch.uint8)
    if t.dtype == torch.uint8:
        return t
    raise ValueError(f"{name} must be float8_e4m3fn or uint8 codes, got {t.dtype}")


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _unit_last(t: torch.Tensor) -> torch.Tensor:
    if t.stride(-1) != 1 or (t.data_ptr() % 16) != 0 or (t.dim() >= 2 and (t.stride(-2) * t.element_size()) % 16 != 0):
        t = t.contiguous()
    return t


def _2d(t: torch.Tensor) -> torch.Tensor:
    t2 = t.reshape(-1, t.shape[-1])
    return _unit_last(t2)


def _bias_dtype(b: Optional[torch.Tensor]) -> int:
    if b is None:
        return L.MXQ_DTYPE_F32
    if b.dtype == torch.float32:
        return L.MXQ_DTYPE_F32
    if b.dtype == torch.bfloat16:
        return L.MXQ_DTYPE_BF16
    raise ValueError(f"bias must be fp32 or bf16, got {b.dtype}")


def init(device: int = 0) -> None:
    L.check("mxq_init", L.load().mxq_init(device))


def per_token_group_quant_fp8(x: torch.Tensor, group: int = 128) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 [..., K] -> (e4m3 codes [..., K] as float8_e4m3fn, fp32 scales [..., K/group])."""
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    _require_cuda(x)
    shape = x.shape
    x2 = x.reshape(-1, shape[-1])
    if x2.stride(-1) != 1 or x2.data_ptr() % 16 or x2.stride(0) % 8:
        x2 = x2.contiguous()
    M, K = x2.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, K // group if group else 0), dtype=torch.float32, device=x.device)
    st = L.load().mxq_per_token_group_quant_fp8(x2.data_ptr(), M, K, x2.stride(0), group, q.data_ptr(),
                                                s.data_ptr(), _stream())
    L.check("mxq_per_token_group_quant_fp8", st)
    return q.view(_E4M3).view(*shape), s.view(*shape[:-1], s.shape[-1])


def fp8_scaled_mm(x: torch.Tensor, weight: torch.Tensor, scale: torch.Tensor,
                  bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-tensor W8A16: bf16 [..., K] @ e4m3 [N, K]^T * scale (+ bias) -> bf16 [..., N]."""
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    w = _as_u8(weight, "weight").contiguous()
    if scale.numel() != 1 or scale.dtype != torch.float32:
        raise ValueError("scale must be a single fp32 value (0-d or [1])")
    _require_cuda(x, w, scale, bias)
    x2 = _2d(x)
    M, K = x2.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"weight K {w.shape[1]} != input K {K}")
    if bias is not None and bias.numel() != N:
        raise ValueError("bias must have N elements")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    sc = scale.reshape(1).contiguous()
    b = None if bias is None else bias.contiguous()
    lib = L.load()
    ws_bytes = lib.mxq_fp8_scaled_mm_workspace_size(M, N, K)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    st = lib.mxq_fp8_scaled_mm(x2.data_ptr(), M, K, x2.stride(0), w.data_ptr(), N, sc.data_ptr(), _ptr(b),
                               _bias_dtype(b), out.data_ptr(), N, ws.data_ptr(), ws_bytes, _stream())
    L.check("mxq_fp8_scaled_mm", st)
    return out.view(*x.shape[:-1], N)


def fp8_scaled_bmm(x: torch.Tensor, weight: torch.Tensor, scale: torch.Tensor,
                   bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Batched per-tensor W8A16: bf16 [B, M, K] @ e4m3 [B, N, K]^T * scale[b] (+ bias[b]) -> bf16 [B, M, N].

    ``scale`` holds one fp32 value (shared) or B values; ``bias`` is None, [N] (shared) or
    [B, N].  Each entry equals ``fp8_scaled_mm`` on that entry, bit for bit.
    """
    if x.dtype != torch.bfloat16 or x.dim() != 3:
        raise ValueError("x must be bf16 [B, M, K]")
    w = _as_u8(weight, "weight")
    if w.dim() != 3:
        raise ValueError("weight must be [B, N, K]")
    B, M, K = x.shape
    N = w.shape[1]
    if w.shape[0] != B or w.shape[2] != K:
        raise ValueError(f"weight shape {tuple(w.shape)} does not match input {tuple(x.shape)}")
    if scale.dtype != torch.float32 or scale.numel() not in (1, B):
        raise ValueError("scale must hold 1 or B fp32 values")
    if bias is not None and (bias.shape[-1] != N or bias.numel() not in (N, B * N)):
        raise ValueError("bias must be [N] or [B, N]")
    w = w.contiguous()
    _require_cuda(x, w, scale, bias)
    if x.stride(-1) != 1 or x.stride(1) % 8 != 0 or x.stride(0) % 8 != 0:
        x = x.contiguous()
    sc = scale.reshape(-1).contiguous()
    b = None
    b_stride = 0
    if bias is not None:
        b = bias.reshape(-1, N).contiguous()
        b_stride = N if b.shape[0] == B and B > 1 else 0
    out = torch.empty((B, M, N), dtype=torch.bfloat16, device=x.device)
    st = L.load().mxq_fp8_scaled_bmm(x.data_ptr(), B, M, K, x.stride(1), x.stride(0), w.data_ptr(), N, N * K,
                                     sc.data_ptr(), 1 if sc.numel() == B and B > 1 else 0, _ptr(b), _bias_dtype(b),
                                     b_stride, out.data_ptr(), N, M * N, _stream())
    L.check("mxq_fp8_scaled_bmm", st)
    return out


def block_fp8_linear(x: torch.Tensor, weight: torch.Tensor, block_size: Sequence[int], weight_scale: torch.Tensor,
                     input_scale: Optional[torch.Tensor] = None,
                     bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block-wise FP8 W8A8 linear -> bf16 [..., N].

    ``x`` is bf16 (quantised per token per 128 columns inside the call) or e4m3
    codes with ``input_scale`` [..., K/128].  ``weight_scale`` has logical shape
    [ceil(N / block_n), K / 128] and may have any strides (the transposed
    storage of a load-time relayout included).
    """
    if not isinstance(block_size, (list, tuple)) or len(block_size) != 2:
        raise ValueError(f"block_size must have two entries, got {block_size}")
    block_n, block_k = int(block_size[0]), int(block_size[1])
    if block_k != 128 or block_n not in (1, 128):
        raise ValueError(f"block_size must be [1, 128] or [128, 128], got {list(block_size)}")
    w = _as_u8(weight, "weight")
    if w.stride(-1) != 1:
        w = w.contiguous()
    w = w.contiguous()
    _require_cuda(x, w, weight_scale, input_scale, bias)
    if weight_scale.dtype != torch.float32 or weight_scale.dim() != 2:
        raise ValueError("weight_scale must be a 2-D fp32 tensor")
    N, K = w.shape
    if input_scale is None:
        if x.dtype != torch.bfloat16:
            raise ValueError("x must be bf16 when input_scale is None")
        a = _2d(x)
        a_dtype = L.MXQ_DTYPE_BF16
        a_scale = None
    else:
        a = _2d(_as_u8(x, "x"))
        a_dtype = L.MXQ_DTYPE_E4M3
        a_scale = input_scale.reshape(-1, input_scale.shape[-1]).contiguous()
        if a_scale.dtype != torch.float32:
            raise ValueError("input_scale must be fp32")
    M = a.shape[0]
    if a.shape[1] != K:
        raise ValueError(f"weight K {K} != input K {a.shape[1]}")
    if tuple(weight_scale.shape) != (-(-N // block_n), K // 128):
        raise ValueError(f"weight_scale shape {tuple(weight_scale.shape)} != {(-(-N // block_n), K // 128)}")
    if a_scale is not None and tuple(a_scale.shape) != (M, K // 128):
        raise ValueError("input_scale must be [..., K/128]")
    b = None if bias is None else bias.contiguous()
    if b is not None and b.numel() != N:
        raise ValueError("bias must have N elements")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    lib = L.load()
    ws_bytes = lib.mxq_block_fp8_linear_workspace_size(M, N, K, a_dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    st = lib.mxq_block_fp8_linear(a.data_ptr(), a_dtype, _ptr(a_scale), M, K, a.stride(0), w.data_ptr(), N,
                                  weight_scale.data_ptr(), weight_scale.stride(0), weight_scale.stride(1), block_n,
                                  block_k, _ptr(b), _bias_dtype(b), out.data_ptr(), L.MXQ_DTYPE_BF16, N,
                                  ws.data_ptr(), ws_bytes, _stream())
    L.check("mxq_block_fp8_linear", st)
    return out.view(*x.shape[:-1], N)


def mxfp8_quant(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 [..., K] -> (e4m3 codes [..., K] as float8_e4m3fn, e8m0 scale codes uint8 [..., K/32])."""
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    _require_cuda(x)
    shape = x.shape
    x2 = x.reshape(-1, shape[-1])
    if x2.stride(-1) != 1 or x2.data_ptr() % 16 or x2.stride(0) % 8:
        x2 = x2.contiguous()
    M, K = x2.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    L.check("mxq_mxfp8_quant", L.load().mxq_mxfp8_quant(x2.data_ptr(), M, K, x2.stride(0), q.data_ptr(),
                                                         s.data_ptr(), _stream()))
    return q.view(_E4M3).view(*shape), s.view(*shape[:-1], s.shape[-1])


_MX_W = {"e4m3": L.MXQ_DTYPE_E4M3, "e2m1": L.MXQ_DTYPE_E2M1}


def mx_linear(x: torch.Tensor, weight: torch.Tensor, weight_scale: torch.Tensor, w_format: str = "e2m1",
              input_scale: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MX-scaled linear -> bf16 [..., N].

    ``x``: bf16 [..., K] (MXFP8-quantised per token per 32 columns inside the call), or e4m3
    codes with ``input_scale`` e8m0 uint8 [..., K/32].  ``weight``: e4m3 [N, K]
    (``w_format="e4m3"``, MXFP8) or packed e2m1 uint8 [N, K/2] (``"e2m1"``, MXFP4) with
    ``weight_scale`` e8m0 uint8 [N, K/32]."""
    if w_format not in _MX_W:
        raise ValueError(f"w_format must be 'e4m3' or 'e2m1', got {w_format!r}")
    w = _as_u8(weight, "weight").contiguous()
    sw = weight_scale.contiguous()
    if sw.dtype != torch.uint8:
        raise ValueError("weight_scale must be uint8 e8m0 codes")
    _require_cuda(x, w, sw, input_scale, bias)
    N = w.shape[0]
    K = w.shape[1] * (2 if w_format == "e2m1" else 1)
    if input_scale is None:
        if x.dtype != torch.bfloat16:
            raise ValueError("x must be bf16 when input_scale is None")
        a, a_dtype, a_scale = _2d(x), L.MXQ_DTYPE_BF16, None
    else:
        a, a_dtype = _2d(_as_u8(x, "x")), L.MXQ_DTYPE_E4M3
        a_scale = input_scale.reshape(-1, input_scale.shape[-1]).contiguous()
        if a_scale.dtype != torch.uint8:
            raise ValueError("input_scale must be uint8 e8m0 codes")
    M = a.shape[0]
    if a.shape[1] != K:
        raise ValueError(f"weight K {K} != input K {a.shape[1]}")
    if tuple(sw.shape) != (N, K // 32):
        raise ValueError(f"weight_scale must be [{N}, {K // 32}]")
    if a_scale is not None and tuple(a_scale.shape) != (M, K // 32):
        raise ValueError("input_scale must be [..., K/32]")
    b = None if bias is None else bias.contiguous()
    if b is not None and b.numel() != N:
        raise ValueError("bias must have N elements")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    lib = L.load()
    ws_bytes = lib.mxq_mx_linear_workspace_size(M, N, K, a_dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    st = lib.mxq_mx_linear(a.data_ptr(), a_dtype, _ptr(a_scale), M, K, a.stride(0), w.data_ptr(), _MX_W[w_format], N,
                           sw.data_ptr(), _ptr(b), _bias_dtype(b), out.data_ptr(), N, ws.data_ptr(), ws_bytes,
                           _stream())
    L.check("mxq_mx_linear", st)
    return out.view(*x.shape[:-1], N)


def moe_max_blocks(M: int, topk: int, E: int, block_m: int) -> int:
    return int(L.load().mxq_moe_max_blocks(M, topk, E, block_m))


def moe_align(topk_ids: torch.Tensor, E: int, block_m: int):
    """int32 [M, topk] -> (sorted_ids, expert_ids, offsets, num_blocks) device tensors."""
    if topk_ids.dtype != torch.int32 or topk_ids.dim() != 2:
        raise ValueError("topk_ids must be int32 [M, topk]")
    _require_cuda(topk_ids)
    ids = topk_ids.contiguous()
    M, topk = ids.shape
    nb = moe_max_blocks(M, topk, E, block_m)
    dev = ids.device
    sorted_ids = torch.empty(max(nb * block_m, 1), dtype=torch.int32, device=dev)
    expert_ids = torch.empty(max(nb, 1), dtype=torch.int32, device=dev)
    offsets = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    num_blocks = torch.empty(1, dtype=torch.int32, device=dev)
    st = L.load().mxq_moe_align(ids.data_ptr(), M, topk, E, block_m, sorted_ids.data_ptr(), expert_ids.data_ptr(),
                                offsets.data_ptr(), num_blocks.data_ptr(), _stream())
    L.check("mxq_moe_align", st)
    return sorted_ids[:nb * block_m], expert_ids[:nb], offsets, num_blocks


def _moe_common(x, topk_ids, topk_weights):
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be bf16 [M, H]")
    if topk_ids.dtype != torch.int32 or topk_weights.dtype != torch.float32:
        raise ValueError("topk_ids must be int32 and topk_weights fp32")
    if topk_ids.shape != topk_weights.shape or topk_ids.shape[0] != x.shape[0]:
        raise ValueError("topk_ids / topk_weights must be [M, topk]")
    return x.contiguous(), topk_ids.contiguous(), topk_weights.contiguous()


def fused_moe_workspace(M: int, H: int, I: int, E: int, topk: int, weights: int, act_quant: bool,
                        device) -> torch.Tensor:
    n = L.load().mxq_fused_moe_workspace_size(M, H, I, E, topk, weights, int(act_quant))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def fused_moe_workspace_layout(M: int, H: int, I: int, E: int, topk: int, weights: int,
                               act_quant: bool) -> Dict[str, int]:
    """Byte offsets of the fused MoE's intermediates in its workspace (-1: region unused),
    plus ``block_m`` (``mxq_fused_moe_workspace_layout``)."""
    arr = (C_i64 * len(L.MOE_WS_FIELDS))()
    L.check("mxq_fused_moe_workspace_layout",
            L.load().mxq_fused_moe_workspace_layout(M, H, I, E, topk, weights, int(act_quant), arr))
    return {k: int(arr[i]) for i, k in enumerate(L.MOE_WS_FIELDS)}


def fused_moe_plan(M: int, H: int, I: int, E: int, topk: int, weights: int, act_quant: bool = False,
                   weight_layout: str = "plain", dispatch: Optional["Dispatch"] = None) -> Dict[str, object]:
    """The kernel plan a fused-MoE call of these sizes would run (``mxq_fused_moe_plan``; host
    only): path, tile family, the block classes that can occur (set of class ids), rows per
    block and K chunks per stage, and where the SiLU-and-mul and the combine run."""
    arr = (ctypes.c_int32 * len(L.MOE_PLAN_FIELDS))()
    L.check("mxq_fused_moe_plan",
            L.load().mxq_fused_moe_plan(M, H, I, E, topk, weights, int(act_quant), _layout(weight_layout),
                                        _dispatch(dispatch), arr))
    out: Dict[str, object] = {}
    for i, k in enumerate(L.MOE_PLAN_FIELDS):
        v = int(arr[i])
        if k == "classes":
            out[k] = {c for c in range(5) if v >> c & 1}
        elif k in L.MOE_PLAN_NAMES:
            out[k] = L.MOE_PLAN_NAMES[k][v]
        else:
            out[k] = v
    return out


class Dispatch(NamedTuple):
    """Per-call dispatch of the fused MoE (``struct mxq_moe_dispatch``); None = the defaults."""
    mode: int = L.MXQ_DISPATCH_PER_BLOCK
    forced_class: int = 0
    tiny_max_rows: int = L.MXQ_TINY_ROWS_AUTO
    tiny_kernel: int = L.MXQ_TINY_MFMA
    k_split: int = L.MXQ_K_SPLIT_AUTO
    sort: int = L.MXQ_SORT_AUTO
    fuse: int = L.MXQ_FUSE_AUTO


def _dispatch(d: Optional[Dispatch]):
    if d is None:
        return None
    return ctypes.byref(L.MoeDispatch(int(d.mode), int(d.forced_class), int(d.tiny_max_rows), int(d.tiny_kernel),
                                      int(d.k_split), int(d.sort),
                                      int(d.fuse)))


def silu_and_mul(ic0: torch.Tensor, quant: bool = False):
    """bf16 [rows, 2I] (gate | up) -> bf16 [rows, I] = silu(gate) * up, or with ``quant`` the
    e4m3 codes [rows, I] and fp32 scales [rows, I/128] of that product (1x128 groups)."""
    if ic0.dtype != torch.bfloat16 or ic0.dim() != 2 or ic0.shape[1] % 2:
        raise ValueError("ic0 must be bf16 [rows, 2I]")
    _require_cuda(ic0)
    if ic0.stride(-1) != 1 or ic0.data_ptr() % 16 or ic0.stride(0) % 8:
        ic0 = ic0.contiguous()
    rows, two_i = ic0.shape
    I = two_i // 2
    lib = L.load()
    if quant:
        q = torch.empty((rows, I), dtype=torch.uint8, device=ic0.device)
        s = torch.empty((rows, I // 128), dtype=torch.float32, device=ic0.device)
        st = lib.mxq_silu_and_mul(ic0.data_ptr(), rows, I, ic0.stride(0), None, q.data_ptr(), s.data_ptr(),
                                  _stream())
        L.check("mxq_silu_and_mul", st)
        return q.view(_E4M3), s
    out = torch.empty((rows, I), dtype=torch.bfloat16, device=ic0.device)
    st = lib.mxq_silu_and_mul(ic0.data_ptr(), rows, I, ic0.stride(0), out.data_ptr(), None, None, _stream())
    L.check("mxq_silu_and_mul", st)
    return out


_LAYOUTS = {"plain": L.MXQ_LAYOUT_PLAIN, "tiled": L.MXQ_LAYOUT_TILED}


def _layout(weight_layout: str) -> int:
    if weight_layout not in _LAYOUTS:
        raise ValueError(f"weight_layout must be 'plain' or 'tiled', got {weight_layout!r}")
    return _LAYOUTS[weight_layout]


def _tiled_row(row_bytes: int) -> int:
    return -(-row_bytes // 128) * 128


def moe_prepack(w: torch.Tensor) -> torch.Tensor:
    """Routed-expert weights [E, N, row_bytes] (e4m3 or packed e2m1 codes) -> the tiled layout
    of ``mxq_moe_prepack``, returned as uint8 [E, N, ceil(row_bytes / 128) * 128]."""
    w = _as_u8(w, "w").contiguous()
    if w.dim() != 3:
        raise ValueError("w must be [E, N, row_bytes]")
    _require_cuda(w)
    E, N, rb = w.shape
    lib = L.load()
    n = lib.mxq_moe_prepack_size(E, N, rb)
    if n == 0:
        raise ValueError(f"N ({N}) and row_bytes ({rb}) must be positive multiples of 16")
    out = torch.empty((E, N, _tiled_row(rb)), dtype=torch.uint8, device=w.device)
    assert out.numel() == n
    L.check("mxq_moe_prepack", lib.mxq_moe_prepack(w.data_ptr(), E, N, rb, out.data_ptr(), _stream()))
    return out


def moe_prepack_scales(s: torch.Tensor) -> torch.Tensor:
    """e8m0 MX scales [E, N, groups] -> the tiled layout of ``mxq_moe_prepack_scales``, returned as
    uint8 [E, N, ceil(groups / 8) * 8]."""
    if s.dtype != torch.uint8 or s.dim() != 3:
        raise ValueError("scales must be uint8 [E, N, groups]")
    _require_cuda(s)
    s = s.contiguous()
    E, N, G = s.shape
    lib = L.load()
    n = lib.mxq_moe_prepack_scales_size(E, N, G)
    if n == 0:
        raise ValueError(f"N ({N}) must be a positive multiple of 16")
    out = torch.empty((E, N, -(-G // 8) * 8), dtype=torch.uint8, device=s.device)
    assert out.numel() == n
    L.check("mxq_moe_prepack_scales", lib.mxq_moe_prepack_scales(s.data_ptr(), E, N, G, out.data_ptr(), _stream()))
    return out


def fused_moe_fp8(x, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale, w1_bias=None, act_quant=False,
                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  weight_layout: str = "plain", dispatch: Optional[Dispatch] = None) -> torch.Tensor:
    """Routed MoE with block-FP8 experts (W8A16, or W8A8 with ``act_quant``) -> bf16 [M, H].

    ``weight_layout="tiled"``: ``w1`` / ``w2`` come from :func:`moe_prepack`."""
    layout = _layout(weight_layout)
    x, ids, wts = _moe_common(x, topk_ids, topk_weights)
    w1 = _as_u8(w1, "w1").contiguous()
    w2 = _as_u8(w2, "w2").contiguous()
    _require_cuda(x, ids, wts, w1, w2, w1_scale, w2_scale, w1_bias)
    M, H = x.shape
    E, two_i, h1 = w1.shape
    I = two_i // 2
    topk = ids.shape[1]
    rb1, rb2 = (H, I) if layout == L.MXQ_LAYOUT_PLAIN else (_tiled_row(H), _tiled_row(I))
    if h1 != rb1 or tuple(w2.shape) != (E, H, rb2):
        raise ValueError(f"w1 must be [E, 2I, {rb1}] and w2 [E, H, {rb2}] for the {weight_layout} layout")
    if tuple(w1_scale.shape) != (E, -(-2 * I // 128), H // 128) or tuple(w2_scale.shape) != (E, -(-H // 128), I // 128):
        raise ValueError("block scales must be [E, ceil(2I/128), H/128] and [E, ceil(H/128), I/128]")
    s1 = w1_scale.float().contiguous()
    s2 = w2_scale.float().contiguous()
    b1 = None if w1_bias is None else w1_bias.float().contiguous()
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = fused_moe_workspace(M, H, I, E, topk, L.MXQ_WEIGHTS_FP8_BLOCK, act_quant, x.device)
    st = L.load().mxq_fused_moe_fp8(x.data_ptr(), M, H, I, E, topk, ids.data_ptr(), wts.data_ptr(), w1.data_ptr(),
                                    s1.data_ptr(), w2.data_ptr(), s2.data_ptr(), _ptr(b1), int(bool(act_quant)),
                                    layout, _dispatch(dispatch), out.data_ptr(), workspace.data_ptr(),
                                    workspace.numel(), _stream())
    L.check("mxq_fused_moe_fp8", st)
    return out


def fused_moe_mxfp4(x, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale, w1_bias=None,
                    workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    weight_layout: str = "plain", dispatch: Optional[Dispatch] = None) -> torch.Tensor:
    """Routed MoE with MXFP4 experts (packed e2m1 + e8m0 per 32), bf16 activations -> bf16 [M, H].

    ``weight_layout="tiled"``: weights from :func:`moe_prepack`, scales from :func:`moe_prepack_scales`."""
    layout = _layout(weight_layout)
    x, ids, wts = _moe_common(x, topk_ids, topk_weights)
    w1 = w1.contiguous()
    w2 = w2.contiguous()
    s1 = w1_scale.contiguous()
    s2 = w2_scale.contiguous()
    for t, n in ((w1, "w1"), (w2, "w2"), (s1, "w1_scale"), (s2, "w2_scale")):
        if t.dtype != torch.uint8:
            raise ValueError(f"{n} must be uint8")
    _require_cuda(x, ids, wts, w1, w2, s1, s2, w1_bias)
    M, H = x.shape
    E, two_i, hh = w1.shape
    I = two_i // 2
    topk = ids.shape[1]
    if layout == L.MXQ_LAYOUT_PLAIN:
        rb1, rb2, g1, g2 = H // 2, I // 2, H // 32, I // 32
    else:
        rb1, rb2 = _tiled_row(H // 2), _tiled_row(I // 2)
        g1, g2 = -(-(H // 32) // 8) * 8, -(-(I // 32) // 8) * 8
    if hh != rb1 or tuple(w2.shape) != (E, H, rb2):
        raise ValueError(f"w1 must be [E, 2I, {rb1}] and w2 [E, H, {rb2}] for the {weight_layout} layout")
    if tuple(s1.shape) != (E, 2 * I, g1) or tuple(s2.shape) != (E, H, g2):
        raise ValueError(f"scales must be [E, 2I, {g1}] and [E, H, {g2}] for the {weight_layout} layout")
    b1 = None if w1_bias is None else w1_bias.float().contiguous()
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = fused_moe_workspace(M, H, I, E, topk, L.MXQ_WEIGHTS_MXFP4, False, x.device)
    st = L.load().mxq_fused_moe_mxfp4(x.data_ptr(), M, H, I, E, topk, ids.data_ptr(), wts.data_ptr(),
                                      w1.data_ptr(), s1.data_ptr(), w2.data_ptr(), s2.data_ptr(), _ptr(b1),
                                      layout, _dispatch(dispatch), out.data_ptr(), workspace.data_ptr(),
                                      workspace.numel(), _stream())
    L.check("mxq_fused_moe_mxfp4", st)
    return out
