"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and answers the host-only queries and argument checks
(no kernel is launched here)."""

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")


def _lib():
    from mxfp4_block_scaled_expert_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libmxq.so not built")
    return L, L.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("mxq_per_token_group_quant_fp8", "mxq_fp8_scaled_mm", "mxq_fp8_scaled_bmm", "mxq_block_fp8_linear",
              "mxq_moe_align",
              "mxq_fused_moe_fp8", "mxq_fused_moe_mxfp4", "mxq_moe_prepack", "mxq_moe_prepack_scales"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L, lib = _lib()
    raw = C.CDLL(L.LIB_PATH)
    for n in _declared():
        assert hasattr(raw, n), f"{n} declared in mxq.h but not exported"
        assert n in L.SIGNATURES, f"{n} has no ctypes signature in the binding"


def test_library_exports_no_undeclared_c_symbol():
    """Every unmangled (C-linkage) function the library defines is declared in mxq.h: internal
    helpers stay in C++ namespaces, out of the C ABI."""
    import shutil
    import subprocess
    L, _ = _lib()
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    c_syms = {ln.split()[-1] for ln in out.splitlines() if ln.split()[-2:-1] == ["T"] and not ln.split()[-1].startswith("_Z")}
    assert c_syms == set(_declared()), sorted(c_syms ^ set(_declared()))


def test_dispatch_struct_matches_header():
    from mxfp4_block_scaled_expert_amd import _lib as L
    src = open(HEADER).read()
    body = re.search(r"typedef struct mxq_moe_dispatch \{(.*?)\} mxq_moe_dispatch;", src, re.S).group(1)
    assert [f for f, _ in L.MoeDispatch._fields_] == re.findall(r"int32_t (\w+);", body)


def test_status_strings_and_version():
    L, lib = _lib()
    assert lib.mxq_abi_version() == 14
    for code in range(0, 10):
        assert lib.mxq_status_string(code)
    assert b"unknown" in lib.mxq_status_string(99)


def test_max_blocks_matches_formula():
    _, lib = _lib()
    from oracle.align import max_blocks
    for M, topk, E, bm in [(4096, 8, 256, 128), (32, 4, 128, 128), (128, 1, 8, 16), (0, 2, 4, 8), (3, 2, 100, 4)]:
        assert lib.mxq_moe_max_blocks(M, topk, E, bm) == max_blocks(M, topk, E, bm)


def test_workspace_queries():
    L, lib = _lib()
    assert lib.mxq_block_fp8_linear_workspace_size(2048, 7168, 2048, L.MXQ_DTYPE_E4M3) == 0
    n = lib.mxq_block_fp8_linear_workspace_size(2048, 7168, 2048, L.MXQ_DTYPE_BF16)
    assert n == 2048 * 2048 + 2048 * 16 * 4
    # up to 16 rows: the K split's fp32 partial sums too (S slices of M x N, S a power of two
    # up to 8, at most 8 MiB)
    for M, N, K in [(1, 7168, 2048), (16, 2048, 7168), (16, 65536, 16384), (1, 64, 1024)]:
        q = lib.mxq_block_fp8_linear_workspace_size(M, N, K, L.MXQ_DTYPE_BF16)
        e = lib.mxq_block_fp8_linear_workspace_size(M, N, K, L.MXQ_DTYPE_E4M3)
        assert q - e == ((M * K + 255) // 256 * 256) + ((4 * M * K // 128 + 255) // 256 * 256)
        assert e == 0 or (e % (4 * M * N) == 0 and e // (4 * M * N) in (2, 4, 8) and e <= 8 << 20), (M, N, K, e)
    assert lib.mxq_block_fp8_linear_workspace_size(1, 7168, 2048, L.MXQ_DTYPE_E4M3) > 0
    # past 8 rows only where the row tiles' grid is small (32 workgroups at most)
    assert lib.mxq_block_fp8_linear_workspace_size(17, 7168, 2048, L.MXQ_DTYPE_E4M3) == 0
    # 4 row tiles of 8 x 16 column tiles of 64 = 64 workgroups: 8 chunks fill 512
    assert lib.mxq_block_fp8_linear_workspace_size(32, 1024, 7168, L.MXQ_DTYPE_E4M3) == 8 * 32 * 1024 * 4
    # past 64 rows the weight-streaming path stops and the few-tile K split below takes over
    assert lib.mxq_block_fp8_linear_workspace_size(65, 1024, 7168, L.MXQ_DTYPE_E4M3) == 8 * 65 * 1024 * 4
    # 65..1024 rows on few 128 x 128 tiles with long K: the K split's partial sums (at most
    # 16 MiB, M * K at most 8 M), 16 tiles of 128 x 128 here: 8 chunks
    assert lib.mxq_block_fp8_linear_workspace_size(128, 2048, 7168, L.MXQ_DTYPE_E4M3) == 8 * 128 * 2048 * 4
    assert lib.mxq_block_fp8_linear_workspace_size(2048, 2048, 7168, L.MXQ_DTYPE_E4M3) == 0  # 256 tiles
    assert lib.mxq_block_fp8_linear_workspace_size(1025, 1024, 2048, L.MXQ_DTYPE_E4M3) == 0
    a = lib.mxq_fused_moe_workspace_size(4096, 7168, 2048, 256, 8, L.MXQ_WEIGHTS_FP8_BLOCK, 1)
    b = lib.mxq_fused_moe_workspace_size(4096, 7168, 2048, 256, 8, L.MXQ_WEIGHTS_FP8_BLOCK, 0)
    R = 4096 * 8
    assert a >= R * 2 * 2048 * 2 + R * 7168 * 4  # ic0 + y at least
    assert a != b
    assert lib.mxq_fused_moe_workspace_size(0, 7168, 2048, 256, 8, 0, 1) == 0


def test_argument_errors_before_any_launch():
    L, lib = _lib()
    null = None
    # block size validation ("SGLang PR 35605 review", fp8_utils.py listing)
    for bn, bk in [(1, 32), (64, 64), (128, 64), (2, 128)]:
        st = lib.mxq_block_fp8_linear(null, L.MXQ_DTYPE_BF16, null, 4, 256, 256, null, 256, null, 2, 1, bn, bk,
                                      null, 0, null, L.MXQ_DTYPE_BF16, 256, null, 0, null)
        assert st == L.MXQ_ERR_BLOCK
    # the output dtype is bf16 ("SGLang PR 35605 review", fp8_utils.py listing); others are refused
    for od in (L.MXQ_DTYPE_F32, L.MXQ_DTYPE_E4M3, 9):
        st = lib.mxq_block_fp8_linear(null, L.MXQ_DTYPE_BF16, null, 4, 256, 256, null, 256, null, 2, 1, 128, 128,
                                      null, 0, null, od, 256, null, 0, null)
        assert st == L.MXQ_ERR_DTYPE
    st = lib.mxq_block_fp8_linear(null, L.MXQ_DTYPE_BF16, null, 4, 256, 256, null, 256, null, 2, 1, 128, 128,
                                  null, 0, null, L.MXQ_DTYPE_BF16, 256, null, 0, null)
    assert st == L.MXQ_ERR_NULL
    assert lib.mxq_per_token_group_quant_fp8(null, 4, 256, 256, 64, null, null, null) == L.MXQ_ERR_BLOCK
    assert lib.mxq_per_token_group_quant_fp8(null, 4, 200, 200, 128, null, null, null) == L.MXQ_ERR_SHAPE
    assert lib.mxq_per_token_group_quant_fp8(null, 4, 256, 256, 128, null, null, null) == L.MXQ_ERR_NULL
    assert lib.mxq_per_token_group_quant_fp8(null, 0, 256, 256, 128, null, null, null) == L.MXQ_OK
    assert lib.mxq_fp8_scaled_mm(null, 4, 100, 100, null, 8, null, null, 0, null, 8, null, 0, null) == L.MXQ_ERR_SHAPE
    assert lib.mxq_fp8_scaled_mm(null, 4, 128, 128, null, 8, null, null, 7, null, 8, null, 0, null) == L.MXQ_ERR_NULL
    # few rows with K a multiple of 128: a K split needs its partial sums in the workspace
    assert lib.mxq_fp8_scaled_mm_workspace_size(97, 224, 576) == 0
    n = lib.mxq_fp8_scaled_mm_workspace_size(1, 2048, 7168)
    assert n > 0 and n % (4 * 2048) == 0 and n // (4 * 2048) in (2, 4, 8)
    # K not a multiple of 128: not streamed; the ring-fed tiles (16 of 16 x 128) split K in 8
    assert lib.mxq_fp8_scaled_mm_workspace_size(1, 2048, 7136) == 8 * 2048 * 4
    assert lib.mxq_fp8_scaled_mm_workspace_size(1024, 2048, 7168) == 0  # the tiles fill the GPU
    assert lib.mxq_fp8_scaled_mm_workspace_size(64, 2044, 7168) == 0  # N not a multiple of 8
    fake = C.c_void_p(1 << 20)
    assert lib.mxq_fp8_scaled_mm(fake, 1, 7168, 7168, fake, 2048, fake, null, 0, fake, 2048, null, 0,
                                 null) == L.MXQ_ERR_WORKSPACE
    # batched per-tensor: K % 32, lda, batch limit, overlapping outputs, strides, null pointers
    bmm = lib.mxq_fp8_scaled_bmm
    assert bmm(null, 2, 4, 100, 100, 400, null, 8, 800, null, 0, null, 0, 0, null, 8, 32, null) == L.MXQ_ERR_SHAPE
    assert bmm(null, 70000, 4, 128, 128, 512, null, 8, 1024, null, 0, null, 0, 0, null, 8, 32, null) == L.MXQ_ERR_SHAPE
    assert bmm(null, 2, 4, 128, 128, 512, null, 8, 1024, null, 0, null, 0, 0, null, 8, 31, null) == L.MXQ_ERR_SHAPE
    assert bmm(null, 2, 4, 128, 128, 500, null, 8, 1024, null, 0, null, 0, 0, null, 8, 32, null) == L.MXQ_ERR_SHAPE
    assert bmm(null, 2, 4, 128, 128, 512, null, 8, 1000, null, 0, null, 0, 0, null, 8, 32, null) == L.MXQ_ERR_SHAPE
    fake = C.c_void_p(0x1000)  # never dereferenced: the dtype check comes first
    assert bmm(null, 2, 4, 128, 128, 512, null, 8, 1024, null, 0, fake, 9, 0, null, 8, 32, null) == L.MXQ_ERR_DTYPE
    assert bmm(null, 2, 4, 128, 128, 512, null, 8, 1024, null, 0, null, 0, 0, null, 8, 32, null) == L.MXQ_ERR_NULL
    assert bmm(null, 2, 4, 128, 128, 0, null, 8, 0, null, 0, null, 0, 0, null, 8, 32, null) == L.MXQ_ERR_NULL
    assert bmm(null, 0, 4, 128, 128, 512, null, 8, 1024, null, 0, null, 0, 0, null, 8, 32, null) == L.MXQ_OK
    fp8 = lib.mxq_fused_moe_fp8
    mx4 = lib.mxq_fused_moe_mxfp4
    assert fp8(null, 4, 100, 128, 8, 2, null, null, null, null, null, null, null, 0, 0, null, null, null, 0,
               null) == L.MXQ_ERR_SHAPE
    assert mx4(null, 4, 100, 128, 8, 2, null, null, null, null, null, null, null, 0, null, null, null, 0,
               null) == L.MXQ_ERR_SHAPE
    assert fp8(null, 4, 256, 128, 8, 2, null, null, null, null, null, null, null, 0, 0, null, null, null, 0,
               null) == L.MXQ_ERR_NULL
    assert fp8(null, 4, 256, 128, 8, 2, null, null, null, null, null, null, null, 0, 2, null, null, null, 0,
               null) == L.MXQ_ERR_ARG
    assert mx4(null, 4, 256, 128, 8, 2, null, null, null, null, null, null, null, 5, null, null, null, 0,
               null) == L.MXQ_ERR_ARG
    # per-call dispatch: every field validated before any pointer is looked at
    for bad in ((7, 0, 4, 0, 0, 0, 0), (0, 0, 17, 0, 0, 0, 0), (0, 0, -2, 0, 0, 0, 0), (0, 0, 4, 5, 0, 0, 0),
                (1, 5, 16, 0, 0, 0, 0), (1, -1, 16, 0, 0, 0, 0), (0, 0, 4, 0, 3, 0, 0), (0, 0, 4, 0, -1, 0, 0),
                (0, 0, 4, 0, 16, 0, 0), (0, 0, 4, 0, 0, 2, 0), (0, 0, 4, 0, 0, -1, 0), (0, 0, 4, 0, 0, 0, 2),
                (0, 0, 4, 0, 0, 0, -1)):
        d = C.byref(L.MoeDispatch(*bad))
        assert fp8(null, 4, 256, 128, 8, 2, null, null, null, null, null, null, null, 0, 0, d, null, null, 0,
                   null) == L.MXQ_ERR_ARG, bad
        assert mx4(null, 4, 256, 128, 8, 2, null, null, null, null, null, null, null, 0, d, null, null, 0,
                   null) == L.MXQ_ERR_ARG, bad
    for good in ((0, 0, 16, 0, 0, 0, 0), (1, 4, 4, 1, 1, 1, 1), (2, 0, 0, 0, 2, 0, 1), (0, 0, -1, 0, 4, 1, 0),
                 (0, 0, 8, 0, 8, 0, 1)):
        d = C.byref(L.MoeDispatch(*good))
        assert fp8(null, 4, 256, 128, 8, 2, null, null, null, null, null, null, null, 0, 0, d, null, null, 0,
                   null) == L.MXQ_ERR_NULL, good
    # SiLU-and-mul: I % 8 (I % 128 when re-quantising), ld_in >= 2I, required pointers
    sm = lib.mxq_silu_and_mul
    assert sm(null, 4, 100, 200, null, null, null, null) == L.MXQ_ERR_SHAPE
    assert sm(null, 4, 64, 100, null, null, null, null) == L.MXQ_ERR_SHAPE
    assert sm(null, 4, 64, 128, null, fake, null, null) == L.MXQ_ERR_SHAPE
    assert sm(null, 4, 64, 128, null, null, null, null) == L.MXQ_ERR_NULL
    assert sm(null, 4, 128, 256, null, fake, null, null) == L.MXQ_ERR_NULL
    assert sm(null, 0, 128, 256, null, null, null, null) == L.MXQ_OK
    # load-time relayout: N and row bytes multiples of 16
    assert lib.mxq_moe_prepack(null, 2, 24, 128, null, null) == L.MXQ_ERR_SHAPE
    assert lib.mxq_moe_prepack(null, 2, 32, 136, null, null) == L.MXQ_ERR_SHAPE
    assert lib.mxq_moe_prepack(null, 2, 32, 128, null, null) == L.MXQ_ERR_NULL
    assert lib.mxq_moe_prepack_scales(null, 2, 24, 90, null, null) == L.MXQ_ERR_SHAPE
    assert lib.mxq_moe_prepack_scales(null, 2, 32, 90, null, null) == L.MXQ_ERR_NULL
    assert lib.mxq_moe_align(null, 4, 2, 2000, 16, null, null, null, null, null) == L.MXQ_ERR_SHAPE



def test_moe_workspace_layout_query():
    """Every region lies inside the workspace, regions do not overlap, and each is as large as
    its tensor; unused regions report -1."""
    L, lib = _lib()
    from mxfp4_block_scaled_expert_amd.ops import fused_moe_workspace_layout
    for (M, H, I, E, topk, wf, aq) in [(4096, 7168, 2048, 256, 8, L.MXQ_WEIGHTS_FP8_BLOCK, 1),
                                       (128, 2048, 1024, 8, 1, L.MXQ_WEIGHTS_FP8_BLOCK, 0),
                                       (32, 2880, 2880, 128, 4, L.MXQ_WEIGHTS_MXFP4, 0)]:
        lay = fused_moe_workspace_layout(M, H, I, E, topk, wf, aq)
        total = lib.mxq_fused_moe_workspace_size(M, H, I, E, topk, wf, aq)
        R = M * topk
        bm = lay["block_m"]
        mb = lib.mxq_moe_max_blocks(M, topk, E, bm)
        size = {"sorted_ids": 4 * mb * bm, "expert_ids": 4 * mb, "offsets": 4 * (mb + 1), "num_blocks": 4,
                "qx": M * H, "sx": 4 * M * (H // 128), "ic0": 2 * R * 2 * I, "ic1": 2 * R * I,
                "ic1_q": R * I, "ic1_s": 4 * R * (I // 128), "y": 4 * R * H,
                "partial": 4 * 8 * R * max(2 * I, H)}  # K-split slices: 8 for R = 128
        used = {k: v for k, v in lay.items() if k != "block_m" and v >= 0}
        if aq:
            assert lay["ic1"] == -1 and min(lay["qx"], lay["sx"], lay["ic1_q"], lay["ic1_s"]) >= 0
        else:
            assert lay["qx"] == lay["sx"] == lay["ic1_q"] == lay["ic1_s"] == -1 and lay["ic1"] >= 0
        assert (lay["partial"] >= 0) == (not aq and R <= 1024)
        spans = sorted((v, v + size[k], k) for k, v in used.items())
        for (a0, a1, ka), (b0, b1, kb) in zip(spans, spans[1:]):
            assert a1 <= b0, (ka, kb)
        assert spans[-1][1] <= total
        assert all(v % 256 == 0 for v in used.values())
    arr = (C.c_int64 * 13)()
    assert lib.mxq_fused_moe_workspace_layout(0, 7168, 2048, 256, 8, 0, 1, arr) == L.MXQ_ERR_SHAPE
    assert lib.mxq_fused_moe_workspace_layout(4, 256, 128, 8, 2, 0, 1, None) == L.MXQ_ERR_NULL


def test_prepack_size_queries():
    _, lib = _lib()
    # weights: E * N * ceil(row_bytes / 128) * 128
    assert lib.mxq_moe_prepack_size(128, 5760, 1440) == 128 * 5760 * 1536
    assert lib.mxq_moe_prepack_size(256, 4096, 7168) == 256 * 4096 * 7168
    assert lib.mxq_moe_prepack_size(2, 24, 128) == 0
    # MX scales: E * N * ceil(groups / 8) * 8
    assert lib.mxq_moe_prepack_scales_size(128, 5760, 90) == 128 * 5760 * 96
    assert lib.mxq_moe_prepack_scales_size(1, 16, 8) == 16 * 8
    assert lib.mxq_moe_prepack_scales_size(1, 8, 8) == 0


def test_binding_rejects_bad_block_size_without_gpu():
    import torch
    from mxfp4_block_scaled_expert_amd import ops
    x = torch.zeros(2, 256, dtype=torch.bfloat16)
    w = torch.zeros(256, 256, dtype=torch.uint8)
    s = torch.ones(2, 2)
    for bs in ([1, 32], [64, 64], [128], (128, 128, 1)):
        with pytest.raises(ValueError):
            ops.block_fp8_linear(x, w, bs, s)


def test_batched_binding_rejects_mismatched_shapes_without_gpu():
    import torch
    from mxfp4_block_scaled_expert_amd import ops
    x = torch.zeros(2, 4, 256, dtype=torch.bfloat16)
    w = torch.zeros(2, 128, 256, dtype=torch.uint8)
    with pytest.raises(ValueError):
        ops.fp8_scaled_bmm(x, torch.zeros(3, 128, 256, dtype=torch.uint8), torch.ones(1))
    with pytest.raises(ValueError):
        ops.fp8_scaled_bmm(x, torch.zeros(2, 128, 128, dtype=torch.uint8), torch.ones(1))
    with pytest.raises(ValueError):
        ops.fp8_scaled_bmm(x, w, torch.ones(3))
    with pytest.raises(ValueError):
        ops.fp8_scaled_bmm(x, w, torch.ones(1), torch.zeros(3, 128))
    with pytest.raises(ValueError):
        ops.fp8_scaled_bmm(x.float(), w, torch.ones(1))


def test_fused_moe_plan_host_logic():
    """The host-side plan of a fused-MoE call (mxq_fused_moe_plan: no device touched) for the
    workloads' shapes and the dispatch knobs: which path, tiles, block sizes, K splits and
    fusions the call runs."""
    L, _ = _lib()
    from mxfp4_block_scaled_expert_amd.ops import Dispatch, fused_moe_plan
    FP8, MX = L.MXQ_WEIGHTS_FP8_BLOCK, L.MXQ_WEIGHTS_MXFP4
    # small-block W8A16 (128 tokens top-1 over 8 experts): self-routed 16-row blocks fill the
    # GPU, no K split, the SiLU-and-mul and the combine in the stage epilogues
    c3 = fused_moe_plan(128, 2048, 1024, 8, 1, FP8, weight_layout="tiled")
    assert c3["path"] == "self_routed" and c3["tiles"] == "ring" and 0 not in c3["classes"]
    assert (c3["block_m1"], c3["block_m2"], c3["k_split1"], c3["k_split2"]) == (16, 16, 1, 1)
    assert (c3["silu"], c3["combine"]) == ("stage1_epilogue", "stage2_epilogue")
    # the knobs: no fusion; the sort kept (same splits, so the same sums); a forced K split
    nf = fused_moe_plan(128, 2048, 1024, 8, 1, FP8, dispatch=Dispatch(fuse=L.MXQ_FUSE_NONE))
    assert (nf["path"], nf["silu"], nf["combine"]) == ("self_routed", "kernel", "kernel")
    so = fused_moe_plan(128, 2048, 1024, 8, 1, FP8, dispatch=Dispatch(sort=L.MXQ_SORT_ALWAYS))
    assert (so["path"], so["block_m1"], so["k_split1"], so["k_split2"]) == ("sorted", 128, 1, 1)
    assert (so["silu"], so["combine"]) == ("stage1_epilogue", "kernel")
    ks = fused_moe_plan(128, 2048, 1024, 8, 1, FP8, dispatch=Dispatch(k_split=2))
    assert (ks["k_split1"], ks["k_split2"], ks["silu"], ks["combine"]) == (2, 2, "split_sum", "kernel")
    # 256 tokens top-2 over 8 experts: 64-row self-routed blocks, SiLU fused, top-2 combine kernel
    m256 = fused_moe_plan(256, 2048, 1024, 8, 2, FP8)
    assert (m256["path"], m256["block_m1"], m256["k_split1"]) == ("self_routed", 64, 1)
    assert (m256["silu"], m256["combine"]) == ("stage1_epilogue", "kernel")
    # the largest self-routed routing is 2048 routed rows (512 tokens top-4); one token more sorts
    r2k = fused_moe_plan(512, 2048, 1024, 64, 4, FP8)
    assert (r2k["path"], r2k["block_m1"], r2k["k_split1"]) == ("self_routed", 64, 1)
    assert fused_moe_plan(513, 2048, 1024, 64, 4, FP8)["path"] == "sorted"
    # GPT-OSS decode (32 tokens top-4 over 128 MXFP4 experts): every block tiny, expert streaming;
    # with the sort kept the sorted path runs unsplit too (the same sums)
    c4 = fused_moe_plan(32, 2880, 2880, 128, 4, MX, weight_layout="tiled")
    assert (c4["path"], c4["silu"]) == ("expert_stream", "expert_stream")
    for d in (Dispatch(sort=L.MXQ_SORT_ALWAYS), Dispatch(fuse=L.MXQ_FUSE_NONE)):
        p = fused_moe_plan(15, 384, 512, 1, 1, FP8, dispatch=d)
        assert (p["path"], p["classes"], p["k_split1"], p["k_split2"]) == ("sorted", {0}, 1, 1)
    # MXFP4 on the plain layout with K % 128 != 0: the register-staged tiles, sorted
    mxp = fused_moe_plan(40, 2880, 2880, 8, 4, MX)
    assert (mxp["path"], mxp["tiles"]) == ("sorted", "register")
    assert fused_moe_plan(40, 2880, 2880, 8, 4, MX, weight_layout="tiled")["tiles"] == "ring"
    # DeepSeek prefill (4096 tokens top-8 over 256 experts, W8A8): sorted, every class folded into
    # the 128-row class on the 128 x 256 tile, the SiLU-and-mul with its re-quantisation and the
    # combine as kernels
    c5 = fused_moe_plan(4096, 7168, 2048, 256, 8, FP8, act_quant=True, weight_layout="tiled")
    assert (c5["path"], c5["tiles"], c5["classes"]) == ("sorted", "w8a8_wide", {4})
    assert (c5["block_m1"], c5["k_split1"], c5["silu"], c5["combine"]) == (128, 1, "kernel", "kernel")
    # refusals, as the call's
    lib = L.load()
    arr = (C.c_int32 * len(L.MOE_PLAN_FIELDS))()
    assert lib.mxq_fused_moe_plan(4, 256, 256, 8, 2, 7, 0, 0, None, arr) == L.MXQ_ERR_ARG
    assert lib.mxq_fused_moe_plan(4, 256, 256, 8, 2, MX, 1, 0, None, arr) == L.MXQ_ERR_ARG
    assert lib.mxq_fused_moe_plan(4, 200, 256, 8, 2, FP8, 0, 0, None, arr) == L.MXQ_ERR_SHAPE
    assert lib.mxq_fused_moe_plan(0, 256, 256, 8, 2, FP8, 0, 0, None, arr) == L.MXQ_ERR_SHAPE
    assert lib.mxq_fused_moe_plan(4, 256, 256, 8, 9, FP8, 0, 0, None, arr) == L.MXQ_ERR_SHAPE
    assert lib.mxq_fused_moe_plan(4, 256, 256, 8, 2, FP8, 0, 0, None, None) == L.MXQ_ERR_NULL
