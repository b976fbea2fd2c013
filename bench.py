"""Benchmark of the scaled low-precision GEMM / routed fused-MoE hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-secondary]

Headline workload: block-wise FP8 W8A8 linear, bf16 A [2048, 2048] quantised per
token per 128 columns, e4m3 W [7168, 2048] (0.05 * randn quantised per 128x128
block), bf16 out.  One step = the 1x128 quantisation kernel + the block-scaled
FP8 GEMM, on rotating input sets (> 600 MB in total, so the 256 MB last-level
cache cannot hold the operands between steps), each with its own quantised
buffers.  Inputs are resident in HBM before the timed region starts.

Timing: W warm-up steps, and more until 0.3 s of untimed load has passed (the
clocks settle), then exactly K steps in one window with a HIP event at every
kernel boundary on the kernels' stream: the step, the quantiser and the GEMM
durations come from the same window (median, p10, p90 reported).

Printed: ONE JSON line with the throughput of the step (TFLOP/s), the roofline
of the dominant kernel (the GEMM, against the FP8 dense MFMA peak; its HBM
traffic from the counter profile while the kernel sources are unchanged), the
CPU oracle's throughput on a sample of the same workload, and secondary
measurements: the per-tensor W8A16 GEMM, the small-block W8A16 MoE, the two
routed-MoE workloads (GPT-OSS-shaped MXFP4 decode, DeepSeek-shaped W8A8
prefill) and the batched W8A16 GEMM on MLA-shaped per-head products.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused-MoE & block-FP8 GEMM TFLOP/s + weight GB/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0
# Untimed steps before every timed region last at least this long (the W warm-up steps
# included): with a few steps only, the clocks have not settled and the GEMM measures ~15 %
# slower than after a fraction of a second of load.
SETTLE_S = 0.3

# HBM traffic of the headline GEMM comes from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE) taken on
# this workload and recorded, with a hash of the kernel's sources, in the profile summary below;
# it is reported only while the sources still hash to that value (else null: the counters no
# longer describe the kernel).
GEMM_PROFILE = os.path.join(ROOT, "profiles", "gemm_w8a8_big_block_linear_2048x2048x7168.md")
GEMM_SOURCES = ("gemm_w8a8_big.hip", "lds_dma.hpp", "tile_rows.hpp", "common.hpp", "kernels.hpp")


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--settle", type=float, default=None,
                   help="seconds of untimed load before each timed window (default 0.3; profiling runs use 0)")
    p.add_argument("--sweep-shape", default=None, help="class sweep: comma list of shapes (default all)")
    p.add_argument("--sweep-m", default=None, help="class sweep: comma list of rows per block (default all)")
    p.add_argument("--only", choices=["linear", "decode", "prefill", "small", "mx", "copy", "ablation", "classes"],
                   default=None,
                   help="time one workload only (profiling runs); small = the per-tensor GEMM and the "
                        "small-block W8A16 MoE; copy = counter calibration; ablation = per-block vs "
                        "per-layer tile-class dispatch")
    return p.parse_args()


def _lib():
    from mxfp4_block_scaled_expert_amd import _lib as L
    return L, L.load()


def _check(st, what):
    if st != 0:
        raise RuntimeError(f"{what} failed with status {st}")


def sources_sha16(names=GEMM_SOURCES) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mxfp4_block_scaled_expert_amd", "csrc", n), "rb") as f:
            h.update(n.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stamped_traffic():
    """(bytes per launch or None, note) from the profile's `traffic-stamp:` line."""
    try:
        with open(GEMM_PROFILE) as f:
            line = next((l for l in f if l.startswith("traffic-stamp:")), None)
    except OSError:
        return None, "no profile"
    if line is None:
        return None, "no traffic stamp in the profile"
    stamp = json.loads(line.split(":", 1)[1])
    if stamp.get("sources_sha16") != sources_sha16():
        return None, "kernel sources changed since the counters were taken"
    return int(stamp["traffic_bytes"]), f"FETCH_SIZE/{stamp['fetch_scale']} + WRITE_SIZE/{stamp['write_scale']}"


# ----------------------------------------------------------------------------- timing

class _HipEvents:
    """Timing events created with hipEventDisableSystemFence, on the HIP runtime torch already
    loaded: recording one costs no cache write-back or invalidation, so an event between every
    two kernels barely perturbs them (torch's events do: ~2-3 µs per record here)."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        self.h = ctypes.CDLL(path)
        self.h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            _check(self.h.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE), "hipEventCreate")
            evs.append(e)
        return evs

    def record(self, e, stream: int):
        _check(self.h.hipEventRecord(e, ctypes.c_void_p(stream)), "hipEventRecord")

    def us(self, a, b) -> float:
        """µs between two recorded events (after a device synchronisation)."""
        ms = ctypes.c_float()
        _check(self.h.hipEventElapsedTime(ctypes.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value * 1e3

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(e)


_HIP = None


def _hip():
    global _HIP
    if _HIP is None:
        _HIP = _HipEvents()
    return _HIP


def _stats(us):
    a = np.asarray(us, np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def _settle(step, warmup: int) -> int:
    """`warmup` untimed steps, then more until SETTLE_S of wall time has passed."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < SETTLE_S:
        step(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()  # bounded queue; wall time tracks the GPU
    torch.cuda.synchronize()
    return i


def _time_calls(run, steps: int, warmup: int):
    """Per-call µs of `steps` back-to-back calls (an event between every two calls, all on the
    calls' stream), after the settle pre-roll.  Returns (stats, total µs of the window)."""
    _settle(lambda i: run(), warmup)
    hip = _hip()
    sh = torch.cuda.current_stream().cuda_stream
    ev = hip.create(steps + 1)
    hip.record(ev[0], sh)
    for i in range(steps):
        run()
        hip.record(ev[i + 1], sh)
    torch.cuda.synchronize()
    per = [hip.us(ev[i], ev[i + 1]) for i in range(steps)]
    total = hip.us(ev[0], ev[steps])
    hip.destroy(ev)
    return _stats(per), total


# ----------------------------------------------------------------------------- headline

def bench_linear(steps: int, warmup: int):
    """Headline step = the 1x128 quantiser + the block-FP8 GEMM on one of several rotating input
    sets (each with its own quantised buffers; > 600 MB in all, beyond the 256 MB last-level
    cache).  One timed window of exactly `steps` steps with an event at every kernel boundary,
    so the step, the quantiser and the GEMM durations all come from the same window."""
    from mxfp4_block_scaled_expert_amd import synth
    L, lib = _lib()
    dev = torch.device("cuda", 0)
    M, K, N = 2048, 2048, 7168
    per_set = M * K * 3 + N * K + (N // 128) * (K // 128) * 4 + M * (K // 128) * 4
    n_rot = max(2, -(-(600 << 20) // per_set))
    sets = [synth.block_linear(M, N, K, seed=1002 + i, device=dev) for i in range(n_rot)]
    for d in sets:
        d["q"] = torch.empty(M, K, dtype=torch.uint8, device=dev)
        d["s"] = torch.empty(M, K // 128, dtype=torch.float32, device=dev)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    sh = torch.cuda.current_stream().cuda_stream

    def quant(d):
        _check(lib.mxq_per_token_group_quant_fp8(d["x"].data_ptr(), M, K, K, 128, d["q"].data_ptr(),
                                                 d["s"].data_ptr(), sh), "quant")

    def gemm(d):
        _check(lib.mxq_block_fp8_linear(d["q"].data_ptr(), L.MXQ_DTYPE_E4M3, d["s"].data_ptr(), M, K, K,
                                        d["w"].data_ptr(), N, d["sw"].data_ptr(), K // 128, 1, 128, 128, None, 0,
                                        out.data_ptr(), L.MXQ_DTYPE_BF16, N, None, 0, sh), "block_fp8_linear")

    def step(i):
        d = sets[i % n_rot]
        quant(d)
        gemm(d)

    settled = _settle(step, warmup)
    hip = _hip()
    ev = hip.create(2 * steps + 1)
    t0 = time.perf_counter()
    hip.record(ev[0], sh)
    for i in range(steps):
        d = sets[(settled + i) % n_rot]
        quant(d)
        hip.record(ev[2 * i + 1], sh)
        gemm(d)
        hip.record(ev[2 * i + 2], sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = [hip.us(ev[2 * i], ev[2 * i + 2]) for i in range(steps)]
    quant_us = [hip.us(ev[2 * i], ev[2 * i + 1]) for i in range(steps)]
    gemm_us = [hip.us(ev[2 * i + 1], ev[2 * i + 2]) for i in range(steps)]
    window_us = hip.us(ev[0], ev[2 * steps])
    hip.destroy(ev)

    flops = 2.0 * M * N * K
    gemm_bytes = M * K + M * (K // 128) * 4 + N * K + (N // 128) * (K // 128) * 4 + M * N * 2
    return {
        "M": M, "K": K, "N": N, "flops": flops, "rotating_sets": n_rot, "settle_steps": settled,
        "ms_per_step": window_us / steps / 1e3, "wall_ms_per_step": wall * 1e3 / steps,
        "step_us": _stats(step_us), "quant_us": _stats(quant_us), "gemm_us": _stats(gemm_us),
        "gemm_alg_bytes": gemm_bytes,
    }


def bench_linear_small(steps: int, warmup: int, M: int, N: int, K: int):
    """A block-FP8 W8A8 linear of few rows or few tiles (pre-quantised e4m3 input, 128x128 weight
    blocks) on rotating weight sets beyond the last-level cache, per-call events: the
    weight-streaming path (few rows) or the K-split 128x128 tiles (few tiles); reported with the
    weight bytes' rate against HBM."""
    from mxfp4_block_scaled_expert_amd import synth
    L, lib = _lib()
    dev = torch.device("cuda", 0)
    n_rot = max(2, -(-(600 << 20) // (N * K)))
    base = synth.block_linear(M, N, K, seed=4242, device=dev)
    q = torch.empty(M, K, dtype=torch.uint8, device=dev)
    sq = torch.empty(M, K // 128, dtype=torch.float32, device=dev)
    sh = torch.cuda.current_stream().cuda_stream
    _check(lib.mxq_per_token_group_quant_fp8(base["x"].data_ptr(), M, K, K, 128, q.data_ptr(), sq.data_ptr(), sh),
           "quant")
    ws_n = lib.mxq_block_fp8_linear_workspace_size(M, N, K, L.MXQ_DTYPE_E4M3)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    ws_list = [base["w"]] + [torch.randint(0, 256, (N, K), dtype=torch.uint8, device=dev) & 0x77
                             for _ in range(n_rot - 1)]
    it = [0]

    def run():
        w = ws_list[it[0] % n_rot]
        it[0] += 1
        _check(lib.mxq_block_fp8_linear(q.data_ptr(), L.MXQ_DTYPE_E4M3, sq.data_ptr(), M, K, K, w.data_ptr(), N,
                                        base["sw"].data_ptr(), K // 128, 1, 128, 128, None, 0, out.data_ptr(),
                                        L.MXQ_DTYPE_BF16, N, ws.data_ptr(), ws_n, sh), "block_fp8_linear")
    st, _ = _time_calls(run, steps, warmup)
    wbytes = N * K
    return {"workload": f"block_w8a8_linear_{M}x{K}x{N}", "us": st,
            "tflops": 2.0 * M * N * K / (st["median"] * 1e-6) / 1e12,
            "weight_tbs": wbytes / (st["median"] * 1e-6) / 1e12,
            "hbm_frac": wbytes / (st["median"] * 1e-6) / 8e12, "k_split_workspace_bytes": ws_n}


def bench_per_tensor(steps: int, warmup: int):
    """The per-tensor W8A16 GEMM of the SGLang CPU page's test, bf16 [97, 576] x e4m3 [224, 576]^T
    with an fp32 bias: launch-latency bound (0.29 MB, 25 MFLOP), reported in µs."""
    from mxfp4_block_scaled_expert_amd import synth
    L, lib = _lib()
    dev = torch.device("cuda", 0)
    M, K, N = 97, 576, 224
    d = synth.dense_w8a16(M, N, K, seed=1001, device=dev)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    sh = torch.cuda.current_stream().cuda_stream
    ws_n = lib.mxq_fp8_scaled_mm_workspace_size(M, N, K)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def run():
        _check(lib.mxq_fp8_scaled_mm(d["a"].data_ptr(), M, K, K, d["w"].data_ptr(), N, d["scale"].data_ptr(),
                                     d["bias"].data_ptr(), L.MXQ_DTYPE_F32, out.data_ptr(), N, ws.data_ptr(), ws_n,
                                     sh), "fp8_scaled_mm")
    st, _ = _time_calls(run, steps, warmup)
    byts = M * K * 2 + N * K + N * 4 + M * N * 2
    return {"workload": "per_tensor_w8a16_97x576x224", "us": st, "tflops": 2.0 * M * N * K / (st["median"] * 1e-6) / 1e12,
            "gbs": byts / (st["median"] * 1e-6) / 1e9}


def bench_mx(steps: int, warmup: int, w_format: str):
    """The MX-scaled linear at the headline size, 2048 x 2048 x 7168: MXFP8 activations (e4m3 +
    e8m0 per 32, quantised before timing) x MXFP4 (``e2m1``) or MXFP8 (``e4m3``) weights, on
    rotating input sets beyond the last-level cache; and the MXFP8 quantiser of the bf16 input."""
    from mxfp4_block_scaled_expert_amd import synth
    L, lib = _lib()
    dev = torch.device("cuda", 0)
    M, K, N = 2048, 2048, 7168
    wbytes = N * K // (2 if w_format == "e2m1" else 1)
    per_set = M * K * 3 + wbytes + N * K // 32 + M * K // 32
    n_rot = max(2, -(-(600 << 20) // per_set))
    sets = []
    for i in range(n_rot):
        d = synth.mx_linear(M, N, K, seed=3000 + i, device=dev, w_format=w_format)
        d["q"] = torch.empty(M, K, dtype=torch.uint8, device=dev)
        d["s"] = torch.empty(M, K // 32, dtype=torch.uint8, device=dev)
        sets.append(d)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    sh = torch.cuda.current_stream().cuda_stream
    wd = L.MXQ_DTYPE_E2M1 if w_format == "e2m1" else L.MXQ_DTYPE_E4M3
    it = [0]

    def quant():
        d = sets[it[0] % n_rot]
        it[0] += 1
        _check(lib.mxq_mxfp8_quant(d["x"].data_ptr(), M, K, K, d["q"].data_ptr(), d["s"].data_ptr(), sh), "quant")

    def gemm():
        d = sets[it[0] % n_rot]
        it[0] += 1
        _check(lib.mxq_mx_linear(d["q"].data_ptr(), L.MXQ_DTYPE_E4M3, d["s"].data_ptr(), M, K, K, d["w"].data_ptr(),
                                 wd, N, d["sw"].data_ptr(), None, 0, out.data_ptr(), N, None, 0, sh), "mx_linear")
    for _ in range(n_rot):
        quant()
    q_st, _ = _time_calls(quant, steps, warmup)
    g_st, _ = _time_calls(gemm, steps, warmup)
    flops = 2.0 * M * N * K
    us = g_st["mean"]
    return {"workload": f"mx_linear_2048x2048x7168 MXFP8 activations x {'MXFP4' if w_format == 'e2m1' else 'MXFP8'} "
                        "weights", "gemm_us": g_st, "quant_us": q_st, "tflops": flops / (us * 1e-6) / 1e12,
            "fp8_mfma_frac": flops / (us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS}


# ----------------------------------------------------------------------------- MoE workloads

def _touched_bytes(inp) -> int:
    ids = inp["topk_ids"].cpu().numpy()
    used = np.unique(ids)
    per = 0
    for k in ("w1", "w2", "w1_scale", "w2_scale", "w1_bias"):
        t = inp.get(k)
        if t is not None:
            per += t[0].numel() * t.element_size()
    M, H = inp["x"].shape
    return int(used.size * per + 2 * M * H * 2 + ids.size * 8)


def _moe_setup(name_or_spec, seed: int, layout: str = "tiled", M=None, dispatch=None):
    """Inputs (weights prepacked once for ``layout="tiled"``, as a model would at weight-loading
    time), workspace and a closure running one fused-MoE call."""
    from mxfp4_block_scaled_expert_amd import ops, synth
    from mxfp4_block_scaled_expert_amd import _lib as L
    dev = torch.device("cuda", 0)
    inp = synth.moe_inputs(name_or_spec, seed=seed, device=dev, M=M)
    byts = _touched_bytes(inp)
    if layout == "tiled":
        for k in ("w1", "w2"):
            inp[k] = ops.moe_prepack(inp[k])
        if inp["kind"] == "fused_moe_mxfp4":
            for k in ("w1_scale", "w2_scale"):
                inp[k] = ops.moe_prepack_scales(inp[k])
        torch.cuda.synchronize()
    Mt, H = inp["x"].shape
    I, E, topk = inp["I"], inp["E"], inp["topk"]
    mx = inp["kind"] == "fused_moe_mxfp4"
    ws = ops.fused_moe_workspace(Mt, H, I, E, topk, L.MXQ_WEIGHTS_MXFP4 if mx else L.MXQ_WEIGHTS_FP8_BLOCK,
                                 inp["act_quant"], dev)
    out = torch.empty(Mt, H, dtype=torch.bfloat16, device=dev)

    def run():
        if mx:
            ops.fused_moe_mxfp4(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"],
                                inp["w2"], inp["w2_scale"], inp["w1_bias"], workspace=ws, out=out,
                                weight_layout=layout, dispatch=dispatch[0] if dispatch else None)
        else:
            ops.fused_moe_fp8(inp["x"], inp["topk_ids"], inp["topk_weights"], inp["w1"], inp["w1_scale"],
                              inp["w2"], inp["w2_scale"], None, act_quant=inp["act_quant"], workspace=ws, out=out,
                              weight_layout=layout, dispatch=dispatch[0] if dispatch else None)

    flops = 2.0 * Mt * topk * (2 * I * H + H * I)
    return {"inp": inp, "run": run, "out": out, "bytes": byts, "flops": flops, "M": Mt}


def bench_moe(name: str, steps: int, warmup: int, seed: int, layout: str = "tiled"):
    """Times one fused-MoE workload: per-call durations (median, p10, p90), throughput from the
    median."""
    w = _moe_setup(name, seed, layout)
    st, _ = _time_calls(w["run"], steps, warmup)
    us = st["median"]
    byts, flops = w["bytes"], w["flops"]
    return {
        "workload": name, "weight_layout": layout, "us": st, "tflops": flops / (us * 1e-6) / 1e12,
        "touched_bytes": byts, "weight_gbs": byts / (us * 1e-6) / 1e9,
        "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "fp8_mfma_frac": flops / (us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS,
        "distinct_experts": int(np.unique(w["inp"]["topk_ids"].cpu().numpy()).size),
        "plan": _moe_plan(w["inp"], layout),
    }


def _moe_plan(inp, layout: str):
    """The kernel plan the timed call runs (mxq_fused_moe_plan), classes as a sorted list."""
    from mxfp4_block_scaled_expert_amd import ops
    from mxfp4_block_scaled_expert_amd import _lib as L
    M, H = inp["x"].shape
    mx = inp["kind"] == "fused_moe_mxfp4"
    p = ops.fused_moe_plan(M, H, inp["I"], inp["E"], inp["topk"], L.MXQ_WEIGHTS_MXFP4 if mx else L.MXQ_WEIGHTS_FP8_BLOCK,
                           act_quant=bool(inp["act_quant"]), weight_layout=layout)
    p["classes"] = sorted(p["classes"])
    return p


def bench_mla_bmm(steps: int, warmup: int, tokens: int = 64):
    """Batched per-tensor W8A16 on MLA-shaped per-head products (128 heads): the key side
    [T, 128] x [512, 128]^T and the value side [T, 512] x [128, 512]^T, through the C ABI on
    rotating weight sets."""
    from mxfp4_block_scaled_expert_amd import synth
    _, lib = _lib()
    dev = torch.device("cuda", 0)
    st = torch.cuda.current_stream()
    res = {}
    for name, (N, K) in (("key", (512, 128)), ("value", (128, 512))):
        B, T = 128, tokens
        sets = [synth.batched_w8a16(B, T, N, K, seed=2000 + i, device=dev, has_bias=False) for i in range(8)]
        out = torch.empty(B, T, N, dtype=torch.bfloat16, device=dev)
        it = [0]

        def run():
            d = sets[it[0] % len(sets)]
            it[0] += 1
            _check(lib.mxq_fp8_scaled_bmm(d["a"].data_ptr(), B, T, K, K, T * K, d["w"].data_ptr(), N, N * K,
                                          d["scale"].data_ptr(), 1, None, 0, 0, out.data_ptr(), N, T * N,
                                          st.cuda_stream), "mxq_fp8_scaled_bmm")
        st_, _ = _time_calls(run, steps, warmup)
        us = st_["median"]
        byts = B * N * K + B * T * K * 2 + B * T * N * 2
        res[name] = {"shape": f"{B}x[{T},{K}]x[{N},{K}]^T", "us": st_, "gbs": byts / (us * 1e-6) / 1e9,
                     "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        del sets
    return res


def bench_dispatch_ablation(steps: int, warmup: int):
    """The pages' central comparison at kernel level: each expert block choosing its tile class
    from its own row count (the default) against one class for the whole layer chosen from the
    average rows per expert, over decode batch sizes and routing skews.  One JSON line per case;
    `speedup` = layer-average time / per-block time."""
    from mxfp4_block_scaled_expert_amd import ops, synth
    from mxfp4_block_scaled_expert_amd import _lib as L
    ds = dict(kind="fused_moe_fp8", E=256, topk=8, H=7168, I=2048, act_quant=True)
    cases = [
        ("c3 counts (4,5,33,0,0,12,1,73), W8A16", "moe_block_fp8_w8a16_e8_h2048_i1024", None, 1003),
        ("GPT-OSS MXFP4 decode M=32", "moe_mxfp4_gptoss_decode_m32", 32, 1004),
        ("GPT-OSS MXFP4 decode M=64", "moe_mxfp4_gptoss_decode_m32", 64, 1004),
        ("DeepSeek W8A8 M=64 Zipf 1.1", dict(ds, zipf=1.1), 64, 1005),
        ("DeepSeek W8A8 M=512 uniform", dict(ds, zipf=0.0), 512, 1005),
        ("DeepSeek W8A8 M=512 Zipf 1.1", dict(ds, zipf=1.1), 512, 1005),
        ("DeepSeek W8A8 M=4096 uniform", dict(ds, zipf=0.0), 4096, 1005),
        ("DeepSeek W8A8 M=4096 Zipf 1.1", dict(ds, zipf=1.1), 4096, 1005),
    ]
    rows = []
    for label, spec, M, seed in cases:
        sel = [None]  # the dispatch the closure passes, switched between the two timings
        w = _moe_setup(spec, seed, "tiled", M=M, dispatch=sel)
        big = w["M"] >= 512
        n, wu = (max(3, steps // 10), 2) if big else (steps, warmup)
        res = {}
        for mode, key in ((L.MXQ_DISPATCH_PER_BLOCK, "per_block_us"), (L.MXQ_DISPATCH_LAYER_AVERAGE, "layer_avg_us")):
            sel[0] = ops.Dispatch(mode)
            res[key] = _time_calls(w["run"], n, wu)[0]["median"]
        row = {"case": label, "M": w["M"], **res, "speedup": res["layer_avg_us"] / res["per_block_us"],
               "per_block_weight_gbs": w["bytes"] / (res["per_block_us"] * 1e-6) / 1e9}
        print(json.dumps(row), flush=True)
        rows.append(row)
        del w
        torch.cuda.empty_cache()
    return rows


SWEEP_SHAPES = {
    # (spec with the experts that receive rows, active experts)
    "gptoss_mxfp4": (dict(kind="fused_moe_mxfp4", H=2880, I=2880), 32),
    "deepseek_w8a8": (dict(kind="fused_moe_fp8", H=7168, I=2048, act_quant=True), 32),
    "w8a16_e8": (dict(kind="fused_moe_fp8", H=2048, I=1024, act_quant=False), 8),
}
SWEEP_M = (1, 2, 4, 8, 12, 16, 24, 32, 48, 64, 96, 128)


def bench_class_sweep(steps: int, warmup: int, shapes=None, ms=None):
    """Evidence for the per-block tile-class bounds: `E` experts each receive exactly m routed
    rows (top-1, so every block holds m rows), the fused MoE runs with every class forced in
    turn (0 = tiny-block kernel, 1..4 = 16/32/64/128-row tiles) and with the per-block default;
    one JSON line per (shape, m) with the median µs per call and the touched-weight GB/s of
    each."""
    from mxfp4_block_scaled_expert_amd import ops, synth
    from mxfp4_block_scaled_expert_amd import _lib as L
    rows = []
    for name in (shapes or SWEEP_SHAPES):
        base, E = SWEEP_SHAPES[name]
        for m in (ms or SWEEP_M):
            spec = dict(base, E=E, topk=1, counts=tuple([m] * E))
            sel = [None]
            w = _moe_setup(spec, 1100 + m, "tiled", dispatch=sel)
            res = {"shape": name, "m": m, "experts": E}
            for key, d in [("default", None)] + [(f"class{c}", ops.Dispatch(L.MXQ_DISPATCH_FORCED, c, 16))
                                                 for c in range(5)]:
                sel[0] = d
                us = _time_calls(w["run"], steps, warmup)[0]["median"]
                res[key + "_us"] = us
                res[key + "_gbs"] = w["bytes"] / (us * 1e-6) / 1e9
            best = min(range(5), key=lambda c: res[f"class{c}_us"])
            res["best_class"] = best
            res["default_over_best"] = res["default_us"] / res[f"class{best}_us"]
            print(json.dumps(res), flush=True)
            rows.append(res)
            del w
            torch.cuda.empty_cache()
    return rows


# ----------------------------------------------------------------------------- CPU oracle

def cpu_baseline(budget_s: float = 12.0):
    """The plain C++ oracle (loops, double accumulation, OpenMP over output rows on every host
    core) on a bounded sample of the headline workload: the first rows of the 2048 x 2048 x
    7168 block-FP8 linear with bf16 input (quantise + linear), sized from a short probe to take
    about `budget_s` seconds."""
    from mxfp4_block_scaled_expert_amd import synth
    from oracle import cref
    M, K, N = 2048, 2048, 7168
    d = synth.block_linear(M, N, K, seed=1002, device="cpu")
    xb = d["x"].view(torch.int16).numpy().view(np.uint16)
    w = d["w"].numpy()
    sw = d["sw"].numpy()
    probe = 16
    t0 = time.perf_counter()
    cref.block_fp8_linear_bf16(xb[:probe], w, sw, 128)
    per_row = (time.perf_counter() - t0) / probe
    rows = int(max(probe, min(M, budget_s / max(per_row, 1e-9))))
    # one call on the sampled rows; when the whole workload takes less than the budget, whole
    # calls are repeated until it is spent
    calls, dt = 0, 0.0
    while calls == 0 or (rows == M and dt < budget_s):
        t0 = time.perf_counter()
        cref.block_fp8_linear_bf16(xb[:rows], w, sw, 128)
        dt += time.perf_counter() - t0
        calls += 1
    return {"value": 2.0 * rows * N * K * calls / dt / 1e12, "unit": "TFLOP/s", "cores": cref.threads(),
            "kind": "oracle",
            "sample": f"C++ oracle (oracle/cpp/oracle.cpp), first {rows} of 2048 rows of the 2048x2048x7168 "
                      f"block-FP8 linear with bf16 input (quantise + linear), {calls} call(s), {dt:.1f} s"}


def calibrate_copy(steps: int = 10, mib: int = 256):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
    (run under rocprofv3 --pmc; every launch reads and writes exactly `mib` MiB)."""
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"calibration": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n, "launches": steps}


def main():
    a = _args()
    global SETTLE_S
    if a.settle is not None:
        SETTLE_S = a.settle
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "requested_gpus": a.gpus}), flush=True)
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    torch.cuda.set_device(0)
    from mxfp4_block_scaled_expert_amd import ops
    ops.init(0)

    if a.only == "copy":
        print(json.dumps(calibrate_copy()), flush=True)
        return
    if a.only == "ablation":
        bench_dispatch_ablation(a.steps, a.warmup)
        return
    if a.only == "classes":
        bench_class_sweep(a.steps, a.warmup, a.sweep_shape.split(",") if a.sweep_shape else None,
                          [int(v) for v in a.sweep_m.split(",")] if a.sweep_m else None)
        return
    if a.only == "decode":
        print(json.dumps(bench_moe("moe_mxfp4_gptoss_decode_m32", a.steps, a.warmup, 1004)), flush=True)
        return
    if a.only == "prefill":
        print(json.dumps(bench_moe("moe_block_fp8_w8a8_deepseek_prefill_m4096", a.steps, a.warmup, 1005)),
              flush=True)
        return
    if a.only == "mx":
        print(json.dumps(bench_mx(a.steps, a.warmup, "e2m1")), flush=True)
        print(json.dumps(bench_mx(a.steps, a.warmup, "e4m3")), flush=True)
        return
    if a.only == "small":
        print(json.dumps(bench_per_tensor(a.steps, a.warmup)), flush=True)
        print(json.dumps(bench_moe("moe_block_fp8_w8a16_e8_h2048_i1024", a.steps, a.warmup, 1003)), flush=True)
        return

    lin = bench_linear(a.steps, a.warmup)
    if a.only == "linear":
        print(json.dumps(lin), flush=True)
        return
    value = lin["flops"] / (lin["ms_per_step"] * 1e-3) / 1e12
    g_us = lin["gemm_us"]["mean"]
    achieved = lin["flops"] / (g_us * 1e-6) / 1e12
    traffic, traffic_note = stamped_traffic()
    roof = {
        "kernel": "gemm_w8a8_big_kernel (block-FP8 W8A8, 256x256 tiles, direct-to-LDS operands)",
        "bound": "mfma", "achieved": achieved, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": achieved / FP8_PEAK_TFLOPS, "traffic": traffic, "traffic_source": traffic_note,
        "alg_flops_per_launch": lin["flops"], "alg_bytes_per_launch": lin["gemm_alg_bytes"],
        "avg_launch_us": g_us, "launch_us": lin["gemm_us"],
    }
    secondary = {}
    if not a.no_secondary:
        secondary["per_tensor_w8a16_97x576x224"] = bench_per_tensor(a.steps, a.warmup)
        secondary["block_linear_decode_m16_k7168_n2048"] = bench_linear_small(max(10, a.steps), a.warmup, 16, 2048, 7168)
        secondary["block_linear_few_tiles_m128_k7168_n2048"] = bench_linear_small(max(10, a.steps), a.warmup, 128, 2048,
                                                                                    7168)
        secondary["w8a16_small_blocks_e8"] = bench_moe("moe_block_fp8_w8a16_e8_h2048_i1024", a.steps, a.warmup,
                                                       1003)
        torch.cuda.empty_cache()
        secondary["gptoss_mxfp4_decode_m32"] = bench_moe("moe_mxfp4_gptoss_decode_m32", max(10, a.steps),
                                                        a.warmup, 1004)
        torch.cuda.empty_cache()
        secondary["deepseek_w8a8_prefill_m4096"] = bench_moe("moe_block_fp8_w8a8_deepseek_prefill_m4096",
                                                            max(5, a.steps // 2), 2, 1005)
        torch.cuda.empty_cache()
        secondary["mla_bmm_128heads_t64"] = bench_mla_bmm(max(10, a.steps), a.warmup)
        torch.cuda.empty_cache()
        secondary["mx_linear_mxfp4_weights"] = bench_mx(a.steps, a.warmup, "e2m1")
        torch.cuda.empty_cache()
        secondary["mx_linear_mxfp8_weights"] = bench_mx(a.steps, a.warmup, "e4m3")
        torch.cuda.empty_cache()
    cpu = None if a.no_cpu_baseline else cpu_baseline()
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": lin["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": "block_w8a8_linear_2048x2048x7168 (1x128 act quant + 128x128 weight blocks)",
                   "M": lin["M"], "K": lin["K"], "N": lin["N"], "rotating_input_sets": lin["rotating_sets"]},
        "roofline": roof, "cpu_baseline": cpu,
        "detail": {"step_us": lin["step_us"], "quant_us": lin["quant_us"], "gemm_us": lin["gemm_us"],
                   "wall_ms_per_step": lin["wall_ms_per_step"], "settle_steps": lin["settle_steps"],
                   "settle_s": SETTLE_S},
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
