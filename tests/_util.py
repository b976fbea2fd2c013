"""Test helpers: moving tensors between torch and the oracle's numpy bit
patterns, and the parity assertions used by the GPU tests."""

import numpy as np
import torch

# bf16 outputs must agree with the oracle's bf16 result within these bounds
ATOL = 1e-2
RTOL = 1e-2


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 numpy bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return t.detach().contiguous().cpu().numpy()


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().float().numpy()


def bits_to_float(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def assert_bf16_close(got_bits: np.ndarray, want_bits: np.ndarray, atol=ATOL, rtol=RTOL, what=""):
    g = bits_to_float(got_bits)
    w = bits_to_float(want_bits)
    assert g.shape == w.shape, (g.shape, w.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - w)
    bound = atol + rtol * np.abs(w)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements outside atol={atol} rtol={rtol}; "
            f"first {idx.tolist()} got {g[bad][:5]} want {w[bad][:5]}")


def assert_bf16_close_requant(got_bits, want_bits, what="", frac=0.02, wide=5.0):
    """Bar for paths that re-quantise an intermediate (the W8A8 fused MoE).

    The 1x128 re-quantisation of ic1 turns last-bit differences of the stage-1
    sums (the FP8 matrix cores do not accumulate a 128-term block exactly) into
    occasional different e4m3 codes or group scales, which move single outputs
    by up to a few percent.  So: at most ``frac`` of the elements may leave the
    atol = rtol = 1e-2 band, none may leave ``wide`` times that band, and the
    mean error stays below 1e-2 of the output's rms (a systematic error fails).
    """
    g = bits_to_float(got_bits).astype(np.float64)
    w = bits_to_float(want_bits).astype(np.float64)
    assert g.shape == w.shape and np.all(np.isfinite(g)), what
    err = np.abs(g - w)
    band = ATOL + RTOL * np.abs(w)
    out = err > band
    assert out.mean() <= frac, f"{what}: {out.mean():.4%} of elements outside the 1e-2 band"
    worst = err > wide * band
    assert not worst.any(), f"{what}: {int(worst.sum())} elements beyond {wide}x the band, max err {err.max()}"
    rms = np.sqrt(np.mean(w * w)) + 1e-30
    assert err.mean() <= 1e-2 * rms, f"{what}: mean error {err.mean()} vs rms {rms}"


def gpu():
    return torch.device("cuda", 0)
