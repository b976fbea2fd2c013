"""Pins for the oracle per-token 1x128 group quantiser: closed-form invariants
and an independent restatement that uses torch's own e4m3 cast."""

import numpy as np
import torch

from oracle import codecs as C
from oracle.quant import per_token_group_quant_fp8, group_quant_f32


def _bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _random_x(M, K, seed, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    if spread:  # groups with very different magnitudes
        x *= np.exp2(rng.integers(-20, 20, size=(M, K // 128, 1))).repeat(128, axis=2).reshape(M, K)
    return _bf16(x)


def test_amax_element_maps_to_max_code_and_scale_is_amax_over_448():
    xb = _random_x(64, 1024, 1)
    q, s = per_token_group_quant_fp8(xb)
    x = C.bf16_to_f32(xb).reshape(64, 8, 128)
    amax = np.abs(x).max(axis=2)
    # s is the fp32 quotient amax / 448, bit for bit (torch division as the check)
    s_t = (torch.from_numpy(amax) / torch.tensor(448.0)).numpy()
    assert np.array_equal(s.view(np.uint32), s_t.view(np.uint32))
    qg = q.reshape(64, 8, 128)
    idx = np.abs(x).argmax(axis=2)
    top = np.take_along_axis(qg, idx[..., None], axis=2)[..., 0]
    sign = np.take_along_axis(x, idx[..., None], axis=2)[..., 0] < 0
    assert np.all(top == np.where(sign, 0xFE, 0x7E))


def test_constant_and_zero_groups():
    x = np.zeros((3, 256), np.float32)
    x[0, :128] = 3.5
    x[1, 128:] = -0.25
    x[2, :] = 0.0
    x[2, 5] = -0.0
    q, s = group_quant_f32(x)
    assert np.all(q[0, :128] == 0x7E) and s[0, 0] == np.float32(3.5) / np.float32(448)
    assert np.all(q[1, 128:] == 0xFE) and s[1, 1] == np.float32(0.25) / np.float32(448)
    eps_s = np.float32(1e-10) / np.float32(448)
    assert s[0, 1] == eps_s and s[2, 0] == eps_s and s[2, 1] == eps_s
    assert np.all(q[2, :5] == 0) and q[2, 5] == 0x80 and np.all(q[0, 128:] == 0)


def test_rounding_error_within_half_e4m3_ulp():
    xb = _random_x(32, 2048, 2)
    q, s = per_token_group_quant_fp8(xb)
    x = C.bf16_to_f32(xb).astype(np.float64)
    srep = np.repeat(s, 128, axis=1).astype(np.float64)
    y = x / srep
    dq = C.E4M3_TABLE[q]
    a = np.abs(y)
    # e4m3 spacing at |y|: 2^(floor(log2|y|) - 3) for normals, 2^-9 below 2^-6
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    ulp = np.exp2(e - 3)
    assert np.all(np.abs(dq - y) <= ulp / 2 * (1 + 1e-6))


def test_matches_torch_restatement_bit_exact():
    for seed, (M, K) in enumerate([(1, 128), (17, 512), (64, 2048), (5, 7168)]):
        xb = _random_x(M, K, 10 + seed, spread=(seed % 2 == 0))
        q, s = per_token_group_quant_fp8(xb)
        xt = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).float().view(M, K // 128, 128)
        amax = xt.abs().amax(dim=2)
        st = torch.clamp(amax, min=1e-10) / 448.0
        qt = (xt / st[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).view(M, K)
        assert np.array_equal(s.view(np.uint32), st.numpy().view(np.uint32))
        assert np.array_equal(q, qt.numpy())


def test_group_independence_and_row_independence():
    xb = _random_x(8, 512, 3)
    q, s = per_token_group_quant_fp8(xb)
    q1, s1 = per_token_group_quant_fp8(xb[3:4, 128:256])
    assert np.array_equal(q1, q[3:4, 128:256]) and np.array_equal(s1, s[3:4, 1:2])
