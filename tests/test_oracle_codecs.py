"""Pins for the oracle codecs: torch's own float8 / bfloat16 conversions (an
independent library implementation) and the format specifications' named
values (tests/golden/ocp_codec_points.json)."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import codecs as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_e4m3_table_matches_torch_decode():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mine = C.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan], mine[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(mine[~nan]))


def test_e4m3_named_values():
    g = _golden("ocp_codec_points.json")["e4m3"]
    for k, v in g.items():
        if k == "nan_codes":
            for c in v:
                assert np.isnan(C.E4M3_TABLE[int(c, 16)])
            continue
        got = C.E4M3_TABLE[int(k, 16)]
        assert got == v and np.signbit(got) == np.signbit(v), k
    assert np.nanmax(C.E4M3_TABLE) == C.E4M3_MAX == 448.0


def _torch_e4m3(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_all_bf16_values_in_range():
    # every bf16 bit pattern whose value lies in [-448, 448]
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = C.bf16_to_f32(pats)
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    v = v[keep]
    assert np.array_equal(C.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_midpoints_and_neighbours():
    pos = C.E4M3_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    vals = np.concatenate([mids, up, dn, pos.astype(np.float32)])
    vals = vals[np.abs(vals) <= 448]
    vals = np.concatenate([vals, -vals])
    mine = C.e4m3_encode(vals)
    assert np.array_equal(mine, _torch_e4m3(vals))
    # ties go to the even code
    tie_codes = C.e4m3_encode(mids)
    assert np.all(tie_codes % 2 == 0)


def test_e4m3_encode_random_fp32_bits():
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    assert v.size > 500_000
    assert np.array_equal(C.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_sign_of_zero_and_range_check():
    z = np.array([0.0, -0.0, -1e-30, 1e-30, -448.0, 448.0], dtype=np.float32)
    assert list(C.e4m3_encode(z)) == [0x00, 0x80, 0x80, 0x00, 0xFE, 0x7E]
    with pytest.raises(ValueError):
        C.e4m3_encode(np.array([448.5], np.float32))
    with pytest.raises(ValueError):
        C.e4m3_encode(np.array([np.nan], np.float32))


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties (low half == 0x8000) with both parities of the kept bit
    ties = (rng.integers(0, 2 ** 16, size=20000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    bits = np.concatenate([bits, ties])
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(C.f32_to_bf16(x), ref)
    # bf16 -> fp32 is exact: round trip of every bf16 pattern
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = C.bf16_to_f32(pats)
    ok = ~np.isnan(f)
    assert np.array_equal(C.f32_to_bf16(f)[ok], pats[ok])
    tref = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(f[ok], tref[ok])


def test_e2m1_table_named_values_and_structure():
    mags = _golden("ocp_codec_points.json")["e2m1_magnitudes"]
    assert list(C.E2M1_TABLE[:8]) == mags
    assert list(-C.E2M1_TABLE[8:]) == mags
    assert np.signbit(C.E2M1_TABLE[8])  # 0x8 is -0


def test_e2m1_unpack_order():
    # byte 0x21: low nibble 0x1 (0.5) is element 0, high nibble 0x2 (1.0) element 1
    packed = np.array([[0x21, 0xF7]], dtype=np.uint8)
    assert list(C.e2m1_decode_packed(packed)[0]) == [0.5, 1.0, 6.0, -6.0]


def test_e8m0_matches_torch_and_named_values():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    mine = C.e8m0_decode(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    g = _golden("ocp_codec_points.json")["e8m0"]
    for k in ("127", "128", "0", "254"):
        assert mine[int(k)] == g[k]
    assert np.isnan(mine[g["nan_code"]])
