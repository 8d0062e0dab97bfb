"""Pins for the oracle's MX codecs and the UE8M0 round-up requantization (CPU only).

W4A8 page ("Inputs": float8_e4m3fn activations with UE8M0 block-32 scale
codes, MXFP4 weights; intro: UE8M0 round-up requantization).
"""
import numpy as np
import pytest
import torch

import oracle as O


def test_e4m3_decode_exhaustive_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0


def test_minifloat_decoder_matches_torch_e5m2_finite_codes():
    # the generic decoder that the e2m1 instance uses also reproduces e5m2
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    finite = ((codes >> 2) & 0x1F) != 0x1F
    got = O.minifloat_decode(codes, 5, 2, 15)
    np.testing.assert_array_equal(got[finite], ref[finite])


def test_e2m1_decode_values():
    v = O.e2m1_decode(np.arange(16))
    np.testing.assert_array_equal(v[:8], [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    np.testing.assert_array_equal(v[8:], -v[:8])


def test_ue8m0_decode_exhaustive_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = O.ue8m0_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[:255], ref[:255])


def test_e4m3_encode_against_torch_cast():
    g = np.random.default_rng(0)
    grid = np.concatenate([np.linspace(-448, 448, 200001), g.uniform(-1, 1, 100000) * 2.0 ** -6,
                           g.uniform(-1, 1, 100000) * 2.0 ** -9])
    # exact midpoints between neighbouring codes (ties go to the even code)
    vals = O.e4m3_decode(np.arange(0, 126))
    grid = np.concatenate([grid, (vals[:-1] + vals[1:]) / 2, -(vals[:-1] + vals[1:]) / 2])
    # float32 inputs (the requantization decides on float32 values); torch's float64
    # cast goes through float32 first, which would double-round float64 inputs
    grid = grid.astype(np.float32)
    ref = torch.from_numpy(grid).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(grid.astype(np.float64))
    # +-0 may differ only in sign of zero
    same = (got == ref) | ((got & 0x7F) == 0) & ((ref & 0x7F) == 0)
    assert same.all(), grid[~same][:10]


def test_requant_invariants():
    g = np.random.default_rng(1)
    a = (g.standard_normal((64, 256)) * np.exp(g.uniform(-12, 12, (64, 1)))).astype(np.float32)
    a[3, 32:64] = 0.0
    vals, sc = O.requant_e4m3(a)
    assert sc.shape == (64, 8)
    amax = np.abs(a.astype(np.float64)).reshape(64, 8, 32).max(-1)
    nz = amax > 0
    scale = np.exp2(sc.astype(np.float64) - 127)
    r = amax[nz] / scale[nz]
    assert np.all(r <= 448.0) and np.all(r > 224.0)      # smallest power of two that fits
    assert sc[3, 1] == 0 and np.all(vals[3, 32:64] == 0)
    deq = O.mx_dequant(vals, sc)
    # e4m3 has 3 mantissa bits: error <= half an ulp, i.e. 2^-4 relative in the
    # normal range and 2^-10 * scale absolute in the subnormal range
    err = np.abs(deq - a)
    bound = np.maximum(np.abs(a) * 2.0 ** -4, np.repeat(scale, 32, axis=1) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))
    # re-quantising already-quantised data changes no value (a block whose maximum
    # rounded down to 224 * 2^e may re-encode one binade lower, to the same values)
    vals2, sc2 = O.requant_e4m3(deq.astype(np.float32))
    assert np.all((sc2 == sc) | (sc2 == sc - 1))
    np.testing.assert_array_equal(O.mx_dequant(vals2, sc2), deq)


def test_requant_exact_power_of_two_boundary():
    # amax exactly 448 * 2^e takes exponent e (not e+1); a hair above takes e+1
    a = np.zeros((2, 32), np.float32)
    a[0, 5] = 448.0 * 2.0 ** -3
    a[1, 5] = np.nextafter(np.float32(448.0 * 2.0 ** -3), np.float32(1e9))
    _, sc = O.requant_e4m3(a)
    assert sc[0, 0] == 127 - 3 and sc[1, 0] == 127 - 2


def test_fp4_packing_golden():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_packing.json")) as f:
        fx = json.load(f)
    b = np.array(fx["bytes"], dtype=np.uint8)
    np.testing.assert_array_equal(O.unpack_e2m1(b), fx["codes"])
    np.testing.assert_array_equal(O.e2m1_decode(O.unpack_e2m1(b)), fx["values"])
    # one 32-wide block: the fixture bytes followed by zeros
    row = np.zeros(16, np.uint8)
    row[:4] = b
    v = O.mx_dequant_fp4(row[None], np.array([[fx["scale_code"]]], np.uint8))[0]
    np.testing.assert_array_equal(v[:8], fx["scaled_values"])
    assert np.all(v[8:] == 0)


def test_mx_dequant_fp8_scales_each_block():
    codes = np.full((1, 64), 0x38, np.uint8)            # e4m3 1.0 everywhere
    v = O.mx_dequant_fp8(codes, np.array([[127 + 3, 127 - 2]], np.uint8))
    np.testing.assert_array_equal(v[0, :32], 8.0)
    np.testing.assert_array_equal(v[0, 32:], 0.25)
