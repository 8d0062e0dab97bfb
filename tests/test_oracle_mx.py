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


# --- fp8 per-tensor family (StepFun page, intro: fp8 per-tensor weights) ----------
def _torch_pt_codes(a32, scale):
    """Independent route: torch float32 reciprocal and product, clamp, float8 cast."""
    t = torch.from_numpy(np.asarray(a32, np.float32))
    r = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32)
    y = (t * r).clamp(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("scale", [0.5, 3.0, 0.0357, 1.7e-3])
def test_per_tensor_requant_matches_torch_float32_route(scale):
    g = np.random.default_rng(11)
    a = (g.standard_normal(200000) * np.exp(g.uniform(-10, 9, 200000))).astype(np.float32)
    vals, codes = O.requant_e4m3_per_tensor(a, scale)
    ref = _torch_pt_codes(a, scale)
    same = (codes == ref) | (((codes & 0x7F) == 0) & ((ref & 0x7F) == 0))
    assert same.all(), a[~same][:8]
    np.testing.assert_array_equal(
        vals, torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy() * float(np.float32(scale)))


def test_per_tensor_requant_saturates_and_keeps_sign():
    s = 0.25
    a = np.array([1e30, -1e30, 448 * s, -448 * s, 464 * s, 0.0, -0.0], np.float32)
    vals, codes = O.requant_e4m3_per_tensor(a, s)
    assert list(codes[:5]) == [0x7E, 0xFE, 0x7E, 0xFE, 0x7E]          # +-448, never NaN
    np.testing.assert_array_equal(vals[:2], [448 * s, -448 * s])
    assert np.all(vals[5:] == 0)


def test_per_tensor_requant_decides_on_the_float32_reciprocal():
    # a = 7 * 0.048828125 is exact in float32, and a / 7 = 0.048828125 is the tie
    # between the e4m3 values 0.046875 (even mantissa) and 0.05078125; the float32
    # reciprocal of 7 is rounded up, so the float32 product lands just above the tie
    # and the code rounds up, where an exact division would round down
    a = np.array([0.341796875], np.float32)
    assert float(a[0]) / 7.0 == 0.048828125
    assert float(np.float32(a[0] * (np.float32(1.0) / np.float32(7.0)))) > 0.048828125
    _, codes = O.requant_e4m3_per_tensor(a, 7.0)
    assert O.e4m3_decode(codes)[0] == 0.05078125
    assert _torch_pt_codes(a, 7.0)[0] == codes[0]


def test_fp8_dequant_per_expert_broadcast():
    codes = np.full((3, 2, 4), 0x38, np.uint8)                 # e4m3 1.0
    v = O.fp8_dequant(codes, np.array([1.0, 2.0, 0.5], np.float32))
    np.testing.assert_array_equal(v[:, 0, 0], [1.0, 2.0, 0.5])
    assert np.all(v == v[:, :1, :1])
    np.testing.assert_array_equal(O.fp8_dequant(np.array([0xB8, 0x7E], np.uint8), 0.5), [-0.5, 224.0])


def test_moe_forward_fp8_per_tensor_matches_torch_pipeline():
    """The forward with the per-tensor requantization against a torch pipeline that
    decodes with torch's float8 type and re-encodes with torch's cast."""
    import math
    g = np.random.default_rng(12)
    T, H, I, E, k = 6, 32, 16, 3, 2
    xq = torch.from_numpy(g.standard_normal((T, H)).astype(np.float32) * 3).to(torch.float8_e4m3fn)
    w1q = torch.from_numpy((g.standard_normal((E, 2 * I, H)) / math.sqrt(H)).astype(np.float32) * 64).to(
        torch.float8_e4m3fn)
    w2q = torch.from_numpy((g.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32) * 64).to(
        torch.float8_e4m3fn)
    xs = np.float32(0.5)
    w1s = np.array([1 / 64, 1 / 32, 3 / 256], np.float32)
    w2s = np.array([1 / 64, 1 / 128, 5 / 256], np.float32)
    act_s = 0.03
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = g.random((T, k))
    got = O.moe_forward(O.fp8_dequant(xq.view(torch.uint8).numpy(), xs), ids, w,
                        O.fp8_dequant(w1q.view(torch.uint8).numpy(), w1s),
                        O.fp8_dequant(w2q.view(torch.uint8).numpy(), w2s), num_experts=E,
                        act_scale=act_s)
    ref = torch.zeros((T, H), dtype=torch.float64)
    xd = xq.double() * float(xs)
    for t in range(T):
        for s in range(k):
            e = int(ids[t, s])
            h = xd[t] @ (w1q[e].double() * float(w1s[e])).T
            a = torch.nn.functional.silu(h[I:]) * h[:I]
            aq = torch.from_numpy(_torch_pt_codes(a.float().numpy(), act_s)).view(torch.float8_e4m3fn)
            y = (aq.double() * float(np.float32(act_s))) @ (w2q[e].double() * float(w2s[e])).T
            ref[t] += w[t, s] * y
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_table_dequant_helper_equals_oracle():
    """The GPU tests decode full expert banks through parity.mx_dequant_table; it must
    give exactly the oracle's values (NaN codes aside, which the inputs never hold)."""
    from parity import mx_dequant_table
    g = np.random.default_rng(7)
    packed = g.integers(0, 256, size=(64, 96), dtype=np.uint8)
    codes8 = g.integers(0, 256, size=(64, 192), dtype=np.uint8)
    codes8[(codes8 & 0x7F) == 0x7F] = 0
    sc = g.integers(100, 160, size=(64, 6), dtype=np.uint8)
    np.testing.assert_array_equal(mx_dequant_table("mxfp4", packed, sc), O.mx_dequant_fp4(packed, sc))
    np.testing.assert_array_equal(mx_dequant_table("mxfp8", codes8, sc), O.mx_dequant_fp8(codes8, sc))
