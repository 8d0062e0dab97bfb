"""GPU parity: ragged bf16 grouped GEMM fwd / dgrad / wgrad against the oracle.

Integer-valued operands make every fp32 partial sum exact, so those cases are
bit-exact at any size; real-valued cases meet the bf16 tolerance."""
import numpy as np
import pytest
import torch

import mixture_experts_expert_softmax_amd as M
import moe_synth as S
import oracle as O
from parity import assert_close_bf16, bf16_round, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALL_SIZES = [
    [300, 0, 1, 257, 64, 513],       # spans several 256-row tiles, empty and 1-row groups
    [1], [0, 0, 5], [256, 256], [17, 90, 255, 1],
    # 150 groups, many empty: the tile dealing scans 64 groups at a time (3 passes)
    [int(v) for v in np.random.default_rng(7).integers(0, 12, 150) * (np.arange(150) % 3 > 0)],
]


def _to_dev(case):
    return (case.x.to(DEV), case.g.to(DEV), case.w.to(DEV),
            torch.from_numpy(case.offs).to(DEV))


def _f(t):
    return S.bf16_to_f32(t)


@pytest.mark.parametrize("sizes", SMALL_SIZES)
@pytest.mark.parametrize("K,N", [(128, 256), (96, 320), (512, 64)])
def test_grouped_gemm_small_real(sizes, K, N):
    c = S.grouped_gemm_case(seed=len(sizes) + K, sizes=np.array(sizes), K=K, N=N)
    x, g, w, offs = _to_dev(c)
    M_ = int(c.offs[-1])
    y = M.grouped_gemm_fwd(x, w, offs)
    assert_close_bf16(y, O.grouped_gemm_fwd(_f(c.x), _f(c.w), c.offs), what="fwd")
    dx = M.grouped_gemm_dgrad(g, w, offs)
    assert_close_bf16(dx, O.grouped_gemm_dgrad(_f(c.g), _f(c.w), c.offs), what="dgrad")
    ref_dw = O.grouped_gemm_wgrad(_f(c.g), _f(c.x), c.offs)
    dw32 = M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.float32)
    np.testing.assert_allclose(to_np(dw32), ref_dw, rtol=1e-4, atol=1e-4 * max(1, np.sqrt(M_)))
    dwb = M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.bfloat16)
    _check_wgrad_bf16(to_np(dwb), ref_dw)
    for e, m in enumerate(sizes):
        if m == 0:
            assert torch.all(dw32[e] == 0) and torch.all(dwb[e] == 0)


def _check_wgrad_bf16(got, ref):
    for e in range(ref.shape[0]):
        if np.all(ref[e] == 0):
            assert np.all(got[e] == 0)
            continue
        assert_close_bf16(got[e], ref[e], what=f"wgrad bf16 expert {e}")


def test_grouped_gemm_integer_exact_small():
    c = S.grouped_gemm_case(seed=3, sizes=np.array([300, 0, 1, 257, 64, 513]), K=192, N=288,
                            integer_valued=True)
    x, g, w, offs = _to_dev(c)
    # every fp32 partial sum is an exact integer; the bf16 outputs are its single RNE rounding
    np.testing.assert_array_equal(to_np(M.grouped_gemm_fwd(x, w, offs)),
                                  bf16_round(O.grouped_gemm_fwd(_f(c.x), _f(c.w), c.offs)))
    np.testing.assert_array_equal(to_np(M.grouped_gemm_dgrad(g, w, offs)),
                                  bf16_round(O.grouped_gemm_dgrad(_f(c.g), _f(c.w), c.offs)))
    ref_dw = O.grouped_gemm_wgrad(_f(c.g), _f(c.x), c.offs)
    np.testing.assert_array_equal(to_np(M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.float32)), ref_dw)
    np.testing.assert_array_equal(to_np(M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.bfloat16)),
                                  bf16_round(ref_dw))


def _sweep_shapes(n=10, seed=11):
    """Seeded random shapes: N and K multiples of 32 at every residue modulo the
    256-wide tiles, ragged groups (empty ones, single rows, counts that are not
    multiples of 32, and more than one 256-row tile)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 9))
        K = 32 * int(rng.integers(1, 25))
        N = 32 * int(rng.integers(1, 25))
        sizes = rng.choice([0, 1, int(rng.integers(2, 40)), int(rng.integers(40, 300)),
                            int(rng.integers(300, 700))], size=E)
        out.append((i, K, N, [int(v) for v in sizes]))
    return out


@pytest.mark.parametrize("i,K,N,sizes", _sweep_shapes())
def test_grouped_gemm_shape_sweep_integer_exact(i, K, N, sizes):
    """fwd / dgrad / wgrad on integer-valued operands are exact at any shape, so the
    tile edges (rows, columns and contraction past a 256 or 32 boundary, empty and
    1-row groups) must match the oracle bit for bit."""
    c = S.grouped_gemm_case(seed=100 + i, sizes=np.array(sizes), K=K, N=N, integer_valued=True)
    x, g, w, offs = _to_dev(c)
    np.testing.assert_array_equal(to_np(M.grouped_gemm_fwd(x, w, offs)),
                                  bf16_round(O.grouped_gemm_fwd(_f(c.x), _f(c.w), c.offs)))
    np.testing.assert_array_equal(to_np(M.grouped_gemm_dgrad(g, w, offs)),
                                  bf16_round(O.grouped_gemm_dgrad(_f(c.g), _f(c.w), c.offs)))
    ref_dw = O.grouped_gemm_wgrad(_f(c.g), _f(c.x), c.offs)
    np.testing.assert_array_equal(to_np(M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.float32)), ref_dw)
    np.testing.assert_array_equal(to_np(M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.bfloat16)),
                                  bf16_round(ref_dw))


@pytest.fixture(scope="module")
def full_int():
    return S.grouped_gemm_case(seed=0, integer_valued=True)


def _split_ws():
    return torch.empty(M.lib().moe_gemm_split_workspace_size(), dtype=torch.uint8, device=DEV)


def test_grouped_gemm_full_size_integer_exact(full_int):
    """E=16, sum_m=8192, K=2048, N=4096 with Dirichlet sizes: integer inputs are exact,
    with or without the split workspace (the dgrad's 328 tiles leave a last round of 72
    that is cut along N)."""
    c = full_int
    x, g, w, offs = _to_dev(c)
    ws = _split_ws()
    ref_y = bf16_round(O.grouped_gemm_fwd(_f(c.x), _f(c.w), c.offs))
    ref_dx = bf16_round(O.grouped_gemm_dgrad(_f(c.g), _f(c.w), c.offs))
    np.testing.assert_array_equal(to_np(M.grouped_gemm_fwd(x, w, offs)), ref_y)
    np.testing.assert_array_equal(to_np(M.grouped_gemm_fwd(x, w, offs, workspace=ws)), ref_y)
    np.testing.assert_array_equal(to_np(M.grouped_gemm_dgrad(g, w, offs)), ref_dx)
    np.testing.assert_array_equal(to_np(M.grouped_gemm_dgrad(g, w, offs, workspace=ws)), ref_dx)
    ref_dw = O.grouped_gemm_wgrad(_f(c.g), _f(c.x), c.offs)
    np.testing.assert_array_equal(to_np(M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.float32)), ref_dw)
    np.testing.assert_array_equal(to_np(M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.bfloat16)),
                                  bf16_round(ref_dw))


def test_grouped_gemm_full_size_real():
    """The real-valued cfg at full size: every output element of fwd and dgrad (with and
    without the split workspace) and of both wgrad dtypes against the oracle."""
    c = S.grouped_gemm_case(seed=0)
    x, g, w, offs = _to_dev(c)
    ws = _split_ws()
    xs, gs, wsf = _f(c.x), _f(c.g), _f(c.w)
    ref_y = O.grouped_gemm_fwd(xs, wsf, c.offs)
    ref_dx = O.grouped_gemm_dgrad(gs, wsf, c.offs)
    for kw in ({}, {"workspace": ws}):
        assert_close_bf16(M.grouped_gemm_fwd(x, w, offs, **kw), ref_y, what=f"fwd {list(kw)}")
        assert_close_bf16(M.grouped_gemm_dgrad(g, w, offs, **kw), ref_dx, what=f"dgrad {list(kw)}")
    ref_dw = O.grouped_gemm_wgrad(gs, xs, c.offs)
    dw32 = to_np(M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.float32))
    dwb = to_np(M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.bfloat16))
    for e in range(c.E):
        m = int(c.sizes[e])
        if m == 1:   # a 1-row product is exact in fp32
            np.testing.assert_array_equal(dw32[e], ref_dw[e])
        np.testing.assert_allclose(dw32[e], ref_dw[e], rtol=1e-4, atol=1e-3)
    _check_wgrad_bf16(dwb, ref_dw)


def test_grouped_gemm_replay_bitwise_and_offsets_rewritten():
    c = S.grouped_gemm_case(seed=5, sizes=np.array([700, 3, 0, 1333]), K=256, N=512)
    x, g, w, offs = _to_dev(c)
    y1 = M.grouped_gemm_fwd(x, w, offs)
    y2 = M.grouped_gemm_fwd(x, w, offs)
    assert torch.equal(y1, y2)
    d1 = M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.float32)
    d2 = M.grouped_gemm_wgrad(g, x, offs, out_dtype=torch.float32)
    assert torch.equal(d1, d2)
    # new offsets written into the same device tensor are read by the next launch
    new = np.array([1, 1000, 1001, 2036], dtype=np.int32)
    offs.copy_(torch.from_numpy(new))
    y3 = M.grouped_gemm_fwd(x, w, offs)
    assert_close_bf16(y3, O.grouped_gemm_fwd(_f(c.x), _f(c.w), new), what="rewritten offs")


def test_grouped_gemm_indptr_convention():
    c = S.grouped_gemm_case(seed=6, sizes=np.array([40, 0, 300]), K=64, N=128)
    x, g, w, offs = _to_dev(c)
    indptr = torch.cat([torch.zeros(1, dtype=torch.int32, device=DEV), offs])
    assert torch.equal(M.grouped_gemm_fwd(x, w, offs), M.grouped_gemm_fwd(x, w, indptr))
    assert torch.equal(M.grouped_gemm_wgrad(g, x, offs), M.grouped_gemm_wgrad(g, x, indptr, E=3,
                                                                              offs_kind="indptr"))


def test_grouped_gemm_empty_rows():
    w = torch.randn(3, 64, 32, device=DEV).to(torch.bfloat16)
    x = torch.empty((0, 32), dtype=torch.bfloat16, device=DEV)
    g = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    offs = torch.zeros(3, dtype=torch.int32, device=DEV)
    assert M.grouped_gemm_fwd(x, w, offs).shape == (0, 64)
    dw = torch.full((3, 64, 32), 7.0, device=DEV)
    M.grouped_gemm_wgrad(g, x, offs, out=dw)
    assert torch.all(dw == 0)


def test_fc2_short_tiles_cut_along_k_integer_exact():
    """32 groups of 256 rows and a last group of 40 rows at N = 2048: 264 tiles of
    256 x 256, so on a 256-CU device the last round is the last group's 8 short tiles,
    each cut along K into parts whose fp32 partials the last part sums. A tile of at
    most 64 rows runs a quarter of the MFMAs (32 rows per wave); on integer-valued
    operands the result is exact, with or without the cut."""
    sizes = np.array([256] * 32 + [40])
    K, N = 1024, 2048
    c = S.grouped_gemm_case(seed=21, sizes=sizes, K=K, N=N, integer_valued=True)
    act, w2 = c.x.to(DEV), c.w.to(DEV)
    offs = torch.from_numpy(c.offs).to(DEV)
    M_ = int(sizes.sum())
    y_cut = M.moe_fc2(act, w2, offs, M_, 1, len(sizes))
    y_whole = M.moe_fc2(act, w2, offs, M_, 1, len(sizes), split=False)
    torch.cuda.synchronize()
    assert torch.equal(y_cut, y_whole)
    got = to_np(y_cut)
    x64, w64 = _f(c.x), _f(c.w)
    last = slice(M_ - 40, M_)
    np.testing.assert_array_equal(got[last], bf16_round(O.grouped_gemm_fwd(x64[last], w64[-1:], [40])))
    np.testing.assert_array_equal(got[:256], bf16_round(O.grouped_gemm_fwd(x64[:256], w64[:1], [256])))
