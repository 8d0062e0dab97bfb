"""GPU: the deterministic paths give the same bits whatever the launch grid and the
tile dealing (SM90 fused-MoE page, Parameters: the non-fused finalize combines in a
fixed order; BGMV page, order_remap: a remapped dispatch is bitwise identical to the
identity one; grouped-GEMM page, intro: no atomics).

No knob changes a kernel's grid directly; the grid and the dealing of tiles to
workgroups and XCDs follow from the problem size. Computing a part of a problem on
its own (a slice of the tokens, one group of a grouped product) therefore runs the
same elements under a different grid, on other workgroups and XCDs, and must give
exactly the rows of the whole problem's result.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_softmax_amd as M
import moe_synth as S
import oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_finalize_same_bits_for_any_token_slice():
    g = np.random.default_rng(61)
    T, k, H = 5000, 8, 1024
    ids = g.integers(0, 64, size=(T, k)).astype(np.int32)
    srt = O.sort_routes(ids, 64, 32, 16)
    y = S.to_bf16(g.standard_normal((max(srt["n_local"], 1), H), dtype=np.float32)).to(DEV)
    w = torch.from_numpy(g.random((T, k)).astype(np.float32)).to(DEV)
    e2p = torch.from_numpy(srt["e2p"]).to(DEV)
    whole = M.moe_finalize(y, e2p, w)
    for t0, t1 in [(0, 1), (1, 4097), (2999, 5000), (123, 130)]:
        part = M.moe_finalize(y, e2p[t0 * k:t1 * k].contiguous(), w[t0:t1].contiguous())
        assert torch.equal(part, whole[t0:t1]), (t0, t1)


@pytest.fixture(scope="module")
def grouped():
    E, K, N = 12, 512, 768
    sizes = S.dirichlet_group_sizes(E, 3000, 0.3, seed=62)
    g = np.random.default_rng(62)
    x = S.to_bf16(g.standard_normal((3000, K), dtype=np.float32)).to(DEV)
    gr = S.to_bf16(g.standard_normal((3000, N), dtype=np.float32)).to(DEV)
    w = S.to_bf16(g.standard_normal((E, N, K), dtype=np.float32) / np.sqrt(K)).to(DEV)
    ends = np.cumsum(sizes).astype(np.int32)
    return sizes, ends, x, gr, w


def _groups(sizes, ends):
    for e, (n, f) in enumerate(zip(sizes.tolist(), ends.tolist())):
        yield e, f - n, f


def test_grouped_fwd_and_dgrad_same_bits_per_group(grouped):
    sizes, ends, x, gr, w = grouped
    offs = torch.from_numpy(ends).to(DEV)
    y = M.grouped_gemm_fwd(x, w, offs)
    dx = M.grouped_gemm_dgrad(gr, w, offs)
    for e, s, f in _groups(sizes, ends):
        if f == s:
            continue
        one = torch.tensor([f - s], dtype=torch.int32, device=DEV)
        ye = M.grouped_gemm_fwd(x[s:f].contiguous(), w[e:e + 1].contiguous(), one)
        de = M.grouped_gemm_dgrad(gr[s:f].contiguous(), w[e:e + 1].contiguous(), one)
        assert torch.equal(ye, y[s:f]), e
        assert torch.equal(de, dx[s:f]), e


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_grouped_wgrad_same_bits_per_group(grouped, out_dtype):
    sizes, ends, x, gr, w = grouped
    offs = torch.from_numpy(ends).to(DEV)
    dw = M.grouped_gemm_wgrad(gr, x, offs, out_dtype=out_dtype)
    for e, s, f in _groups(sizes, ends):
        if f == s:
            assert torch.count_nonzero(dw[e]) == 0
            continue
        one = torch.tensor([f - s], dtype=torch.int32, device=DEV)
        de = M.grouped_gemm_wgrad(gr[s:f].contiguous(), x[s:f].contiguous(), one,
                                  out_dtype=out_dtype)
        assert torch.equal(de[0], dw[e]), e
