"""Pins for the oracle's grouped GEMMs, FFN forward and finalize (CPU only).

Grouped GEMM: grouped-GEMM page, operation table. FFN: SM90 fused-MoE page,
formula, and the StepFun page's SwiGLUStep clamp. Finalize: SM90 fused-MoE
page, use_fused_finalize=False path.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


def _case(seed, sizes, K, N, integer=False):
    g = np.random.default_rng(seed)
    M = int(np.sum(sizes))
    E = len(sizes)
    if integer:
        x = g.integers(-3, 4, size=(M, K)).astype(np.float64)
        gg = g.integers(-3, 4, size=(M, N)).astype(np.float64)
        w = g.integers(-3, 4, size=(E, N, K)).astype(np.float64)
    else:
        x = g.standard_normal((M, K))
        gg = g.standard_normal((M, N))
        w = g.standard_normal((E, N, K))
    return x, gg, w, np.cumsum(sizes).astype(np.int32)


# ----------------------------------------------------------------- grouped GEMM
def test_grouped_gemm_brute_force_loops():
    sizes = [2, 0, 3, 1]
    x, gg, w, offs = _case(0, sizes, K=5, N=3, integer=True)
    y = O.grouped_gemm_fwd(x, w, offs)
    dx = O.grouped_gemm_dgrad(gg, w, offs)
    dw = O.grouped_gemm_wgrad(gg, x, offs)
    start = 0
    for e, m in enumerate(sizes):
        for r in range(start, start + m):
            for n in range(3):
                assert y[r, n] == sum(x[r, c] * w[e, n, c] for c in range(5))
            for c in range(5):
                assert dx[r, c] == sum(gg[r, n] * w[e, n, c] for n in range(3))
        for n in range(3):
            for c in range(5):
                assert dw[e, n, c] == sum(gg[r, n] * x[r, c] for r in range(start, start + m))
        start += m
    assert np.all(dw[1] == 0.0)


def test_grouped_gemm_adjoint_identities():
    # <fwd(X,W), G> = sum_e <W[e], wgrad(G,X)[e]> = <dgrad(G,W), X>: a transposed
    # operand or a swapped index in any of the three breaks these equalities
    sizes = [5, 0, 1, 9, 3]
    x, gg, w, offs = _case(1, sizes, K=7, N=6)
    y = O.grouped_gemm_fwd(x, w, offs)
    dx = O.grouped_gemm_dgrad(gg, w, offs)
    dw = O.grouped_gemm_wgrad(gg, x, offs)
    a = np.sum(y * gg)
    b = np.sum(w * dw)
    c = np.sum(dx * x)
    assert abs(a - b) < 1e-10 * (1 + abs(a)) and abs(a - c) < 1e-10 * (1 + abs(a))


def test_grouped_gemm_is_block_diagonal_dense_product():
    sizes = [4, 1, 0, 6]
    x, gg, w, offs = _case(2, sizes, K=8, N=5)
    full = torch.from_numpy(x) @ torch.from_numpy(w.reshape(-1, 8)).T  # [M, E*N]
    ref = np.zeros((x.shape[0], 5))
    start = 0
    for e, m in enumerate(sizes):
        ref[start:start + m] = full[start:start + m, e * 5:(e + 1) * 5].numpy()
        start += m
    np.testing.assert_allclose(O.grouped_gemm_fwd(x, w, offs), ref, rtol=1e-13, atol=1e-13)


def test_grouped_gemm_rows_past_last_offset_untouched_and_empty_wgrad_zero():
    x, gg, w, _ = _case(3, [3, 3], K=4, N=4)
    offs = np.array([2, 2], dtype=np.int32)  # second group empty, rows 2..5 outside
    y = O.grouped_gemm_fwd(x, w, offs)
    assert np.all(y[2:] == 0)
    dw = O.grouped_gemm_wgrad(gg, x, offs)
    assert np.all(dw[1] == 0)


# ---------------------------------------------------------------------- FFN
def test_silu_against_torch_and_odd_identity():
    z = np.linspace(-60, 60, 2401)
    np.testing.assert_allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(O.silu(z) - O.silu(-z), z, rtol=1e-13, atol=1e-13)
    assert O.silu(0.0) == 0.0
    assert O.silu(-1000.0) == 0.0 and O.silu(1000.0) == 1000.0


def _tiny_ffn_inputs(seed, T=3, H=4, I=2, E=4, k=2):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H))
    w1 = g.standard_normal((E, 2 * I, H))
    w2 = g.standard_normal((E, H, I))
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = g.random((T, k))
    w /= w.sum(1, keepdims=True)
    return x, w1, w2, ids, w


@pytest.mark.parametrize("kind", ["swiglu", "swiglu_step"])
def test_moe_forward_brute_force_per_token(kind):
    x, w1, w2, ids, w = _tiny_ffn_inputs(4)
    x = x * 3.0  # let the clamp at limit 1.5 fire
    T, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    limits = np.array([1.5, 2.0, 100.0, 0.5])
    out = O.moe_forward(x, ids, w, w1, w2, num_experts=E, activation_kind=kind, limits=limits)
    for t in range(T):
        for hcol in range(H):
            acc = 0.0
            for s in range(ids.shape[1]):
                e = int(ids[t, s])
                lim = limits[e]
                val = 0.0
                for j in range(I):
                    up = sum(x[t, c] * w1[e, j, c] for c in range(H))
                    gate = sum(x[t, c] * w1[e, I + j, c] for c in range(H))
                    if kind == "swiglu_step":
                        up = min(max(up, -lim), lim)
                        gate = min(max(gate, -lim), lim)
                    a = gate / (1.0 + math.exp(-gate)) * up
                    val += a * w2[e, hcol, j]
                acc += w[t, s] * val
            assert abs(out[t, hcol] - acc) < 1e-12 * (1 + abs(acc))


def test_moe_forward_dense_special_case_is_torch_swiglu_mlp():
    g = np.random.default_rng(5)
    T, H, I = 16, 32, 24
    x = g.standard_normal((T, H))
    w1 = g.standard_normal((1, 2 * I, H)) / math.sqrt(H)
    w2 = g.standard_normal((1, H, I)) / math.sqrt(I)
    ids = np.zeros((T, 1), dtype=np.int32)
    out = O.moe_forward(x, ids, np.ones((T, 1)), w1, w2, num_experts=1)
    xt = torch.from_numpy(x)
    up_w, gate_w = torch.from_numpy(w1[0, :I]), torch.from_numpy(w1[0, I:])  # [up | gate] bank
    ref = (F.silu(xt @ gate_w.T) * (xt @ up_w.T)) @ torch.from_numpy(w2[0]).T
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_swiglu_step_reductions():
    g = np.random.default_rng(6)
    h = g.standard_normal((50, 64)) * 10
    # infinite limit is plain SwiGLU, bit for bit
    np.testing.assert_array_equal(O.activation(h, "swiglu_step", math.inf), O.activation(h, "swiglu"))
    # every pre-activation beyond +-L: a = silu(+-L) * (+-L)
    L = 3.0
    hs = np.sign(h) * (np.abs(h) + L)
    a = O.activation(hs, "swiglu_step", L)
    up_sign, gate_sign = np.sign(hs[:, :32]), np.sign(hs[:, 32:])
    expect = (gate_sign * L) / (1 + np.exp(-gate_sign * L)) * (up_sign * L)
    np.testing.assert_allclose(a, expect, rtol=1e-15)


def test_moe_forward_shards_sum_to_unsharded_and_foreign_is_zero():
    x, w1, w2, ids, w = _tiny_ffn_inputs(7, T=20, H=8, I=4, E=6, k=3)
    full = O.moe_forward(x, ids, w, w1, w2, num_experts=6)
    parts = []
    for off, L in [(0, 2), (2, 3), (5, 1)]:
        parts.append(O.moe_forward(x, ids, w, w1[off:off + L], w2[off:off + L], num_experts=6,
                                   local_offset=off))
    np.testing.assert_allclose(sum(parts), full, rtol=1e-12, atol=1e-12)
    # a shard no route reaches gives exact zeros
    ids_far = np.full_like(ids, 5)
    z = O.moe_forward(x, ids_far, w, w1[:2], w2[:2], num_experts=6, local_offset=0)
    assert np.all(z == 0.0)


def test_permuted_pipeline_reaches_the_definition():
    """sort -> gather -> grouped FC1 -> activation -> grouped FC2 -> finalize, built from
    the oracle's own steps, equals the per-token definition of the forward."""
    x, w1, w2, ids, w = _tiny_ffn_inputs(8, T=40, H=16, I=8, E=7, k=3)
    off, L, E = 2, 4, 7
    srt = O.sort_routes(ids, E, L, off)
    xp = x[srt["p2e"] // 3]
    h = O.grouped_gemm_fwd(xp, w1[off:off + L], srt["offs"])
    a = O.activation(h, "swiglu")
    y = O.grouped_gemm_fwd(a, w2[off:off + L], srt["offs"])
    out = O.finalize(y, srt["e2p"], w)
    ref = O.moe_forward(x, ids, w, w1[off:off + L], w2[off:off + L], num_experts=E, local_offset=off)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------- finalize
def test_finalize_one_hot_and_brute_force():
    g = np.random.default_rng(9)
    T, k, H, n = 6, 3, 5, 10
    y = g.standard_normal((n, H))
    e2p = np.array([0, -1, 4, 3, 2, -1, -1, -1, -1, 9, 1, 5, 6, 7, 8, -1, -1, -1][: T * k], dtype=np.int32)
    w = g.random((T, k))
    out = O.finalize(y, e2p, w)
    for t in range(T):
        ref = np.zeros(H)
        for s in range(k):
            p = e2p[t * k + s]
            if p >= 0:
                ref = ref + w[t, s] * y[p]
        np.testing.assert_allclose(out[t], ref, rtol=1e-15, atol=1e-15)
    onehot = np.zeros((T, k))
    onehot[:, 0] = 1.0
    o1 = O.finalize(y, e2p, onehot)
    for t in range(T):
        p = e2p[t * k]
        np.testing.assert_array_equal(o1[t], y[p] if p >= 0 else 0.0)
