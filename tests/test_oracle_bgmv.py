"""Pins for the oracle's BGMV MoE-LoRA shrink and expand (CPU only).

BGMV page ("flashinfer.fused_moe.prepare_bgmv_moe"): signature, Parameters and the
description (each output accumulates its routes in fixed input order)."""
import numpy as np
import torch

import oracle as O


def _case(seed=0, T=6, H=24, r=8, N=16, nl=3, E=4, P=11):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H))
    A = g.standard_normal((nl, E, r, H))
    B = g.standard_normal((nl, E, N, r))
    tok = g.integers(0, T, P).astype(np.int32)
    ex = g.integers(0, E, P).astype(np.int32)
    li = g.integers(0, nl, T).astype(np.int32)
    w = g.random(P)
    return x, A, B, tok, ex, li, w


def test_brute_force_loops():
    x, A, B, tok, ex, li, w = _case()
    tok[3] = -1          # invalid token
    ex[5] = 9            # invalid expert
    li[int(tok[7])] = -1 if tok[7] != tok[0] else li[int(tok[7])]
    y, s = O.bgmv_moe(x, A, B, tok, ex, li, w)
    T, H = x.shape
    nl, E, r, _ = A.shape
    N = B.shape[2]
    for p in range(len(tok)):
        t, e = int(tok[p]), int(ex[p])
        valid = 0 <= t < T and 0 <= e < E and 0 <= li[t] < nl
        for j in range(r):
            ref = sum(x[t, h] * A[li[t], e, j, h] for h in range(H)) if valid else 0.0
            assert abs(s[p, j] - ref) < 1e-12 * (1 + abs(ref))
    for t in range(T):
        for c in range(N):
            ref = 0.0
            for p in range(len(tok)):
                e = int(ex[p])
                if tok[p] != t or not (0 <= e < E and 0 <= li[t] < nl):
                    continue
                ref += w[p] * sum(s[p, j] * B[li[t], e, c, j] for j in range(r))
            assert abs(y[t, c] - ref) < 1e-12 * (1 + abs(ref))
    assert np.all(s[3] == 0) and np.all(s[5] == 0)


def test_matches_torch_gathered_bmm_and_scatter():
    x, A, B, tok, ex, li, w = _case(seed=1, T=20, H=64, r=16, N=48, nl=4, E=8, P=50)
    y, s = O.bgmv_moe(x, A, B, tok, ex, li, w)
    X, At, Bt = torch.from_numpy(x), torch.from_numpy(A), torch.from_numpy(B)
    t, e = torch.from_numpy(tok.astype(np.int64)), torch.from_numpy(ex.astype(np.int64))
    l = torch.from_numpy(li.astype(np.int64))[t]
    S = torch.bmm(At[l, e], X[t][:, :, None])[:, :, 0]                 # [P, r]
    Z = torch.bmm(Bt[l, e], S[:, :, None])[:, :, 0]                     # [P, N]
    M = torch.zeros((x.shape[0], len(tok)), dtype=torch.float64)
    M[t, torch.arange(len(tok))] = torch.from_numpy(w)
    np.testing.assert_allclose(s, S.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, (M @ Z).numpy(), rtol=1e-11, atol=1e-11)


def test_invariants_order_empty_tokens_linearity_and_bf16_shrink():
    x, A, B, tok, ex, li, w = _case(seed=2, T=10, H=32, r=8, N=24, P=15)
    tok[tok == 4] = 5                                     # token 4 has no pair
    y, s = O.bgmv_moe(x, A, B, tok, ex, li, w)
    assert np.all(y[4] == 0)
    perm = np.random.default_rng(3).permutation(len(tok))
    y2, s2 = O.bgmv_moe(x, A, B, tok[perm], ex[perm], li, w[perm])
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(s2, s[perm])
    y3, _ = O.bgmv_moe(x, A, B, tok, ex, li, 2.5 * w)
    np.testing.assert_allclose(y3, 2.5 * y, rtol=1e-12, atol=1e-12)
    yb, sb = O.bgmv_moe(x, A, B, tok, ex, li, w, shrink_dtype="bf16")
    assert np.all(np.abs(sb - s) <= 2.0 ** -8 * np.abs(s))                # one bf16 rounding
    assert not np.array_equal(sb, s)
