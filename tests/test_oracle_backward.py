"""Pins for the oracle's layer and router backward (CPU only).

Grouped-GEMM page (operation table and Autograd section: dgrad / wgrad, zero
weight gradients for empty groups); SM90 fused-MoE page (forward formula, EP
shard); StepFun page (Renormalize routing, SwiGLUStep clamp limit).
Independent routes: torch autograd in float64 on a torch transcription of the
forward definition, and central finite differences of the oracle's own forward.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


def _case(seed=0, T=7, H=12, I=10, E=4, k=2, scale=1.0):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H)) * scale
    w1 = g.standard_normal((E, 2 * I, H)) / math.sqrt(H)
    w2 = g.standard_normal((E, H, I)) / math.sqrt(I)
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = g.random((T, k))
    w /= w.sum(1, keepdims=True)
    dout = g.standard_normal((T, H))
    return x, w1, w2, ids, w, dout


def _torch_grads(x, w1, w2, ids, w, dout, E, off, L, kind, limits):
    xt = torch.tensor(x, requires_grad=True)
    w1t = torch.tensor(w1[off:off + L], requires_grad=True)
    w2t = torch.tensor(w2[off:off + L], requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    I = w1.shape[1] // 2
    out = torch.zeros(x.shape, dtype=torch.float64)
    for t in range(x.shape[0]):
        for s in range(ids.shape[1]):
            e = int(ids[t, s]) - off
            if not 0 <= e < L:
                continue
            h = w1t[e] @ xt[t]
            u, g = h[:I], h[I:]
            if kind == "swiglu_step":
                lim = float(limits[e])
                u, g = torch.clamp(u, -lim, lim), torch.clamp(g, -lim, lim)
            out = out.index_add(0, torch.tensor([t]), (wt[t, s] * (w2t[e] @ (F.silu(g) * u)))[None])
    out.backward(torch.tensor(dout))
    return xt.grad.numpy(), w1t.grad.numpy(), w2t.grad.numpy(), wt.grad.numpy()


@pytest.mark.parametrize("kind", ["swiglu", "swiglu_step"])
@pytest.mark.parametrize("shard", [None, (1, 2)])
def test_backward_matches_torch_autograd(kind, shard):
    x, w1, w2, ids, w, dout = _case(seed=1, scale=3.0)   # scale 3: the clamp at 1.5 fires
    E = w1.shape[0]
    off, L = (0, E) if shard is None else shard
    limits = np.array([1.5, 2.0, 100.0, 0.7])[off:off + L]
    got = O.moe_backward(x, ids, w, w1[off:off + L], w2[off:off + L], dout, num_experts=E,
                         local_offset=off, activation_kind=kind, limits=limits)
    ref = _torch_grads(x, w1, w2, ids, w, dout, E, off, L, kind, limits)
    for gv, rv in zip(got, ref):
        np.testing.assert_allclose(gv, rv, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("kind", ["swiglu", "swiglu_step"])
def test_backward_central_differences(kind):
    x, w1, w2, ids, w, dout = _case(seed=2, T=5, H=6, I=4, E=3, k=2, scale=2.0)
    limits = np.array([1.2, 3.0, 0.9])
    kw = dict(num_experts=3, activation_kind=kind, limits=limits)

    def loss(x_, w1_, w2_, w_):
        return float(np.sum(dout * O.moe_forward(x_, ids, w_, w1_, w2_, **kw)))

    dx, dw1, dw2, dw = O.moe_backward(x, ids, w, w1, w2, dout, **kw)
    eps = 1e-6
    g = np.random.default_rng(3)
    for arr, grad, pos in ((x, dx, 0), (w1, dw1, 1), (w2, dw2, 2), (w, dw, 3)):
        for _ in range(12):
            idx = tuple(g.integers(0, n) for n in arr.shape)
            args = [x, w1, w2, w]
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args[pos] = plus
            lp = loss(*args)
            args[pos] = minus
            lm = loss(*args)
            # a clamp kink inside [v - eps, v + eps] would break the difference; no
            # pre-activation of these draws lies that close to a limit
            assert abs((lp - lm) / (2 * eps) - grad[idx]) < 1e-6 * (1 + abs(grad[idx]))


def test_activation_backward_clamp_boundary_and_torch():
    lim = 2.0
    u = np.array([-3.0, -2.0, -1.0, 0.0, 2.0, 2.5])
    g = np.array([0.5, -2.0, 2.0, 3.0, -0.5, 1.0])
    h = np.concatenate([u, g])[None]
    da = np.linspace(0.3, 1.8, 6)[None]
    got = O.activation_backward(h, da, "swiglu_step", lim)
    ut = torch.tensor(u, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    a = F.silu(torch.clamp(gt, -lim, lim)) * torch.clamp(ut, -lim, lim)
    a.backward(torch.tensor(da[0]))
    # torch's clamp passes the gradient at the limits themselves (inclusive)
    np.testing.assert_allclose(got[0, :6], ut.grad.numpy(), rtol=1e-14, atol=0)
    np.testing.assert_allclose(got[0, 6:], gt.grad.numpy(), rtol=1e-14, atol=0)
    assert got[0, 0] == 0 and got[0, 5] == 0 and got[0, 9] == 0   # clamped: no gradient
    got2 = O.activation_backward(h, da, "swiglu")
    ut.grad = None
    gt.grad = None
    (F.silu(gt) * ut).backward(torch.tensor(da[0]))
    np.testing.assert_allclose(got2[0], np.concatenate([ut.grad.numpy(), gt.grad.numpy()]), rtol=1e-14)


def test_backward_empty_expert_and_foreign_routes():
    x, w1, w2, ids, w, dout = _case(seed=4, T=6, E=4, k=2)
    ids[:, :] = np.array([0, 3])                    # experts 1 and 2 receive nothing
    dx, dw1, dw2, dw = O.moe_backward(x, ids, w, w1[:3], w2[:3], dout, num_experts=4)
    assert np.all(dw1[1] == 0) and np.all(dw2[2] == 0)
    assert np.all(dw[:, 1] == 0)                    # slot 1 routes to foreign expert 3
    assert np.any(dw1[0] != 0) and np.any(dx != 0)


def test_route_backward_matches_torch_autograd():
    g = np.random.default_rng(5)
    T, E, k = 9, 16, 4
    logits = g.standard_normal((T, E))
    ids, w = O.route(logits, k)
    dw = g.standard_normal((T, k))
    lt = torch.tensor(logits, requires_grad=True)
    sel = torch.gather(lt, 1, torch.tensor(ids, dtype=torch.int64))
    torch.softmax(sel, dim=1).backward(torch.tensor(dw))
    got = O.route_backward(ids, w, dw, E)
    np.testing.assert_allclose(got, lt.grad.numpy(), rtol=1e-10, atol=1e-14)
    assert np.all(got.sum(1) < 1e-12)                # softmax gradients sum to zero per token
