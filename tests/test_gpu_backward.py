"""GPU parity: the layer backward (training forward + moe_ffn_backward) and the
routing backward against the oracle's chain rule (grouped-GEMM page, Autograd
section; SM90 fused-MoE page formula; StepFun page routing and SwiGLUStep).

The oracle takes the bf16 inputs widened to float64 and keeps everything exact.
The library hands dy, dh, the dx rows (and the forward's act and y) over in bf16,
each rounding off by at most u = 2^-8 relative, and accumulates in float32. The
bar is a first-order bound per gradient element derived from those roundings
(`_grad_bounds`): a rounded operand contributes u times the sum of absolute
summands it enters, and the error that the rounding of dy puts into
da = dy @ w2 reaches dh through the activation's derivative. Each gradient must
lie within its bound element by element, and within relative L2 1e-2 overall.
(A CPU emulation of exactly these roundings stays below 0.6 of the bound.)
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_softmax_amd as M
import moe_synth as S
import oracle as O
from parity import check_grads as _check, grad_bounds as _grad_bounds, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _fwd_bwd(c, dout, grad_dtype=torch.bfloat16):
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    lim = None if c.limits is None else torch.from_numpy(c.limits).to(DEV)
    x, w1, w2 = c.x.to(DEV), c.w1.to(DEV), c.w2.to(DEV)
    out, saved = M.moe_ffn_forward_train(x, ids, w, w1, w2, c.num_experts, c.num_local,
                                         c.local_offset, c.activation, lim)
    grads = M.moe_ffn_backward(dout.to(DEV), saved, x, ids, w, w1, w2, c.num_experts, c.num_local,
                               c.local_offset, c.activation, lim, grad_dtype=grad_dtype)
    return out, grads, ids, w


def _oracle(c, ids, w, dout):
    return O.moe_backward(S.bf16_to_f32(c.x), ids.cpu().numpy(), w.cpu().numpy().astype(np.float64),
                          S.bf16_to_f32(c.w1), S.bf16_to_f32(c.w2), S.bf16_to_f32(dout),
                          num_experts=c.num_experts, local_offset=c.local_offset,
                          activation_kind=c.activation, limits=c.limits)


@pytest.mark.parametrize("activation", ["swiglu", "swiglu_step"])
def test_backward_small_layer(activation):
    """T=300, H=512, I=768: several row blocks per expert and column tiles (3 of 256
    for dgrad, 6 x 2 for the FC1 wgrad), ragged groups."""
    c = S.moe_case("bwd_small", 300, 512, 768, 8, 2, activation=activation,
                   limit_range=(1.0, 3.0), x_scale=2.0, seed=11)
    dout = S.upstream_grad(11, c.T, c.H)
    out, grads, ids, w = _fwd_bwd(c, dout)
    ref = _oracle(c, ids, w, dout)
    _check(grads, ref, _grad_bounds(c, ids, w, dout), f"bwd {activation}")
    # the training forward computes the same layer as the inference forward
    lim = None if c.limits is None else torch.from_numpy(c.limits).to(DEV)
    out_inf = M.moe_ffn_forward(c.x.to(DEV), ids, w, c.w1.to(DEV), c.w2.to(DEV), c.num_experts,
                                c.num_local, c.local_offset, c.activation, lim)
    assert torch.equal(out, out_inf)


def test_backward_clamp_masks_fire():
    """SwiGLUStep with limits well inside the pre-activation range: a large share of
    the gradient is cut by the clamp masks, and the result still matches."""
    c = S.moe_case("bwd_clamp", 128, 256, 256, 4, 2, activation="swiglu_step",
                   limit_range=(0.3, 0.6), x_scale=4.0, seed=12)
    dout = S.upstream_grad(12, c.T, c.H)
    _, grads, ids, w = _fwd_bwd(c, dout)
    ref = _oracle(c, ids, w, dout)
    _check(grads, ref, _grad_bounds(c, ids, w, dout), "bwd clamp")


def test_backward_expert_shard_fp32_grads_and_empty_experts():
    """256 experts, 32 local from id 64, top-8 (foreign routes give no gradient), float32
    weight gradients; experts of the shard that receive no route get exactly zero."""
    c = S.moe_case("bwd_shard", 64, 256, 128, 256, 8, num_local=32, local_offset=64,
                   activation="swiglu_step", limit_range=(5.0, 9.0), seed=13)
    dout = S.upstream_grad(13, c.T, c.H)
    _, grads, ids, w = _fwd_bwd(c, dout, grad_dtype=torch.float32)
    ref = _oracle(c, ids, w, dout)
    _check(grads, ref, _grad_bounds(c, ids, w, dout), "bwd shard")
    loc = ids.cpu().numpy() - 64
    empty = [e for e in range(32) if not np.any(loc == e)]
    assert empty, "the case should leave some local experts without routes"
    for e in empty:
        assert torch.count_nonzero(grads[1][e]) == 0 and torch.count_nonzero(grads[2][e]) == 0
    foreign = (loc < 0) | (loc >= 32)
    assert np.all(to_np(grads[3])[foreign] == 0)


def test_backward_is_bitwise_reproducible_and_zero_tokens():
    c = S.moe_case("bwd_rep", 200, 256, 256, 8, 2, seed=14)
    dout = S.upstream_grad(14, c.T, c.H)
    _, g1, _, _ = _fwd_bwd(c, dout)
    _, g2, _, _ = _fwd_bwd(c, dout)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    # T = 0: no rows, weight gradients exactly zero
    x0 = c.x[:0].to(DEV)
    ids0 = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    w0 = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    w1, w2 = c.w1.to(DEV), c.w2.to(DEV)
    _, saved = M.moe_ffn_forward_train(x0, ids0, w0, w1, w2, 8)
    dx, dw1, dw2, _ = M.moe_ffn_backward(torch.empty((0, c.H), dtype=torch.bfloat16, device=DEV),
                                         saved, x0, ids0, w0, w1, w2, 8)
    assert dx.shape == (0, c.H)
    assert torch.count_nonzero(dw1) == 0 and torch.count_nonzero(dw2) == 0


def test_autograd_wrapper_matches_direct_calls():
    c = S.moe_case("bwd_autograd", 96, 256, 256, 8, 2, seed=15)
    dout = S.upstream_grad(15, c.T, c.H).to(DEV)
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    x = c.x.to(DEV).requires_grad_(True)
    wt = w.clone().requires_grad_(True)
    w1 = c.w1.to(DEV).requires_grad_(True)
    w2 = c.w2.to(DEV).requires_grad_(True)
    out = M.MoEFunction.apply(x, wt, w1, w2, ids, c.num_experts)
    out.backward(dout)
    _, grads, _, _ = _fwd_bwd(c, dout)
    for got, want in zip((x.grad, w1.grad, w2.grad, wt.grad), (grads[0], grads[1], grads[2], grads[3])):
        assert torch.equal(got, want)


@pytest.mark.parametrize("T,E,k", [(300, 8, 2), (97, 64, 8), (33, 256, 8), (5, 1024, 16)])
def test_route_backward(T, E, k):
    g = np.random.default_rng(T + E)
    logits = torch.from_numpy(g.standard_normal((T, E)).astype(np.float32)).to(DEV)
    ids, w = M.moe_route(logits, k)
    dw = torch.from_numpy(g.standard_normal((T, k)).astype(np.float32)).to(DEV)
    got = M.moe_route_backward(ids, w, dw, E)
    ref = O.route_backward(ids.cpu().numpy(), w.cpu().numpy(), dw.cpu().numpy(), E)
    np.testing.assert_allclose(to_np(got), ref, rtol=2e-5, atol=2e-6)
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, ids.cpu().numpy().astype(np.int64), True, axis=1)
    assert np.all(to_np(got)[~sel] == 0)


def test_backward_mixtral_full_shape():
    """T=4096, H=4096, I=14336, 8 experts, top-2: every gradient against the oracle."""
    c = S.mixtral_moe(seed=3)
    dout = S.upstream_grad(3, c.T, c.H)
    _, grads, ids, w = _fwd_bwd(c, dout)
    torch.cuda.synchronize()
    ref = _oracle(c, ids, w, dout)
    _check(grads, ref, _grad_bounds(c, ids, w, dout), "bwd mixtral")
