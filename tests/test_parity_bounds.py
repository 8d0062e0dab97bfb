"""CPU checks of the derived error bars the GPU tests use (tests/parity.py).

A bound that is too tight fails correct kernels; one that is too loose hides bugs.
Both directions are checked against a CPU emulation of the library's number
handling (float32 products and sums, bf16 hand-off of act and y, float32 or bf16
combine), on the oracle's exact result:
* the emulation stays within parity.forward_bound element by element;
* plausible mistakes of a kernel (the clamp limit of another expert, the clamp on
  one half dropped, the up and gate halves swapped, one route left out) do not.
"""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle as O
from parity import forward_bound


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _emulate(c, ids, w, fused=False, mistake=None):
    """The layer as the GPU computes it, in float32 with bf16 hand-offs."""
    x = S.bf16_to_f32(c.x)
    w1, w2 = S.bf16_to_f32(c.w1), S.bf16_to_f32(c.w2)
    T, k = ids.shape
    L, I = c.num_local, c.I
    loc = O.local_expert(ids, c.num_experts, L, c.local_offset).reshape(T, k)
    ys = np.zeros((T, k, c.H), np.float32)
    for e in range(L):
        tt, ss = np.nonzero(loc == e)
        if tt.size == 0:
            continue
        h = (x[tt] @ w1[e].T).astype(np.float32)
        u, g = h[:, :I], h[:, I:]
        if mistake == "swap_halves":
            u, g = g, u
        if c.activation == "swiglu_step":
            lim = np.float32(c.limits[(e + 1) % L] if mistake == "other_limit" else c.limits[e])
            if mistake != "no_up_clamp":
                u = np.clip(u, -lim, lim)
            g = np.clip(g, -lim, lim)
        a = _bf16(g / (np.float32(1) + np.exp(-g)) * u)
        ys[tt, ss] = _bf16(a @ w2[e].T)
    wf = w.astype(np.float32)
    if mistake == "drop_route":
        wf = wf.copy()
        t0 = int(np.nonzero(loc[:, 1] >= 0)[0][0])
        wf[t0, 1] = 0
    if fused:
        out = np.zeros((T, c.H), np.float32)
        for s in range(k):
            add = _bf16(np.where(loc[:, s:s + 1] >= 0, wf[:, s:s + 1] * ys[:, s], 0))
            out = _bf16(out + add)
        return out
    out = np.zeros((T, c.H), np.float32)
    for s in range(k):
        out += np.where(loc[:, s:s + 1] >= 0, wf[:, s:s + 1] * ys[:, s], np.float32(0))
    return _bf16(out)


def _case(activation, x_scale):
    return S.moe_case("bound", 96, 128, 64, 16, 4, num_local=8, local_offset=4,
                      activation=activation, limit_range=(5.0, 9.0), x_scale=x_scale, seed=5)


def _ref_and_bound(c, fused=False):
    ids, w = O.route(c.logits, c.top_k)
    x, w1, w2 = S.bf16_to_f32(c.x), S.bf16_to_f32(c.w1), S.bf16_to_f32(c.w2)
    kw = dict(num_experts=c.num_experts, local_offset=c.local_offset,
              activation_kind=c.activation, limits=c.limits)
    ref = O.moe_forward(x, ids, w, w1, w2, **kw)
    return ids, w, ref, forward_bound(x, ids, w, w1, w2, fused=fused, **kw)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("activation,x_scale", [("swiglu", 1.0), ("swiglu_step", 1.0),
                                                ("swiglu_step", 8.0)])
def test_emulated_library_rounding_is_within_the_bound(activation, x_scale, fused):
    c = _case(activation, x_scale)
    ids, w, ref, bound = _ref_and_bound(c, fused)
    got = _emulate(c, ids, w, fused)
    ratio = np.abs(got - ref) / (bound + 1e-30)
    assert ratio.max() <= 1.0, ratio.max()
    if x_scale > 1:   # the clamp is exercised on both halves
        h = S.bf16_to_f32(c.x) @ S.bf16_to_f32(c.w1)[0].T
        assert np.mean(np.abs(h) > c.limits[0]) > 0.2


@pytest.mark.parametrize("mistake", ["other_limit", "no_up_clamp", "swap_halves", "drop_route"])
def test_planted_mistakes_exceed_the_bound(mistake):
    c = _case("swiglu_step", 8.0)
    ids, w, ref, bound = _ref_and_bound(c)
    got = _emulate(c, ids, w, mistake=mistake)
    assert np.any(np.abs(got - ref) > bound)
