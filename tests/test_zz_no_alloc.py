"""GPU: moe_ffn_forward_noalloc (the forward with the library's fixed scratch memory,
for callers that cannot allocate) against moe_ffn_forward on the same inputs, and
against the oracle: two calls in a row, the second on a smaller input, per format.

The two entry points run the same launches over the same workspace layout, so the
outputs must be bitwise equal; the oracle bar is that of the other layer tests.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_softmax_amd as M
import moe_synth as S
import oracle as O
from parity import assert_close_bf16, mx_dequant_table

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16_pair(c):
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    lim = None if c.limits is None else torch.from_numpy(c.limits).to(DEV)
    x, w1, w2 = c.x.to(DEV), c.w1.to(DEV), c.w2.to(DEV)
    kw = dict(num_local_experts=c.num_local, local_expert_offset=c.local_offset,
              activation=c.activation, clamp_limit=lim)
    out = torch.full((c.T, c.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    got = M.moe_ffn_forward_noalloc(x, ids, w, w1, w2, c.num_experts, out=out, **kw)
    want = M.moe_ffn_forward(x, ids, w, w1, w2, c.num_experts, **kw)
    torch.cuda.synchronize()
    return got, want, ids, w


def test_noalloc_bf16_two_calls_second_smaller():
    cases = [S.moe_case("na_big", 512, 512, 1024, 64, 8, num_local=32, local_offset=16,
                        activation="swiglu_step", limit_range=(1.0, 3.0), x_scale=2.0, seed=71),
             S.moe_case("na_small", 37, 512, 1024, 64, 8, num_local=32, local_offset=16,
                        activation="swiglu_step", limit_range=(1.0, 3.0), x_scale=2.0, seed=72)]
    assert M.moe_ffn_workspace_size(512, 512, 1024, 64, 8, 32, 16) <= M.NOALLOC_SCRATCH_BYTES
    for c in cases:
        got, want, ids, w = _bf16_pair(c)
        assert torch.equal(got, want), c.name
        ref = O.moe_forward(S.bf16_to_f32(c.x), ids.cpu().numpy(), w.cpu().numpy().astype(np.float64),
                            S.bf16_to_f32(c.w1), S.bf16_to_f32(c.w2), num_experts=c.num_experts,
                            local_offset=c.local_offset, activation_kind=c.activation,
                            limits=c.limits)
        assert_close_bf16(got, ref, what=c.name)


def test_noalloc_rows_mode_and_mxfp4_two_calls():
    # finalize "none": y rows and e2p, on the bf16 path
    c = S.moe_case("na_rows", 200, 256, 512, 8, 2, seed=73)
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    x, w1, w2 = c.x.to(DEV), c.w1.to(DEV), c.w2.to(DEV)
    y1, e1 = M.moe_ffn_forward_noalloc(x, ids, w, w1, w2, 8, finalize="none")
    y2, e2 = M.moe_ffn_forward(x, ids, w, w1, w2, 8, finalize="none")
    torch.cuda.synchronize()
    n = int((e2 >= 0).sum().item())
    assert torch.equal(e1, e2) and torch.equal(y1[:n], y2[:n])
    # MXFP4 weights: a 64-token call, then a 5-token one
    full = S.w4a8_moe(seed=74, T=64, H=512, I=256, E=16, top_k=4)
    d = {k_: torch.from_numpy(np.ascontiguousarray(getattr(full, k_))).to(DEV)
         for k_ in ("x", "x_sf", "w1", "w1_sf", "w2", "w2_sf")}
    w1d = mx_dequant_table("mxfp4", full.w1, full.w1_sf)
    w2d = mx_dequant_table("mxfp4", full.w2, full.w2_sf)
    for T in (64, 5):
        ids, w = M.moe_route(torch.from_numpy(full.logits[:T]).to(DEV), full.top_k)
        x, x_sf = d["x"][:T].contiguous(), d["x_sf"][:T].contiguous()
        got = M.moe_ffn_forward_noalloc(x, ids, w, d["w1"], d["w2"], full.num_experts,
                                        weight_format="mxfp4", x_sf=x_sf, w1_sf=d["w1_sf"],
                                        w2_sf=d["w2_sf"])
        want = M.moe_ffn_forward_mx(x, x_sf, ids, w, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"],
                                    full.num_experts)
        torch.cuda.synchronize()
        assert torch.equal(got, want), T
        ref = O.moe_forward(O.mx_dequant_fp8(full.x[:T], full.x_sf[:T]), ids.cpu().numpy(),
                            w.cpu().numpy().astype(np.float64), w1d, w2d,
                            num_experts=full.num_experts, requant=True)
        assert_close_bf16(got, ref, 8e-2, 3e-2, what=f"MXFP4 noalloc T={T}")


def test_noalloc_too_large_is_refused():
    c = S.moe_case("na_huge", 4096, 4096, 14336, 8, 2, seed=75, with_weights=False)
    assert M.moe_ffn_workspace_size(4096, 4096, 14336, 8, 2) > M.NOALLOC_SCRATCH_BYTES
    x = c.x.to(DEV)
    ids = torch.zeros((4096, 2), dtype=torch.int32, device=DEV)
    w = torch.zeros((4096, 2), dtype=torch.float32, device=DEV)
    w1 = torch.empty((8, 2 * 14336, 4096), dtype=torch.bfloat16, device=DEV)
    w2 = torch.empty((8, 4096, 14336), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.MoeError) as ex:
        M.moe_ffn_forward_noalloc(x, ids, w, w1, w2, 8)
    assert ex.value.status == 8
