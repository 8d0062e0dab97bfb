"""GPU: prepared launches under graph capture (StepFun page, "Prepared launches":
no allocation and no host synchronisation in a launch; grouped-GEMM page,
"Prepared launches": new offsets may be written between launches).

Each test captures library calls into one hipGraph (torch.cuda.CUDAGraph on
ROCm), then replays it several times with new inputs written into the captured
buffers, running the eager computation and synchronising between replays, and
checks every replay bitwise against the eager result and against the oracle (to
the same bar as the eager tests of each path). The library clears its counters and
outputs with kernels, never with memset nodes.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_softmax_amd as M
import moe_synth as S
import oracle as O
from parity import (assert_close_bf16, check_grads, grad_bounds, mx_dequant_table, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _capture(fn):
    """Warm up fn on a side stream, then capture it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_bf16_layer_graph_replays_with_new_inputs():
    cases = [S.moe_case("g", 300, 512, 768, 8, 2, activation="swiglu_step", limit_range=(2.0, 4.0),
                        seed=s) for s in (21, 22, 23)]
    c0 = cases[0]
    E, k, H = c0.num_experts, c0.top_k, c0.H
    logits = torch.from_numpy(c0.logits).to(DEV)
    x = c0.x.to(DEV)
    w1, w2 = c0.w1.to(DEV), c0.w2.to(DEV)
    lim = torch.from_numpy(c0.limits).to(DEV)
    ids = torch.empty((c0.T, k), dtype=torch.int32, device=DEV)
    wts = torch.empty((c0.T, k), dtype=torch.float32, device=DEV)
    out = torch.empty((c0.T, H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(M.moe_ffn_workspace_size(c0.T, H, c0.I, E, k, activation="swiglu_step"),
                     dtype=torch.uint8, device=DEV)

    def step():
        M.moe_route(logits, k, ids, wts)
        M.moe_ffn_forward(x, ids, wts, w1, w2, E, activation="swiglu_step", clamp_limit=lim, out=out,
                          workspace=ws)

    g = _capture(step)
    for c in cases[1:] + cases[:1]:
        logits.copy_(torch.from_numpy(c.logits))
        x.copy_(c.x)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ids_e, w_e = M.moe_route(torch.from_numpy(c.logits).to(DEV), k)
        ref = M.moe_ffn_forward(c.x.to(DEV), ids_e, w_e, w1, w2, E, activation="swiglu_step",
                                clamp_limit=lim)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        oref = O.moe_forward(S.bf16_to_f32(c.x), ids_e.cpu().numpy(),
                             w_e.cpu().numpy().astype(np.float64), S.bf16_to_f32(c0.w1),
                             S.bf16_to_f32(c0.w2), num_experts=E, activation_kind="swiglu_step",
                             limits=c0.limits)
        assert_close_bf16(got, oref, what=f"graph replay seed {c.meta['seed']}")


def test_w4a8_decode_graph_replays():
    full = S.w4a8_moe(seed=31, T=64, H=512, I=256, E=16, top_k=4)
    d = {k_: torch.from_numpy(np.ascontiguousarray(getattr(full, k_))).to(DEV)
         for k_ in ("x", "x_sf", "w1", "w1_sf", "w2", "w2_sf")}
    T = 4
    logits = torch.from_numpy(full.logits[:T]).to(DEV)
    x, x_sf = d["x"][:T].clone(), d["x_sf"][:T].clone()
    ids = torch.empty((T, full.top_k), dtype=torch.int32, device=DEV)
    wts = torch.empty((T, full.top_k), dtype=torch.float32, device=DEV)
    out = torch.empty((T, full.H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(M.moe_ffn_workspace_size(T, full.H, full.I, full.num_experts, full.top_k,
                                              weight_format="mxfp4"), dtype=torch.uint8, device=DEV)

    def step():
        M.moe_route(logits, full.top_k, ids, wts)
        M.moe_ffn_forward_mx(x, x_sf, ids, wts, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"],
                             full.num_experts, out=out, workspace=ws)

    g = _capture(step)
    w1d = mx_dequant_table("mxfp4", full.w1, full.w1_sf)
    w2d = mx_dequant_table("mxfp4", full.w2, full.w2_sf)
    for t0 in (8, 20, 40, 0):
        sl = slice(t0, t0 + T)
        logits.copy_(torch.from_numpy(full.logits[sl]))
        x.copy_(d["x"][sl])
        x_sf.copy_(d["x_sf"][sl])
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ids_e, w_e = M.moe_route(torch.from_numpy(full.logits[sl]).to(DEV), full.top_k)
        ref = M.moe_ffn_forward_mx(d["x"][sl].contiguous(), d["x_sf"][sl].contiguous(), ids_e, w_e,
                                   d["w1"], d["w1_sf"], d["w2"], d["w2_sf"], full.num_experts)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        oref = O.moe_forward(O.mx_dequant_fp8(full.x[sl], full.x_sf[sl]), ids_e.cpu().numpy(),
                             w_e.cpu().numpy().astype(np.float64), w1d, w2d,
                             num_experts=full.num_experts, requant=True)
        assert_close_bf16(got, oref, 8e-2, 3e-2, what=f"MXFP4 graph replay tokens {t0}..")


def test_grouped_gemm_graph_with_offsets_rewritten():
    """One captured grouped GEMM replayed over three different group-size vectors that
    share the row capacity; the offsets are device data written between replays."""
    E, M_, K, N = 8, 1024, 256, 512
    g_ = np.random.default_rng(41)
    x = torch.from_numpy(g_.standard_normal((M_, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    w = torch.from_numpy(g_.standard_normal((E, N, K)).astype(np.float32) / 16).to(torch.bfloat16).to(DEV)
    offs = torch.empty(E, dtype=torch.int32, device=DEV)
    y = torch.zeros((M_, N), dtype=torch.bfloat16, device=DEV)
    sizes = [S.dirichlet_group_sizes(E, M_, 0.3, seed=s) for s in (1, 2, 3)]
    offs.copy_(torch.from_numpy(np.cumsum(sizes[0]).astype(np.int32)))
    g = _capture(lambda: M.grouped_gemm_fwd(x, w, offs, out=y))
    for sz in sizes[1:] + sizes[:1]:
        offs.copy_(torch.from_numpy(np.cumsum(sz).astype(np.int32)))
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        ref = M.grouped_gemm_fwd(x, w, offs.clone())
        torch.cuda.synchronize()
        n = int(np.sum(sz))
        assert torch.equal(got[:n], ref[:n])
        oref = O.grouped_gemm_fwd(S.bf16_to_f32(x)[:n], S.bf16_to_f32(w), np.cumsum(sz))
        assert_close_bf16(got[:n], oref, what="grouped fwd graph replay")


def test_training_step_graph_replays():
    c = S.moe_case("gt", 256, 256, 256, 8, 2, seed=51)
    E, k = c.num_experts, c.top_k
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), k)
    x, w1, w2 = c.x.to(DEV), c.w1.to(DEV), c.w2.to(DEV)
    dout = S.upstream_grad(51, c.T, c.H).to(DEV)
    out = torch.empty_like(x)
    _, saved = M.moe_ffn_forward_train(x, ids, w, w1, w2, E, out=out)
    grads = {}

    def step():
        M.moe_ffn_forward_train(x, ids, w, w1, w2, E, out=out, saved=saved)
        grads["g"] = M.moe_ffn_backward(dout, saved, x, ids, w, w1, w2, E)

    g = _capture(step)
    captured = grads["g"]
    for seed in (52, 53):
        dout.copy_(S.upstream_grad(seed, c.T, c.H))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in captured]
        _, sv = M.moe_ffn_forward_train(x, ids, w, w1, w2, E)
        ref = M.moe_ffn_backward(dout.clone(), sv, x, ids, w, w1, w2, E)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        oref = O.moe_backward(S.bf16_to_f32(c.x), ids.cpu().numpy(),
                              w.cpu().numpy().astype(np.float64), S.bf16_to_f32(c.w1),
                              S.bf16_to_f32(c.w2), S.bf16_to_f32(dout), num_experts=E)
        check_grads(got, oref, grad_bounds(c, ids, w, dout), f"graph training replay {seed}")
