"""GPU: the per-bucket tile tuner of the layer's GEMM stages (SM90 fused-MoE page,
Parameters: profile the legal tiles per token bucket, cache the winner; tile_size
follows the rows per expert). Whatever family wins -- or is recorded by hand with
moe_tune_set -- the layer must match the oracle, and clearing the table restores the
built-in rule bit for bit."""
import numpy as np
import pytest
import torch

import mixture_experts_expert_softmax_amd as M
import moe_synth as S
import oracle as O
from parity import assert_close_bf16, bf16_round, to_np
from test_gpu_mx import MX_MAX_ABS, MX_REL, _dev, _fwd, _oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("wfmt,T", [("mxfp4", 24), ("mxfp8", 200), ("fp8", 48)])
def test_tuned_choice_keeps_parity_and_clear_restores(wfmt, T):
    c = S.w4a8_moe(seed=61, T=T, H=512, I=512, E=8, top_k=2, wfmt=wfmt)
    d = _dev(c)
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    M.moe_tune_clear()
    before = _fwd(c, d, ids, w, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"])
    pt = wfmt == "fp8"
    choice = M.moe_tune(d["x"], ids, w, d["w1"], d["w2"], c.num_experts, x_sf=d["x_sf"],
                        w1_sf=d["w1_sf"], w2_sf=d["w2_sf"], act_scale=d["act_scale"] if pt else None)
    assert all(ch in (0, 1) for ch in choice)
    tuned = _fwd(c, d, ids, w, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"])
    assert_close_bf16(tuned, _oracle(c, ids, w), MX_MAX_ABS, MX_REL, what=f"tuned {wfmt} {choice}")
    M.moe_tune_clear()
    after = _fwd(c, d, ids, w, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"])
    torch.cuda.synchronize()
    assert torch.equal(before, after)


MX_FAMILY_CASES = [
    # (T, H, I, E, k, L, off): ragged experts of about 175 and 75 rows, and a local
    # shard
    (700, 512, 384, 8, 2, 8, 0),
    (300, 768, 256, 16, 4, 6, 5),
]


@pytest.mark.parametrize("wfmt", ["mxfp4", "mxfp8", "fp8"])
@pytest.mark.parametrize("T,H,I,E,k,L,off", MX_FAMILY_CASES)
def test_mx_tile_families_match_oracle(T, H, I, E, k, L, off, wfmt):
    """Both fp8-activation stages recorded to each tile family in turn -- the 256-row
    tile (0; its tiles multiply only the 32-row blocks that hold rows) and the
    streaming tile (1, where the shape allows it) -- against the oracle, with ragged
    experts over several tiles, a local shard and the clamped activation."""
    c = S.w4a8_moe(seed=T + I, T=T, H=H, I=I, E=E, top_k=k, x_scale=2.0, wfmt=wfmt)
    d = _dev(c)
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    lim = torch.tensor(np.linspace(2.0, 4.0, L), dtype=torch.float32, device=DEV)
    sl = slice(off, off + L)
    ref = _oracle(c, ids, w, L=L, local_offset=off, activation="swiglu_step",
                  limits=lim.cpu().numpy())
    for choice in (0, 1):
        M.moe_tune_clear()
        for stage in (1, 2):
            M.moe_tune_set(T, H, I, E, k, stage, choice, num_local_experts=L, local_expert_offset=off,
                           weight_format=wfmt)
        out = _fwd(c, d, ids, w, d["w1"][sl], d["w1_sf"][sl], d["w2"][sl], d["w2_sf"][sl],
                   num_local_experts=L, local_expert_offset=off, activation="swiglu_step",
                   clamp_limit=lim)
        assert_close_bf16(out, ref, MX_MAX_ABS, MX_REL, what=f"{wfmt} family {choice}")
    M.moe_tune_clear()


def _layer(c, ids, w, finalize="deterministic"):
    lim = None if c.limits is None else torch.from_numpy(c.limits).to(DEV)
    return M.moe_ffn_forward(c.x.to(DEV), ids, w, c.w1.to(DEV), c.w2.to(DEV), c.num_experts,
                             c.num_local, c.local_offset, c.activation, lim, finalize=finalize)


def _layer_oracle(c, ids, w):
    return O.moe_forward(S.bf16_to_f32(c.x), ids.cpu().numpy(), w.cpu().numpy().astype(np.float64),
                         S.bf16_to_f32(c.w1), S.bf16_to_f32(c.w2), num_experts=c.num_experts,
                         local_offset=c.local_offset, activation_kind=c.activation, limits=c.limits)


BF16_CASES = [
    # (T, H, I, E, k, L, off): ~256 rows per local expert with ragged tails (the expert
    # shard's bucket), ~40 rows per expert, and a row count beyond several 128-row tiles
    (1024, 512, 384, 256, 8, 32, 64),
    (160, 256, 256, 64, 2, 16, 8),
    (700, 256, 640, 4, 2, 4, 0),
]


@pytest.mark.parametrize("T,H,I,E,k,L,off", BF16_CASES)
def test_bf16_tile_families_match_oracle(T, H, I, E, k, L, off):
    """Both bf16 stages recorded to the 256-row, then the 128-row tile (two 32-row blocks
    per row-wave, the 64-row variant for short tails, the split last round), against the
    oracle in both finalize modes; with the table cleared the built-in rule (128 rows when
    T * k <= 64 * E) gives that family's bits."""
    c = S.moe_case("tune128", T, H, I, E, k, num_local=L, local_offset=off,
                   activation="swiglu_step", limit_range=(1.0, 3.0), x_scale=2.0, seed=T + I)
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), k)
    ref = _layer_oracle(c, ids, w)
    outs = {}
    for choice in (0, 1):
        M.moe_tune_clear()
        for stage in (1, 2):
            M.moe_tune_set(T, H, I, E, k, stage, choice, num_local_experts=L, local_expert_offset=off)
        for fin in ("deterministic", "fused"):
            out = _layer(c, ids, w, fin)
            assert_close_bf16(out, ref, what=f"{256 >> choice}-row {fin}")
            if fin == "deterministic":
                outs[choice] = out
    M.moe_tune_clear()
    default = _layer(c, ids, w)
    torch.cuda.synchronize()
    assert torch.equal(default, outs[1 if T * k <= 64 * E else 0])


def test_bf16_128_row_family_integer_exact():
    """On integer-valued operands every fp32 sum is exact, so the 128-row FC2 gives the
    256-row FC2's bits (tile edges, ragged groups, the split last round)."""
    sizes = np.array([300, 0, 1, 129, 64, 513, 127, 200])
    K, N = 512, 768
    c = S.grouped_gemm_case(seed=31, sizes=sizes, K=K, N=N, integer_valued=True)
    act, w2 = c.x.to(DEV), c.w.to(DEV)
    offs = torch.from_numpy(c.offs).to(DEV)
    M_ = int(sizes.sum())
    M.moe_tune_clear()
    y256 = M.moe_fc2(act, w2, offs, M_, 1, len(sizes))
    M.moe_tune_set(M_, N, K, len(sizes), 1, 2, 1)
    y128 = M.moe_fc2(act, w2, offs, M_, 1, len(sizes))
    M.moe_tune_clear()
    torch.cuda.synchronize()
    assert torch.equal(y128[:M_], y256[:M_])
    np.testing.assert_array_equal(to_np(y128)[:M_],
                                  bf16_round(O.grouped_gemm_fwd(S.bf16_to_f32(c.x), S.bf16_to_f32(c.w),
                                                                c.offs)))


def test_bf16_tuner_keeps_parity_and_clear_restores():
    c = S.moe_case("tunebf16", 2048, 512, 512, 64, 4, num_local=16, local_offset=16,
                   activation="swiglu", seed=77)
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    M.moe_tune_clear()
    before = _layer(c, ids, w)
    choice = M.moe_tune(c.x.to(DEV), ids, w, c.w1.to(DEV), c.w2.to(DEV), c.num_experts,
                        num_local_experts=c.num_local, local_expert_offset=c.local_offset)
    assert all(ch in (0, 1) for ch in choice)
    assert_close_bf16(_layer(c, ids, w), _layer_oracle(c, ids, w), what=f"bf16 tuned {choice}")
    M.moe_tune_clear()
    after = _layer(c, ids, w)
    torch.cuda.synchronize()
    assert torch.equal(before, after)


def test_fused_finalize_column_first_dealing():
    """I = 128 with a 32 MiB output: the fused-finalize FC2 deals its tiles column tile
    first (the SM90 page's raster switch); the output still matches the oracle."""
    c = S.moe_case("raster", 4096, 4096, 128, 8, 2, seed=81)
    assert c.T * c.H * 2 >= 32 << 20
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    out = _layer(c, ids, w, "fused")
    torch.cuda.synchronize()
    assert_close_bf16(out, _layer_oracle(c, ids, w), what="fused, column-first dealing")
