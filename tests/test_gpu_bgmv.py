"""GPU parity: BGMV MoE-LoRA shrink + expand (BGMV page) against the oracle.

The oracle rounds the shrink output to bf16 as the page's shrink dtype asks; the
library rounds its float32 sum. Bar, element by element: a shrink value within one
bf16 step (2^-7 relative) of the oracle's plus the float32 accumulation error of its
sum (H 2^-24 of the absolute sum), and y within that shrink error carried through
|w| |s| |B| plus the float32 accumulation of the expand; at least 99% of the shrink
values equal bit for bit. Both pipelines (per pair, and grouped by (LoRA, expert)
bin, BGMV page Parameters: grouped) are held to this bar; the grouped one's weighted
expand rows are rounded once more (w times the row, then the ordered sum), covered by
one more 2^-24 of the absolute terms.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_softmax_amd as M
import moe_synth as S
import oracle as O
from parity import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev(c):
    return dict(x=c.x.to(DEV), a=c.lora_a.to(DEV), b=c.lora_b.to(DEV),
                tok=torch.from_numpy(c.sorted_token_ids).to(DEV),
                ex=torch.from_numpy(c.expert_ids).to(DEV),
                li=torch.from_numpy(c.lora_indices).to(DEV),
                w=torch.from_numpy(c.topk_weights).to(DEV))


def _run(c, d=None, **kw):
    d = d or _dev(c)
    return M.moe_bgmv(d["x"], d["a"], d["b"], d["tok"], d["ex"], d["li"], d["w"], c.num_experts, **kw)


def _check(c, y, s, tok=None, ex=None, li=None, w=None):
    tok = c.sorted_token_ids if tok is None else tok
    ex = c.expert_ids if ex is None else ex
    li = c.lora_indices if li is None else li
    w = c.topk_weights if w is None else w
    x = S.bf16_to_f32(c.x).astype(np.float64)
    A = S.bf16_to_f32(c.lora_a).astype(np.float64)
    B = S.bf16_to_f32(c.lora_b).astype(np.float64)
    H = x.shape[1]
    y_ref, s_ref = O.bgmv_moe(x, A, B, tok, ex, li, w, shrink_dtype="bf16")
    s_abs = O.bgmv_shrink(np.abs(x), np.abs(A), tok, ex, li)
    bs = 2.0 ** -7 * np.abs(s_ref) + H * 2.0 ** -24 * s_abs
    s_got = to_np(s).astype(np.float64)
    assert np.all(np.abs(s_got - s_ref) <= bs + 1e-30), "shrink beyond one bf16 step"
    assert np.mean(s_got == s_ref) >= 0.99
    r = A.shape[2]
    kmax = np.bincount(np.asarray(tok)[(np.asarray(tok) >= 0) & (np.asarray(tok) < x.shape[0])],
                       minlength=1).max(initial=0)
    by = O.bgmv_expand(bs, np.abs(B), tok, ex, li, np.abs(w), x.shape[0])
    by += (r + kmax + 1) * 2.0 ** -24 * O.bgmv_expand(np.abs(s_ref) + bs, np.abs(B), tok, ex, li,
                                                   np.abs(w), x.shape[0])
    y_got = to_np(y).astype(np.float64)
    assert np.all(np.abs(y_got - y_ref) <= by + 1e-30), "y beyond the derived bound"
    return y_ref


@pytest.mark.parametrize("grouped", [None, True])
@pytest.mark.parametrize("order", ["contiguous", "expert", "random"])
@pytest.mark.parametrize("rank", [8, 16, 32, 64])
def test_bgmv_orders_and_ranks(order, rank, grouped):
    c = S.bgmv_case(seed=rank, T=96, H=512, rank=rank, num_loras=3, E=8, top_k=2, order=order)
    y, s = _run(c, grouped=grouped)
    _check(c, y, s)


@pytest.mark.parametrize("grouped", [None, True])
@pytest.mark.parametrize("H,feat_out,top_k,T", [(2688, 2688, 2, 64), (3072, 1024, 8, 40),
                                                 (520, 264, 1, 33)])
def test_bgmv_shapes(H, feat_out, top_k, T, grouped):
    """Hidden sizes of the page (2688, 3072), feat_out != H, top-1 / top-8, widths that
    are multiples of 8 but not of 64 or 256 (partial column tiles)."""
    c = S.bgmv_case(seed=H, T=T, H=H, rank=32, num_loras=2, E=16, top_k=top_k, feat_out=feat_out,
                    order="random")
    y, s = _run(c, grouped=grouped)
    _check(c, y, s)


@pytest.mark.parametrize("rank", [16, 64])
@pytest.mark.parametrize("T", [96, 2048, 2560])
def test_bgmv_grouped_contraction_whole_and_in_two(T, rank):
    """The grouped shrink cuts each 32-route tile's contraction in two when the tiles
    would fill at most half the CUs (T=96) and keeps it whole otherwise (T=2048, 160
    tiles); rank 64 takes two MFMA column blocks per tile. Up to 4096 pairs one
    workgroup bins and places the pairs; 5120 pairs (T=2560) take the clear, bin and
    stable-sort launches. Hidden 1032 ends in a partial
    64-value block and 520 output columns in a partial 512-column tile; all against
    the oracle's bound."""
    c = S.bgmv_case(seed=T + rank, T=T, H=1032, rank=rank, num_loras=4, E=8, top_k=2,
                    feat_out=520, order="random")
    y, s = _run(c, grouped=True)
    _check(c, y, s)


@pytest.mark.parametrize("grouped", [None, True])
def test_bgmv_few_pairs_split_hidden_and_invalid_indices(grouped):
    """3 tokens, 4 pairs: the shrink splits the hidden dimension (a second launch sums
    the partials); invalid token / expert / LoRA indices contribute nothing and tokens
    without a pair get zero rows."""
    c = S.bgmv_case(seed=7, T=3, H=4096, rank=16, num_loras=2, E=8, top_k=2, order="random")
    tok, ex, li, w = (c.sorted_token_ids.copy(), c.expert_ids.copy(), c.lora_indices.copy(),
                      c.topk_weights.copy())
    tok[1] = 3          # past the last token
    ex[4] = 8           # past the last expert
    li[2] = -1          # token 2: no adapter
    d = _dev(c)
    d.update(tok=torch.from_numpy(tok).to(DEV), ex=torch.from_numpy(ex).to(DEV),
             li=torch.from_numpy(li).to(DEV))
    y, s = _run(c, d, grouped=grouped)
    y_ref = _check(c, y, s, tok, ex, li, w)
    assert np.all(to_np(y)[2] == 0) and np.all(y_ref[2] == 0)
    assert np.all(to_np(s)[1] == 0) and np.all(to_np(s)[4] == 0)


@pytest.mark.parametrize("grouped", [None, True])
def test_bgmv_token_with_many_pairs_uses_ordered_scan(grouped):
    """Token 0 owns 24 pairs (beyond the 16-slot route index): its routes are found by
    an ordered scan of all pairs."""
    c = S.bgmv_case(seed=9, T=16, H=256, rank=32, num_loras=2, E=32, top_k=2, order="random")
    g = np.random.default_rng(10)
    extra_ex = g.permutation(32)[:24].astype(np.int32)
    tok = np.concatenate([c.sorted_token_ids, np.zeros(24, np.int32)])
    ex = np.concatenate([c.expert_ids, extra_ex])
    w = np.concatenate([c.topk_weights, g.random(24).astype(np.float32)])
    perm = g.permutation(tok.shape[0])
    tok, ex, w = tok[perm].copy(), ex[perm].copy(), w[perm].copy()
    d = _dev(c)
    d.update(tok=torch.from_numpy(tok).to(DEV), ex=torch.from_numpy(ex).to(DEV),
             w=torch.from_numpy(w).to(DEV))
    y, s = _run(c, d, grouped=grouped)
    _check(c, y, s, tok, ex, None, w)


def test_bgmv_strided_output_replay_and_graph():
    c = S.bgmv_case(seed=11, T=64, H=1024, rank=32, num_loras=4, E=8, top_k=2, order="expert")
    d = _dev(c)
    wide = torch.full((c.x.shape[0], 3000), 7.0, dtype=torch.float32, device=DEV)
    view = wide[:, 100:100 + c.lora_b.shape[2]]
    y1, s1 = _run(c, d, y_accum=view)
    _check(c, y1, s1)
    assert torch.all(wide[:, :100] == 7.0) and torch.all(wide[:, 100 + c.lora_b.shape[2]:] == 7.0)
    y2, _ = _run(c, d)
    assert torch.equal(y2, y1)
    # graph capture: replays with new routing weights written in place
    out = torch.empty((c.x.shape[0], c.lora_b.shape[2]), dtype=torch.float32, device=DEV)
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=DEV)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        _run(c, d, y_accum=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run(c, d, y_accum=out, workspace=ws)
    for k in range(3):
        d["w"].copy_(torch.from_numpy(c.topk_weights * (k + 1.5)))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref, _ = _run(c, d)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)


@pytest.mark.parametrize("grouped", [False, True])
def test_bgmv_page_shape_full_size(grouped):
    """The page's measured shape: hidden 3072, rank 32, 2048 tokens, top-2 contiguous
    (4 LoRAs x 8 experts: 128 routes per bin, where the library picks the grouped
    pipeline itself), both pipelines; each replays bit for bit, and the strided output
    of the grouped one equals its contiguous output."""
    c = S.bgmv_case(seed=0, T=2048, H=3072, rank=32, num_loras=4, E=8, top_k=2)
    d = _dev(c)
    y, s = _run(c, d, grouped=grouped)
    torch.cuda.synchronize()
    _check(c, y, s)
    y2, _ = _run(c, d, grouped=grouped)
    assert torch.equal(y, y2)
    if grouped:
        y_auto, _ = _run(c, d)
        assert torch.equal(y_auto, y)
        wide = torch.full((2048, 3200), 7.0, dtype=torch.float32, device=DEV)
        y3, _ = _run(c, d, grouped=True, y_accum=wide[:, 64:64 + 3072])
        assert torch.equal(y3, y) and torch.all(wide[:, :64] == 7.0)
