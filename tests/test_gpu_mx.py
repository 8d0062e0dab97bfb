"""GPU parity: the fp8-activation layers against the oracle: MXFP4 weights (the W4A8
page's layer), MXFP8 weights (e4m3 codes, same UE8M0 block-32 scales) and fp8 with
per-tensor scales (StepFun page, intro: the fp8 per-tensor weight family).

The oracle works on the dequantized operands in float64 and models the one
lossy step of the method, the requantization of the FC1 output (MXFP8 with the
UE8M0 round-up of the W4A8 page's intro, or e4m3 with the static per-tensor
scale). Tolerance for these outputs: max-abs 8e-2 (applied as |d| / max(1, |ref|))
and relative L2 3e-2.
"""
import numpy as np
import pytest
import torch

import mixture_experts_expert_softmax_amd as M
import moe_synth as S
import oracle as O
from parity import assert_close_bf16, bf16_round, mx_dequant_table, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
MX_MAX_ABS, MX_REL = 8e-2, 3e-2


WFMTS = ["mxfp4", "mxfp8", "fp8"]


def _deq(wfmt, codes, scales):
    if wfmt == "fp8":
        return O.fp8_dequant(codes, scales)
    return mx_dequant_table(wfmt, codes, scales)


class _LazyBank:
    """Expert bank that dequantizes one expert at a time for the oracle (optionally
    remembering the experts it has decoded)."""

    def __init__(self, codes, scales, wfmt, cache=None):
        self.codes, self.scales, self.wfmt, self.cache = codes, scales, wfmt, cache
        self.shape = (codes.shape[0], codes.shape[1], codes.shape[2] * (2 if wfmt == "mxfp4" else 1))

    def __getitem__(self, e):
        if self.cache is not None and e in self.cache:
            return self.cache[e]
        v = _deq(self.wfmt, self.codes[e], self.scales[e])
        if self.cache is not None:
            # float32 halves the memory of a decoded bank: exact for the MX families
            # (code value times a power of two), within 2^-24 relative for fp8 per-tensor
            self.cache[e] = v = v.astype(np.float32)
        return v


def _dev(c):
    keys = ("x", "x_sf", "w1", "w1_sf", "w2", "w2_sf") + (("act_scale",) if c.wfmt == "fp8" else ())
    return {k: torch.from_numpy(np.ascontiguousarray(getattr(c, k))).to(DEV) for k in keys}


def _oracle(c, ids, w, tokens=None, num_experts=None, local_offset=0, L=None,
            activation="swiglu", limits=None, cache1=None, cache2=None):
    ids_n, w_n = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    x, xs = c.x, c.x_sf
    if tokens is not None:
        x, ids_n, w_n = x[tokens], ids_n[tokens], w_n[tokens]
        xs = xs if c.wfmt == "fp8" else xs[tokens]
    w1, w1s, w2, w2s = c.w1, c.w1_sf, c.w2, c.w2_sf
    if L is not None:
        w1, w1s = w1[local_offset:local_offset + L], w1s[local_offset:local_offset + L]
        w2, w2s = w2[local_offset:local_offset + L], w2s[local_offset:local_offset + L]
    pt = c.wfmt == "fp8"
    xd = O.fp8_dequant(x, xs[0]) if pt else O.mx_dequant_fp8(x, xs)
    return O.moe_forward(xd, ids_n, w_n, _LazyBank(w1, w1s, c.wfmt, cache1),
                         _LazyBank(w2, w2s, c.wfmt, cache2),
                         num_experts=num_experts or c.num_experts, local_offset=local_offset,
                         activation_kind=activation, limits=limits, requant=not pt,
                         act_scale=float(c.act_scale[0]) if pt else None)


def _fwd(c, d, ids, w, w1, w1s, w2, w2s, **kw):
    """The layer through the entry point of the case's weight family."""
    if c.wfmt == "fp8":
        return M.moe_ffn_forward_fp8(d["x"], d["x_sf"], ids, w, w1, w1s, w2, w2s, d["act_scale"],
                                     c.num_experts, **kw)
    return M.moe_ffn_forward_mx(d["x"], d["x_sf"], ids, w, w1, w1s, w2, w2s, c.num_experts, **kw)


def _force_family(c, family, stages=(1, 2), L=None, off=0):
    """Record tile family `family` (0 the 256-row tile, 1 the decode kernel) for the
    given stages of case c's shape and bucket; None leaves the built-in rule."""
    M.moe_tune_clear()
    if family is not None:
        for st in stages:
            M.moe_tune_set(c.T, c.H, c.I, c.num_experts, c.top_k, st, family, num_local_experts=L,
                           local_expert_offset=off, weight_format=c.wfmt)


def _run(c, d, ids=None, w=None, **kw):
    if ids is None:
        ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    out = _fwd(c, d, ids, w, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"], **kw)
    return out, ids, w


@pytest.mark.parametrize("wfmt", WFMTS)
@pytest.mark.parametrize("T", [1, 16, 77, 300])
def test_mx_small_layer(T, wfmt):
    c = S.w4a8_moe(seed=T, T=T, H=256, I=384, E=8, top_k=2, wfmt=wfmt)
    out, ids, w = _run(c, _dev(c))
    assert_close_bf16(out, _oracle(c, ids, w), MX_MAX_ABS, MX_REL, what=f"{wfmt} T={T}")


@pytest.mark.parametrize("wfmt", WFMTS)
def test_mx_top8_of_64_small_dims(wfmt):
    c = S.w4a8_moe(seed=5, T=128, H=512, I=256, E=64, top_k=8, wfmt=wfmt)
    out, ids, w = _run(c, _dev(c))
    assert_close_bf16(out, _oracle(c, ids, w), MX_MAX_ABS, MX_REL, what=f"{wfmt} E=64 k=8")


@pytest.mark.parametrize("wfmt", WFMTS)
def test_mx_decode_uneven_contraction_split(wfmt):
    """H=1280 and I=768: 5 and 3 stages of 256 contraction values (MXFP4) or 10 and 6
    of 128 (MXFP8), split unevenly over the decode kernel's 4 waves (with MXFP4 one
    wave of FC2 gets none)."""
    c = S.w4a8_moe(seed=9, T=5, H=1280, I=768, E=16, top_k=4, wfmt=wfmt)
    _force_family(c, 1)   # both stages on the decode kernel
    out, ids, w = _run(c, _dev(c))
    M.moe_tune_clear()
    assert_close_bf16(out, _oracle(c, ids, w), MX_MAX_ABS, MX_REL, what=f"{wfmt} uneven split")


def test_mxfp8_decode_short_contraction():
    """I=128 with MXFP8 weights: FC2 has one 128-value stage, so three of the decode
    kernel's four waves get no contraction at all."""
    c = S.w4a8_moe(seed=10, T=3, H=256, I=128, E=8, top_k=2, wfmt="mxfp8")
    out, ids, w = _run(c, _dev(c))
    assert_close_bf16(out, _oracle(c, ids, w), MX_MAX_ABS, MX_REL, what="mxfp8 I=128")


# T=200 with the built-in rule (the 256-row tile kernel), T=12 on the decode kernel
@pytest.mark.parametrize("wfmt", WFMTS)
@pytest.mark.parametrize("T,family", [(200, None), (12, 1)])
def test_mx_shard_and_step_activation(T, family, wfmt):
    c = S.w4a8_moe(seed=6, T=T, H=256, I=256, E=16, top_k=4, x_scale=4.0, wfmt=wfmt)
    d = _dev(c)
    L, off = 6, 5
    lim = torch.tensor(np.linspace(2.0, 4.0, L), dtype=torch.float32, device=DEV)
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    _force_family(c, family, L=L, off=off)
    out = _fwd(c, d, ids, w, d["w1"][off:off + L], d["w1_sf"][off:off + L], d["w2"][off:off + L],
               d["w2_sf"][off:off + L], num_local_experts=L, local_expert_offset=off,
               activation="swiglu_step", clamp_limit=lim)
    M.moe_tune_clear()
    ref = _oracle(c, ids, w, L=L, local_offset=off, activation="swiglu_step",
                  limits=lim.cpu().numpy())
    assert_close_bf16(out, ref, MX_MAX_ABS, MX_REL, what=f"{wfmt} shard step")


@pytest.mark.parametrize("wfmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("T,family", [(256, 0), (24, 1)])
def test_fc1_requant_matches_oracle_rule(T, family, wfmt):
    """The fused UE8M0 round-up requantization: scale codes equal the oracle's (rare
    one-step flips allowed where the float32 activations differ in the last bits),
    and the dequantized act stays within half an e4m3 step of the exact activation.
    T=256 on the 256-row tile kernel, T=24 on the decode kernel."""
    c = S.w4a8_moe(seed=7, T=T, H=512, I=512, E=4, top_k=2, wfmt=wfmt)
    d = _dev(c)
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    srt = M.moe_sort(ids, c.num_experts)
    _force_family(c, family, stages=(1,))
    act, act_sf = M.moe_fc1_mx(d["x"], d["x_sf"], d["w1"], d["w1_sf"], srt["offs"], srt["p2e"],
                               c.top_k, c.num_experts)
    M.moe_tune_clear()
    n = int(srt["n_local"].item())
    p2e = srt["p2e"][:n].cpu().numpy()
    offs = srt["offs"].cpu().numpy()
    xd = O.mx_dequant_fp8(c.x, c.x_sf)
    a_ref = np.zeros((n, c.I))
    start = 0
    for e in range(c.num_experts):
        rows = slice(start, int(offs[e]))
        h = xd[p2e[rows] // c.top_k] @ _deq(wfmt, c.w1[e], c.w1_sf[e]).T
        a_ref[rows] = O.activation(h, "swiglu")
        start = int(offs[e])
    vals, codes = O.requant_e4m3(a_ref.astype(np.float32))
    got_codes = act_sf[:n].cpu().numpy()
    assert np.mean(got_codes == codes) > 0.995
    assert np.all(np.abs(got_codes.astype(int) - codes.astype(int)) <= 1)
    deq = O.mx_dequant_fp8(act[:n].cpu().numpy(), got_codes)
    scale = np.repeat(np.exp2(got_codes.astype(np.float64) - 127), 32, axis=1)
    # half an e4m3 step (2^-4 relative, 2^-10 of the scale in the subnormal range) plus slack
    bound = np.maximum(np.abs(a_ref) * 2.0 ** -4, scale * 2.0 ** -10) * 1.01 + 1e-6 * np.abs(a_ref)
    assert np.mean(np.abs(deq - a_ref) <= bound) > 0.999


@pytest.mark.parametrize("T,family", [(256, 0), (24, 1)])
def test_fp8_fc1_per_tensor_requant_matches_oracle_rule(T, family):
    """The per-tensor requantization (static scale, float32 reciprocal, saturation at
    +-448): codes equal the oracle's apart from rare flips within the float32
    accumulation error of the activation. x_scale 4 drives some activations past the
    saturation point 448 * act_scale = 16. T=256 on the 256-row tile kernel, T=24 on
    the decode kernel."""
    c = S.w4a8_moe(seed=7, T=T, H=512, I=512, E=4, top_k=2, wfmt="fp8", x_scale=4.0)
    d = _dev(c)
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    srt = M.moe_sort(ids, c.num_experts)
    _force_family(c, family, stages=(1,))
    act = M.moe_fc1_fp8(d["x"], d["x_sf"], d["w1"], d["w1_sf"], d["act_scale"], srt["offs"],
                        srt["p2e"], c.top_k, c.num_experts)
    M.moe_tune_clear()
    n = int(srt["n_local"].item())
    p2e = srt["p2e"][:n].cpu().numpy()
    offs = srt["offs"].cpu().numpy()
    xd = O.fp8_dequant(c.x, c.x_sf[0])
    I = c.I
    h = np.zeros((n, 2 * I))
    habs = np.zeros((n, 2 * I))      # sum over k of |x_k w_k|, which bounds the rounding
    start = 0
    for e in range(c.num_experts):
        rows = slice(start, int(offs[e]))
        w1 = O.fp8_dequant(c.w1[e], c.w1_sf[e])
        xr = xd[p2e[rows] // c.top_k]
        h[rows] = xr @ w1.T
        habs[rows] = np.abs(xr) @ np.abs(w1).T
        start = int(offs[e])
    a_ref = O.activation(h, "swiglu")
    _, codes = O.requant_e4m3_per_tensor(a_ref.astype(np.float32), c.act_scale[0])
    got = act[:n].cpu().numpy()
    sat = np.abs(a_ref) > 16.5
    assert np.mean(sat) > 1e-4                               # saturation is exercised
    assert np.all(O.e4m3_decode(got[sat]) == 448.0 * np.sign(a_ref[sat]))
    assert np.mean(got == codes) > 0.995
    # where they differ, by one code step plus the float32 accumulation error of the
    # activation: a float32 sum of K = 512 products is off by at most
    # K * 2^-24 * sum|x_k w_k| = 2^-15 * sum|x_k w_k| (2^-14 taken for margin), carried
    # through silu(g) * u; it matters where u or g nearly cancels and in the subnormal
    # codes (steps of 2^-9 * act_scale)
    s = float(c.act_scale[0])
    gv, rv = O.e4m3_decode(got) * s, O.e4m3_decode(codes) * s
    u, g = h[:, :I], h[:, I:]
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
    da = 2.0 ** -14 * (np.abs(g * sig) * habs[:, :I] + dsilu * np.abs(u) * habs[:, I:])
    step = np.maximum(np.abs(rv), np.abs(gv)) * 2.0 ** -3 + 2.0 ** -9 * s
    assert np.all(np.abs(gv - rv) <= step + da)


@pytest.mark.parametrize("wfmt,I", [("mxfp4", 256), ("mxfp4", 2048), ("mxfp8", 256), ("mxfp8", 2048)])
def test_mx_fc2_every_tile_height_exact(wfmt, I):
    """FC2 of the 256-row kernel on operands whose fp32 sums are all exact (e4m3
    activations holding integers up to 6, weights that are multiples of 1/2 up to 6 or
    8, block scales 2^-1 .. 2^2): the output is the bf16 rounding of the exact grouped
    product, bit for bit. The experts' row counts give tiles holding 1..64, 65..128,
    129..192 and 193..256 rows (the 32-row blocks a tile multiplies follow its rows),
    empty experts and several tiles per expert. With a contraction of 2048 the block
    scales are copied in groups of 512 values per row (two buffers, each reused)."""
    rng = np.random.default_rng(43)
    sizes = np.array([1, 64, 65, 128, 0, 129, 192, 193, 256, 300, 511, 37, 0, 90])
    L, R, H = len(sizes), int(sizes.sum()), 512
    ends = np.cumsum(sizes).astype(np.int32)
    act_v = rng.integers(-6, 7, size=(R, I)).astype(np.float32)
    act = torch.from_numpy(act_v).to(torch.float8_e4m3fn).view(torch.uint8)
    act_sf = rng.integers(126, 130, size=(R, I // 32)).astype(np.uint8)
    if wfmt == "mxfp4":
        w2 = rng.integers(0, 256, size=(L, H, I // 2)).astype(np.uint8)
    else:
        w2_v = rng.integers(-12, 13, size=(L, H, I)).astype(np.float32) / 2
        w2 = torch.from_numpy(w2_v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    w2_sf = rng.integers(126, 129, size=(L, H, I // 32)).astype(np.uint8)
    y = M.moe_fc2_mx(act.to(DEV), torch.from_numpy(act_sf).to(DEV), torch.from_numpy(w2).to(DEV),
                     torch.from_numpy(w2_sf).to(DEV), torch.from_numpy(ends).to(DEV), R, 1, L)
    torch.cuda.synchronize()
    a_deq = O.mx_dequant_fp8(act.numpy(), act_sf)
    w_deq = mx_dequant_table(wfmt, w2, w2_sf)
    ref = O.grouped_gemm_fwd(a_deq, w_deq, ends)
    np.testing.assert_array_equal(to_np(y)[:R], bf16_round(ref))


@pytest.mark.parametrize("wfmt", WFMTS)
def test_mx_zero_tokens_and_replay(wfmt):
    c = S.w4a8_moe(seed=8, T=64, H=256, I=256, E=8, top_k=2, wfmt=wfmt)
    d = _dev(c)
    o1, ids, w = _run(c, d)
    o2, _, _ = _run(c, d, ids, w)
    assert torch.equal(o1, o2)
    e = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    ew = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    d0 = dict(d, x=d["x"][:0], x_sf=d["x_sf"] if wfmt == "fp8" else d["x_sf"][:0])
    z = _fwd(c, d0, e, ew, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"])
    assert z.shape == (0, 256)


@pytest.fixture(scope="module", params=WFMTS)
def mx_full(request):
    return S.w4a8_moe(seed=0, T=8192, wfmt=request.param), {}, {}


def _tile_cover_tokens(ids, num_experts, tile=256):
    """Tokens that own the first and the last row of every 256-row tile of every
    expert's group in the sorted order: every tile of both GEMMs gets compared."""
    T, k = ids.shape
    srt = O.sort_routes(ids, num_experts, num_experts, 0)
    rows, start = [], 0
    for end in srt["offs"].tolist():
        for r0 in range(start, end, tile):
            rows += [r0, min(r0 + tile, end) - 1]
        start = end
    return np.unique(srt["p2e"][np.asarray(rows, np.int64)] // k)


@pytest.mark.parametrize("T", [1, 16, 128, 1024, 8192])
def test_mx_full_shape(mx_full, T):
    """H=7168, I=2048, 64 experts, top-8 over the decode-to-prefill sweep, for the three
    weight families: every token against the oracle up to T=1024; at T=8192 the tokens
    that own the first and last rows of every 256-row tile of every expert, plus 64
    random ones."""
    full, cache1, cache2 = mx_full
    x_sf = full.x_sf if full.wfmt == "fp8" else full.x_sf[:T]
    c = S.W4A8Case(T, full.H, full.I, full.num_experts, full.top_k, full.logits[:T], full.x[:T],
                   x_sf, full.w1, full.w1_sf, full.w2, full.w2_sf, full.wfmt, full.act_scale)
    out, ids, w = _run(c, _dev(c))
    torch.cuda.synchronize()
    tokens = None
    if T > 1024:
        cover = _tile_cover_tokens(ids.cpu().numpy(), c.num_experts)
        extra = np.random.default_rng(T).choice(T, 64, replace=False)
        tokens = np.unique(np.concatenate([cover, extra]))
        assert tokens.size >= 2 * c.num_experts
    ref = _oracle(c, ids, w, tokens=tokens, cache1=cache1, cache2=cache2)
    got = to_np(out) if tokens is None else to_np(out)[tokens]
    assert_close_bf16(got, ref, MX_MAX_ABS, MX_REL, what=f"{full.wfmt} full T={T}")


@pytest.mark.parametrize("wfmt", WFMTS)
def test_mx_work_queue_matches_stage_entries(wfmt):
    """With 256 rows per expert on average (T=1024, 16 experts, top-4) the layer runs
    both 256-row GEMMs as the work-queue kernel; the stage entry points run the kernel
    with one tile per workgroup. Both compute every tile the same way, so the stage
    chain (sort, FC1, FC2, deterministic finalize) reproduces the layer bit for bit, on
    two calls in a row (the queue counters reset themselves)."""
    c = S.w4a8_moe(seed=11, T=1024, H=1024, I=512, E=16, top_k=4, wfmt=wfmt)
    d = _dev(c)
    M.moe_tune_clear()
    out1, ids, w = _run(c, d)
    out2, _, _ = _run(c, d, ids, w)
    srt = M.moe_sort(ids, c.num_experts)
    if wfmt == "fp8":
        act = M.moe_fc1_fp8(d["x"], d["x_sf"], d["w1"], d["w1_sf"], d["act_scale"], srt["offs"],
                            srt["p2e"], c.top_k, c.num_experts)
        y = M.moe_fc2_fp8(act, d["act_scale"], d["w2"], d["w2_sf"], srt["offs"], c.T, c.top_k,
                          c.num_experts)
    else:
        act, act_sf = M.moe_fc1_mx(d["x"], d["x_sf"], d["w1"], d["w1_sf"], srt["offs"],
                                   srt["p2e"], c.top_k, c.num_experts)
        y = M.moe_fc2_mx(act, act_sf, d["w2"], d["w2_sf"], srt["offs"], c.T, c.top_k,
                         c.num_experts)
    ref = M.moe_finalize(y, srt["e2p"], w)
    torch.cuda.synchronize()
    assert torch.equal(out1, ref)
    assert torch.equal(out2, ref)
    oracle = _oracle(c, ids, w)
    assert_close_bf16(to_np(out1), oracle, MX_MAX_ABS, MX_REL, what=f"{wfmt} queue layer")
