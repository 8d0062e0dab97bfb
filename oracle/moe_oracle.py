"""CPU oracle for the routed Mixture-of-Experts expert layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the tests, the smoke check of ``__graft_entry__`` and the benchmark's
CPU-baseline leg call it. It shares no code with the HIP library.

Everything here is plain numpy in float64 (integer work in int64/int32). Each
function follows one passage of the documentation pages it cites:

* "flashinfer.experimental.cake_stepfun_moe" (the StepFun page): stage list
  (routing "Renormalize top-k", FC1 with the StepFun epilogue, FC2, finalize),
  the per-expert clamp limit of SwiGLUStep (default 7.0), the
  ``expanded_idx_to_permuted_idx`` output of the prepared launch, and its list
  of weight families (bf16, fp8 per-tensor, mxfp8 among them).
* "flashinfer.fused_moe.cake / cake_cute (MXFP4 SiTU routed MoE)" (the W4A8
  page): the MXFP8 activation / MXFP4 weight layouts with UE8M0 block-32
  scales, the canonical [up | gate] w1 bank, fp32 accumulation and the UE8M0
  round-up requantization.
* "Cake ragged BF16 grouped GEMM (experimental)" (the grouped-GEMM page): the
  fwd / dgrad / wgrad operation table and the ragged ``offs`` convention; its
  Autograd section (a backward made of dgrad and wgrad) for the layer backward.
* "flashinfer.fused_moe.cute_dsl_fused_moe_bf16" (the SM90 fused-MoE page):
  the forward formula, the EP shard rule and the two finalize paths.
* "flashinfer.fused_moe.prepare_bgmv_moe" (the BGMV page): the MoE-LoRA shrink
  and expand over routed (token, expert) pairs.

Where a step reaches a result with a plain definition, the function computes
that definition directly; the sort and the requantization are the method's
own discrete steps and are written as such.

Readings taken where the pages are silent (each is listed in the design doc):
routing selects on the raw logits with ties to the lower expert id; the sort
is stable and unpadded; SwiGLUStep clamps both halves symmetrically; a route
to an expert outside the local shard (or outside [0, E)) contributes zero; the
requantized scale is the smallest power of two that fits the block maximum;
the fp8 per-tensor family (named on the StepFun page without a layout) holds
e4m3fn codes with one float32 scale for x, one per expert matrix, and a static
float32 scale for the requantized FC1 output, whose codes saturate at +-448.

Parity pins for every function live in tests/test_oracle_*.py. Parity
unpinned: none of the functions below; the SwiGLUStep formula itself is a
reading (the pages name it without a formula) and is pinned only to that
reading.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "route", "sort_routes", "grouped_gemm_fwd", "grouped_gemm_dgrad",
    "grouped_gemm_wgrad", "silu", "activation", "moe_forward", "moe_route_outputs",
    "finalize", "e4m3_decode", "e4m3_encode", "e2m1_decode", "ue8m0_decode",
    "mx_dequant", "requant_e4m3", "minifloat_decode", "unpack_e2m1", "mx_dequant_fp4",
    "mx_dequant_fp8", "fp8_dequant", "requant_e4m3_per_tensor", "activation_backward",
    "moe_backward", "route_backward", "bgmv_shrink", "bgmv_expand", "bgmv_moe",
]


# ---------------------------------------------------------------------------
# Routing -- StepFun page, intro ("routing (Renormalize top-k)"); the pre-routed
# contract of the SM90 fused-MoE page ("global expert ids plus normalized scales").
# ---------------------------------------------------------------------------
def route(logits: np.ndarray, top_k: int):
    """Renormalized top-k routing.

    Slot s of token t holds the expert with the (s+1)-th largest logit; equal
    logits go to the lower expert id. The weight of slot s is the softmax of
    the selected logits alone, which equals softmax over all experts followed
    by renormalisation over the k selected (the common denominator cancels).

    Returns (ids int32 [T,k], weights float64 [T,k]).
    """
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    ids = np.zeros((T, top_k), dtype=np.int32)
    taken = np.zeros((T, E), dtype=bool)
    rows = np.arange(T)
    for s in range(top_k):
        # the largest logit not yet chosen; np.argmax returns the first (lowest-id) maximum
        cand = np.where(taken, -np.inf, lg)
        best = np.argmax(cand, axis=1)
        ids[:, s] = best
        taken[rows, best] = True
    sel = lg[rows[:, None], ids]
    z = np.exp(sel - sel[:, :1])
    weights = z / z.sum(axis=1, keepdims=True)
    return ids, weights


# ---------------------------------------------------------------------------
# Sort -- grouped-GEMM page (groups are consecutive row ranges, offs = cumulative
# ends, m_indptr with a leading zero, no padding); StepFun page, "Prepared
# launches" (expanded_idx_to_permuted_idx); SM90 fused-MoE page, Parameters
# (expanded index in (token, slot) order; EP via num_local_experts +
# local_expert_offset).
# ---------------------------------------------------------------------------
def local_expert(topk_ids: np.ndarray, num_experts: int, num_local: int, local_offset: int):
    """Local expert index of every route (flattened t*k+s order), -1 if foreign."""
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    loc = ids - local_offset
    ok = (ids >= 0) & (ids < num_experts) & (loc >= 0) & (loc < num_local)
    return np.where(ok, loc, -1)


def sort_routes(topk_ids: np.ndarray, num_experts: int, num_local: int, local_offset: int):
    """Stable, unpadded counting sort of the routes by local expert.

    Returns dict with
      offs     int32 [L]     cumulative end of each expert's rows
      m_indptr int32 [L+1]   [0, offs...]
      e2p      int32 [T*k]   permuted row of expanded index i = t*k+s, -1 if foreign
      p2e      int32 [n]     expanded index of permuted row p (inverse of e2p)
      n_local  int           number of local routes
    Within an expert the rows keep ascending expanded-index order.
    """
    loc = local_expert(topk_ids, num_experts, num_local, local_offset)
    n_routes = loc.shape[0]
    counts = np.array([np.count_nonzero(loc == e) for e in range(num_local)], dtype=np.int64)
    offs = np.cumsum(counts)
    starts = offs - counts
    e2p = np.full(n_routes, -1, dtype=np.int64)
    for e in range(num_local):
        members = np.nonzero(loc == e)[0]          # ascending expanded index
        e2p[members] = starts[e] + np.arange(members.shape[0])
    n_local = int(offs[-1]) if num_local else 0
    p2e = np.zeros(n_local, dtype=np.int64)
    local = e2p >= 0
    p2e[e2p[local]] = np.nonzero(local)[0]
    return dict(offs=offs.astype(np.int32),
                m_indptr=np.concatenate([[0], offs]).astype(np.int32),
                e2p=e2p.astype(np.int32), p2e=p2e.astype(np.int32), n_local=n_local)


# ---------------------------------------------------------------------------
# Grouped GEMM -- grouped-GEMM page, operation table.
# Group e owns rows [offs[e-1], offs[e]) (offs[-1] read as 0).
# ---------------------------------------------------------------------------
def _group_bounds(offs):
    offs = np.asarray(offs, dtype=np.int64).reshape(-1)
    starts = np.concatenate([[0], offs[:-1]])
    return list(zip(starts.tolist(), offs.tolist()))


def grouped_gemm_fwd(x, w, offs):
    """fwd: Y[rows of e] = X[rows of e] @ W[e].T   (x [M,K], w [E,N,K]) -> [M,N] f64.
    Rows past offs[E-1] are left at zero."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = np.zeros((x.shape[0], w.shape[1]))
    for e, (s, f) in enumerate(_group_bounds(offs)):
        if f > s:
            y[s:f] = x[s:f] @ w[e].T
    return y


def grouped_gemm_dgrad(g, w, offs):
    """dgrad: dX[rows of e] = G[rows of e] @ W[e]   (g [M,N], w [E,N,K]) -> [M,K] f64."""
    g = np.asarray(g, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dx = np.zeros((g.shape[0], w.shape[2]))
    for e, (s, f) in enumerate(_group_bounds(offs)):
        if f > s:
            dx[s:f] = g[s:f] @ w[e]
    return dx


def grouped_gemm_wgrad(g, x, offs):
    """wgrad: dW[e] = G[rows of e].T @ X[rows of e]   -> [E,N,K] f64; an empty
    group's dW[e] is exactly zero."""
    g = np.asarray(g, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    bounds = _group_bounds(offs)
    dw = np.zeros((len(bounds), g.shape[1], x.shape[1]))
    for e, (s, f) in enumerate(bounds):
        if f > s:
            dw[e] = g[s:f].T @ x[s:f]
    return dw


# ---------------------------------------------------------------------------
# FFN -- SM90 fused-MoE page, formula: ffn(x; e) = (silu(x @ w1_gate[e].T) *
# (x @ w1_up[e].T)) @ w2[e].T; W4A8 page, "Inputs": w1 rows are up then gate.
# SwiGLUStep: StepFun page, per-expert clamp limit (default 7.0).
# ---------------------------------------------------------------------------
def silu(z):
    """silu(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def activation(h, kind: str, limit: float = 7.0):
    """h [..., 2I] = [up | gate] pre-activations -> a [..., I].

    swiglu:      silu(gate) * up
    swiglu_step: silu(clamp(gate, -limit, limit)) * clamp(up, -limit, limit)
    """
    h = np.asarray(h, dtype=np.float64)
    I = h.shape[-1] // 2
    up, gate = h[..., :I], h[..., I:]
    if kind == "swiglu":
        return silu(gate) * up
    if kind == "swiglu_step":
        return silu(np.clip(gate, -limit, limit)) * np.clip(up, -limit, limit)
    raise ValueError(kind)


def moe_route_outputs(x, topk_ids, w1, w2, *, num_experts, local_offset=0,
                      activation_kind="swiglu", limits=None, requant=False, act_scale=None):
    """y[t, s] = ffn(x[t]; e[t,s]) for every route to a local expert (zeros for
    foreign routes). Returns float64 [T, k, H] and the local-route mask [T, k].

    ``requant`` applies the MXFP8 requantization of the activation (W4A8 page,
    intro: UE8M0 round-up requantization) before FC2; ``act_scale`` instead
    applies the fp8 per-tensor requantization with that static scale.
    """
    if requant and act_scale is not None:
        raise ValueError("requant and act_scale are exclusive")
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    L = w1.shape[0]
    H = x.shape[1]
    loc = local_expert(ids, num_experts, L, local_offset).reshape(T, k)
    y = np.zeros((T, k, H))
    for e in range(L):
        tt, ss = np.nonzero(loc == e)
        if tt.size == 0:
            continue
        w1e = np.asarray(w1[e], dtype=np.float64)
        w2e = np.asarray(w2[e], dtype=np.float64)
        lim = 7.0 if limits is None else float(limits[e])
        h = x[tt] @ w1e.T
        a = activation(h, activation_kind, lim)
        if requant:
            a = mx_dequant(*requant_e4m3(a.astype(np.float32)))
        elif act_scale is not None:
            a = requant_e4m3_per_tensor(a.astype(np.float32), act_scale)[0]
        y[tt, ss] = a @ w2e.T
    return y, loc >= 0


def moe_forward(x, topk_ids, topk_weights, w1, w2, *, num_experts, local_offset=0,
                activation_kind="swiglu", limits=None, requant=False, act_scale=None):
    """out[t] = sum over slots s (ascending) of w[t,s] * ffn(x[t]; e[t,s]),
    foreign routes contributing zero -> float64 [T, H] (unrounded)."""
    y, local = moe_route_outputs(x, topk_ids, w1, w2, num_experts=num_experts,
                                 local_offset=local_offset, activation_kind=activation_kind,
                                 limits=limits, requant=requant, act_scale=act_scale)
    w = np.asarray(topk_weights, dtype=np.float64)
    out = np.zeros((y.shape[0], y.shape[2]))
    for s in range(y.shape[1]):
        out += np.where(local[:, s:s + 1], w[:, s:s + 1] * y[:, s], 0.0)
    return out


# ---------------------------------------------------------------------------
# Finalize -- SM90 fused-MoE page, use_fused_finalize=False: rows in permuted
# order are gathered through expanded_idx_to_permuted_idx, scaled and summed
# in a fixed order.
# ---------------------------------------------------------------------------
def finalize(y_rows, e2p, topk_weights):
    """out[t] = sum_{s ascending, e2p[t*k+s] >= 0} w[t,s] * y_rows[e2p[t*k+s]] (f64)."""
    y_rows = np.asarray(y_rows, dtype=np.float64)
    w = np.asarray(topk_weights, dtype=np.float64)
    T, k = w.shape
    e2p = np.asarray(e2p, dtype=np.int64).reshape(T, k)
    out = np.zeros((T, y_rows.shape[1]))
    for s in range(k):
        p = e2p[:, s]
        ok = p >= 0
        out[ok] += w[ok, s:s + 1] * y_rows[p[ok]]
    return out


# ---------------------------------------------------------------------------
# MX formats -- W4A8 page, "Inputs": x float8_e4m3fn with UE8M0 block-32 scale
# codes; MXFP4 w1/w2 (two e2m1 codes per byte) with UE8M0 block-32 scales.
# Element formats follow the OCP Microscaling specification.
# ---------------------------------------------------------------------------
def minifloat_decode(codes, ebits: int, mbits: int, bias: int, finite_only_nan_code=None):
    """Decode sign|exponent|mantissa minifloat codes to float64 (no inf).

    exponent field 0 is subnormal: m * 2^(1-bias-mbits); otherwise
    (1 + m/2^mbits) * 2^(exp-bias). ``finite_only_nan_code`` (the magnitude
    bits that encode NaN, if any) decodes to NaN.
    """
    c = np.asarray(codes, dtype=np.int64)
    nb = ebits + mbits
    mag_bits = c & ((1 << nb) - 1)
    sign = np.where((c >> nb) & 1, -1.0, 1.0)
    ex = mag_bits >> mbits
    man = mag_bits & ((1 << mbits) - 1)
    sub = man.astype(np.float64) * 2.0 ** (1 - bias - mbits)
    nrm = (1.0 + man / float(1 << mbits)) * np.exp2((ex - bias).astype(np.float64))
    v = sign * np.where(ex == 0, sub, nrm)
    if finite_only_nan_code is not None:
        v = np.where(mag_bits == finite_only_nan_code, np.nan, v)
    return v


def e4m3_decode(codes):
    """OCP float8 e4m3fn: bias 7, no inf, S.1111.111 is NaN, max 448."""
    return minifloat_decode(codes, 4, 3, 7, finite_only_nan_code=0x7F)


def e2m1_decode(codes):
    """OCP fp4 e2m1: bias 1, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, no inf/NaN."""
    return minifloat_decode(codes, 2, 1, 1)


def ue8m0_decode(codes):
    """UE8M0 scale code c -> 2^(c-127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2((c - 127).astype(np.float64)))


def e4m3_encode(v):
    """float -> e4m3fn code, round to nearest, ties to even. |v| must be <= 448
    (larger magnitudes are rejected: the requantization never produces them)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > 448.0) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode: |v| > 448 or NaN")
    # exponent of the binade, floored at the subnormal exponent (1 - bias = -6)
    with np.errstate(divide="ignore"):
        ex = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))), -6.0)
    ex = np.maximum(ex, -6.0)
    step = np.exp2(ex - 3.0)                  # 3 mantissa bits
    q = np.round(a / step) * step             # np.round: half to even
    # q is representable; turn it back into fields
    with np.errstate(divide="ignore"):
        qe = np.where(q > 0, np.floor(np.log2(np.where(q > 0, q, 1.0))), -7.0)
    normal = qe >= -6.0
    exp_field = np.where(normal, qe + 7.0, 0.0).astype(np.int64)
    man_field = np.where(normal, q / np.exp2(qe) * 8.0 - 8.0, q / 2.0 ** -9).astype(np.int64)
    code = (exp_field << 3) | man_field
    code = np.where(np.signbit(v) & (q > 0), code | 0x80, code)
    return code.astype(np.uint8)


def mx_dequant(codes_value, scale_codes, block: int = 32):
    """Block-scaled values: v[..., j] = elem[..., j] * 2^(scale[..., j // block] - 127).
    ``codes_value`` holds already-decoded element values (float)."""
    vals = np.asarray(codes_value, dtype=np.float64)
    sc = ue8m0_decode(scale_codes)
    return vals * np.repeat(sc, block, axis=-1)[..., :vals.shape[-1]]


def requant_e4m3(a32, block: int = 32):
    """MXFP8 requantization with UE8M0 round-up (W4A8 page, intro).

    Per row and per block of 32 along the last axis: e is the smallest integer
    with amax <= 448 * 2^e (an all-zero block takes scale code 0); elements
    become RNE_e4m3(a * 2^-e). The decision is taken on the float32 values
    given. Returns (decoded element values float64, scale codes uint8).
    """
    a = np.asarray(a32, dtype=np.float32).astype(np.float64)
    *lead, n = a.shape
    if n % block:
        raise ValueError("last dim must be a multiple of the block")
    ab = a.reshape(*lead, n // block, block)
    amax = np.abs(ab).max(axis=-1)
    e = np.zeros(amax.shape)
    nz = amax > 0
    # smallest integer e with amax <= 448 * 2^e, checked exactly around log2
    e0 = np.ceil(np.log2(np.where(nz, amax, 1.0) / 448.0))
    e0 = np.where(amax > 448.0 * np.exp2(e0), e0 + 1, e0)
    e0 = np.where(amax <= 448.0 * np.exp2(e0 - 1), e0 - 1, e0)
    e = np.where(nz, e0, 0.0)
    codes_scale = np.where(nz, np.clip(e + 127, 0, 254), 0).astype(np.uint8)
    scale_used = np.exp2(codes_scale.astype(np.float64) - 127.0)
    q = e4m3_encode(ab / scale_used[..., None])
    vals = e4m3_decode(q).reshape(*lead, n)
    return vals, codes_scale


def unpack_e2m1(packed):
    """Two e2m1 codes per byte, element 2j in the low nibble, 2j+1 in the high one
    (W4A8 page, "Inputs": w1 [L, 2I, H/2] packs two values per byte)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def mx_dequant_fp4(packed, scale_codes, block: int = 32):
    """MXFP4 -> float64: e2m1 element value times 2^(scale - 127) per block of 32."""
    return mx_dequant(e2m1_decode(unpack_e2m1(packed)), scale_codes, block)


def mx_dequant_fp8(codes, scale_codes, block: int = 32):
    """MXFP8 (e4m3fn codes) -> float64 with UE8M0 block-32 scales."""
    return mx_dequant(e4m3_decode(codes), scale_codes, block)


# ---------------------------------------------------------------------------
# fp8 with per-tensor scales -- StepFun page, intro (the "fp8 (per-tensor)"
# weight family). The pages give no layout; the reading taken: e4m3fn codes, one
# float32 scale per tensor (x, the FC1 output) or per expert matrix (w1[e], w2[e]).
# ---------------------------------------------------------------------------
def fp8_dequant(codes, scale):
    """value = e4m3fn code value * scale; ``scale`` broadcasts against the leading
    axes (a scalar, or one value per expert for a [L, rows, cols] bank)."""
    v = e4m3_decode(codes)
    sc = np.asarray(scale, dtype=np.float64)
    return v * sc.reshape(sc.shape + (1,) * (v.ndim - sc.ndim))


def requant_e4m3_per_tensor(a32, scale):
    """Per-tensor fp8 requantization of float32 values with a static scale:
    code = RNE_e4m3(clamp(a * r, -448, 448)) where r = float32(1 / scale) and the
    product is rounded to float32 (the decision is taken in float32); saturating,
    since a static scale need not fit the data. Returns (code value * scale as
    float64, codes uint8)."""
    a = np.asarray(a32, dtype=np.float32)
    s32 = np.float32(scale)
    r = np.float32(1.0) / s32
    y = np.clip((a * r).astype(np.float32), np.float32(-448.0), np.float32(448.0))
    codes = e4m3_encode(y.astype(np.float64))
    return e4m3_decode(codes) * float(s32), codes


# ---------------------------------------------------------------------------
# Backward of the layer -- grouped-GEMM page, operation table and Autograd
# section: the backward of each grouped product is its dgrad (dX = G W) and its
# wgrad (dW = G^T X, exactly zero for an empty group). The rest is the chain rule
# through the forward formula of the SM90 fused-MoE page and the activation; the
# clamp of SwiGLUStep passes the gradient where min <= v <= max (a reading: the
# pages give no backward).
# ---------------------------------------------------------------------------
def activation_backward(h, da, kind: str, limit: float = 7.0):
    """dh [..., 2I] = d activation(h) / d h applied to da [..., I] (h = [up | gate]).

    swiglu:      du = da * silu(g),  dg = da * u * silu'(g),
                 silu'(g) = s (1 + g (1 - s)) with s = 1 / (1 + exp(-g))
    swiglu_step: the same at the clamped values, times [-L <= u <= L] for du and
                 [-L <= g <= L] for dg
    """
    h = np.asarray(h, dtype=np.float64)
    da = np.asarray(da, dtype=np.float64)
    I = h.shape[-1] // 2
    u, g = h[..., :I], h[..., I:]
    mu = np.ones_like(u)
    mg = np.ones_like(g)
    if kind == "swiglu_step":
        mu = ((u >= -limit) & (u <= limit)).astype(np.float64)
        mg = ((g >= -limit) & (g <= limit)).astype(np.float64)
        u, g = np.clip(u, -limit, limit), np.clip(g, -limit, limit)
    elif kind != "swiglu":
        raise ValueError(kind)
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-g))
    du = da * g * sg * mu
    dg = da * u * sg * (1.0 + g * (1.0 - sg)) * mg
    return np.concatenate([du, dg], axis=-1)


def moe_backward(x, topk_ids, topk_weights, w1, w2, dout, *, num_experts, local_offset=0,
                 activation_kind="swiglu", limits=None):
    """Gradients of moe_forward (same arguments) for an upstream gradient dout [T, H]:
    returns (dx [T, H], dw1 [L, 2I, H], dw2 [L, H, I], dtopk_weights [T, k]), float64.

    For a route (t, s) to local expert e, with h = x[t] @ w1[e].T, a = act(h),
    y = a @ w2[e].T:  dtopk_weights[t, s] = <dout[t], y>;  dy = w[t, s] dout[t];
    dw2[e] += dy^T a;  da = dy @ w2[e];  dh = act'(h) da;  dw1[e] += dh^T x[t];
    dx[t] += dh @ w1[e]. Foreign routes contribute nothing (their weight gradient
    is 0), and an expert without routes gets exactly zero weight gradients.
    """
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    w = np.asarray(topk_weights, dtype=np.float64)
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    L = w1.shape[0]
    loc = local_expert(ids, num_experts, L, local_offset).reshape(T, k)
    dx = np.zeros_like(x)
    dw1 = np.zeros((L,) + tuple(w1.shape[1:]))
    dw2 = np.zeros((L,) + tuple(w2.shape[1:]))
    dwt = np.zeros((T, k))
    for e in range(L):
        tt, ss = np.nonzero(loc == e)
        if tt.size == 0:
            continue
        w1e = np.asarray(w1[e], dtype=np.float64)
        w2e = np.asarray(w2[e], dtype=np.float64)
        lim = 7.0 if limits is None else float(limits[e])
        h = x[tt] @ w1e.T
        a = activation(h, activation_kind, lim)
        y = a @ w2e.T
        dwt[tt, ss] = np.sum(dout[tt] * y, axis=1)
        dy = w[tt, ss][:, None] * dout[tt]
        dw2[e] = dy.T @ a
        dh = activation_backward(h, dy @ w2e, activation_kind, lim)
        dw1[e] = dh.T @ x[tt]
        np.add.at(dx, tt, dh @ w1e)
    return dx, dw1, dw2, dwt


def route_backward(topk_ids, topk_weights, dtopk_weights, num_experts: int):
    """Gradient of the routing logits through the Renormalize weights (StepFun page,
    intro): w = softmax over the k selected logits, so for a selected expert j at
    slot s, dlogits[t, j] = w[t, s] (dw[t, s] - sum_r w[t, r] dw[t, r]); the
    selection itself is piecewise constant, so unselected logits get 0."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=np.float64)
    dw = np.asarray(dtopk_weights, dtype=np.float64)
    T, k = ids.shape
    dl = np.zeros((T, num_experts))
    inner = np.sum(w * dw, axis=1, keepdims=True)
    g = w * (dw - inner)
    for s in range(k):
        dl[np.arange(T), ids[:, s]] += g[:, s]
    return dl


# ---------------------------------------------------------------------------
# BGMV MoE-LoRA -- "flashinfer.fused_moe.prepare_bgmv_moe" page (the BGMV page):
# signature and Parameters (x [T, H]; one LoRA slice with A [num_loras, E, rank, H]
# and B [num_loras, E, feat_out, rank]; per routed pair a token index, an expert
# index and an FP32 routing weight; a LoRA index per token; shrink output of shape
# [num_pairs, rank] in the weight dtype; FP32 output accumulator [T, feat_out]) and
# the description (each output accumulates its routes in fixed input order).
# Readings: the output is written, not added onto earlier contents; a pair whose
# token, expert or LoRA index is out of range contributes zero.
# ---------------------------------------------------------------------------
def _bgmv_valid(sorted_token_ids, expert_ids, lora_indices, num_tokens, num_experts, num_loras):
    t = np.asarray(sorted_token_ids, dtype=np.int64)
    e = np.asarray(expert_ids, dtype=np.int64)
    li = np.asarray(lora_indices, dtype=np.int64)
    ok = (t >= 0) & (t < num_tokens) & (e >= 0) & (e < num_experts)
    lp = np.where(ok, li[np.clip(t, 0, max(num_tokens - 1, 0))] if num_tokens else -1, -1)
    ok &= (lp >= 0) & (lp < num_loras)
    return t, e, lp, ok


def bgmv_shrink(x, lora_a, sorted_token_ids, expert_ids, lora_indices, shrink_dtype=None):
    """shrink[p, :] = x[t_p] @ lora_a[l, e_p].T with t_p = sorted_token_ids[p],
    l = lora_indices[t_p] (float64; rows of invalid pairs are 0). shrink_dtype="bf16"
    rounds the result to bfloat16 (nearest even), the dtype the page gives the shrink
    output when the weights are bf16."""
    x = np.asarray(x, dtype=np.float64)
    A = lora_a
    num_loras, E, r, H = A.shape
    t, e, l, ok = _bgmv_valid(sorted_token_ids, expert_ids, lora_indices, x.shape[0], E, num_loras)
    out = np.zeros((t.shape[0], r))
    for p in np.nonzero(ok)[0]:
        out[p] = np.asarray(A[l[p], e[p]], dtype=np.float64) @ x[t[p]]
    if shrink_dtype == "bf16":
        import torch
        out = torch.from_numpy(out).to(torch.bfloat16).to(torch.float64).numpy()
    elif shrink_dtype is not None:
        raise ValueError(shrink_dtype)
    return out


def bgmv_expand(shrink, lora_b, sorted_token_ids, expert_ids, lora_indices, topk_weights,
                num_tokens):
    """y[t, :] = sum over the pairs p of token t, ascending p, of
    topk_weights[p] * (shrink[p] @ lora_b[l, e_p].T) (float64; tokens without a valid
    pair get 0)."""
    s = np.asarray(shrink, dtype=np.float64)
    B = lora_b
    num_loras, E, N, r = B.shape
    t, e, l, ok = _bgmv_valid(sorted_token_ids, expert_ids, lora_indices, num_tokens, E, num_loras)
    w = np.asarray(topk_weights, dtype=np.float64)
    y = np.zeros((num_tokens, N))
    for p in np.nonzero(ok)[0]:        # ascending pair index
        y[t[p]] += w[p] * (np.asarray(B[l[p], e[p]], dtype=np.float64) @ s[p])
    return y


def bgmv_moe(x, lora_a, lora_b, sorted_token_ids, expert_ids, lora_indices, topk_weights,
             shrink_dtype=None):
    """Shrink then expand; returns (y [T, feat_out], shrink [num_pairs, rank])."""
    s = bgmv_shrink(x, lora_a, sorted_token_ids, expert_ids, lora_indices, shrink_dtype)
    y = bgmv_expand(s, lora_b, sorted_token_ids, expert_ids, lora_indices, topk_weights,
                    np.asarray(x).shape[0])
    return y, s
