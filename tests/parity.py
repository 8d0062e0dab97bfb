"""Comparison helpers shared by the GPU parity tests (test code only).

Besides the fixed tolerances below, two derived bars: `forward_bound` (the
layer output, for inputs whose magnitudes make the fixed bound meaningless)
and `grad_bounds` / `check_grads` (the layer backward), both first-order bounds
per element from the bf16 hand-offs and float32 accumulation of the library.

bf16 tolerance: max-abs 3e-2 and relative L2 1e-2. bf16 itself cannot place a
value of magnitude >= 8 within 3e-2 (its half-ulp there is 2^-5), so the
max-abs bound is applied elementwise to |got - ref| / max(1, |ref|): for
outputs of magnitude up to 1 it is the plain absolute bound.
"""
import numpy as np
import torch

BF16_MAX_ABS = 3e-2
BF16_REL_L2 = 1e-2


def to_np(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy() if t.dtype.is_floating_point \
            else t.detach().cpu().numpy()
    return np.asarray(t)


def bf16_round(a):
    """Round-to-nearest-even bf16 of float64 values (via float32, exact for the
    integer-valued cases this is used on)."""
    return torch.from_numpy(np.asarray(a, np.float64)).to(torch.float32).to(torch.bfloat16) \
        .to(torch.float64).numpy()


def rel_l2(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def assert_close_bf16(got, ref, max_abs=BF16_MAX_ABS, rel=BF16_REL_L2, what=""):
    got, ref = to_np(got), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if got.size == 0:
        return 0.0, 0.0
    scaled = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    err = float(np.max(scaled))
    r = rel_l2(got, ref)
    assert err <= max_abs and r <= rel, \
        f"{what}: max|d|/max(1,|ref|)={err:.3e} (<= {max_abs}), relL2={r:.3e} (<= {rel})"
    return err, r


U_BF16 = 2.0 ** -8        # unit roundoff of bf16 (8 significand bits, nearest even)
U_F32 = 2.0 ** -24        # unit roundoff of float32


def forward_bound(x, topk_ids, topk_weights, w1, w2, *, num_experts, local_offset=0,
                  activation_kind="swiglu", limits=None, fused=False):
    """First-order bound on |out_gpu - out_exact| per element of the bf16 layer output.

    The layer accumulates in float32 and hands act and y over in bf16 (and, fused,
    adds bf16(w * y) into a bf16 output k times). With exact intermediates h, a, y
    (float64 from the bf16 inputs) and n-term float32 sums off by at most
    n 2^-24 of their absolute sums, in any order:
      h error   <= H 2^-24 (|x| @ |w1|^T);
      act error <= sens * (h error) + (2^-8 + 2^-16) |a|, where sens is |silu(g_c)|
                   for the up half and |u_c silu'(g_c)| for the gate half at the
                   clamped values (the clamp is 1-Lipschitz) and 2^-16 covers the
                   hardware exponential / reciprocal of silu;
      y error   <= (act error) @ |w2|^T + I 2^-24 (|a| @ |w2|^T) + 2^-8 |y|;
      out error <= sum_s |w_s| (y error)_s + k 2^-24 S + 2^-8 |out| (deterministic),
                   sum_s |w_s| (y error)_s + 2 k 2^-8 S (fused: every bf16 atomic add
                   rounds its running sum), with S = sum_s |w_s y_s|.
    Returns float64 [T, H]. Test code: reads the oracle's activation only.
    """
    import oracle as O
    x = np.asarray(x, np.float64)
    ids = np.asarray(topk_ids, np.int64)
    w = np.asarray(topk_weights, np.float64)
    T, k = ids.shape
    L, H = w1.shape[0], x.shape[1]
    loc = O.local_expert(ids, num_experts, L, local_offset).reshape(T, k)
    yerr = np.zeros((T, H))
    S = np.zeros((T, H))
    out = np.zeros((T, H))
    ax = np.abs(x)
    for e in range(L):
        tt, ss = np.nonzero(loc == e)
        if tt.size == 0:
            continue
        w1e = np.asarray(w1[e], np.float64)
        w2e = np.asarray(w2[e], np.float64)
        I = w1e.shape[0] // 2
        lim = 7.0 if limits is None else float(limits[e])
        h = x[tt] @ w1e.T
        eh = H * U_F32 * (ax[tt] @ np.abs(w1e).T)
        a = O.activation(h, activation_kind, lim)
        u, g = h[:, :I], h[:, I:]
        if activation_kind == "swiglu_step":
            u, g = np.clip(u, -lim, lim), np.clip(g, -lim, lim)
        sg = 1.0 / (1.0 + np.exp(-g))
        sens_u = np.abs(g * sg)
        sens_g = np.abs(u * sg * (1.0 + g * (1.0 - sg)))
        ea = sens_u * eh[:, :I] + sens_g * eh[:, I:] + (U_BF16 + 2.0 ** -16 + I * U_F32) * np.abs(a)
        y = a @ w2e.T
        ey = ea @ np.abs(w2e).T + U_BF16 * np.abs(y)
        ws = w[tt, ss][:, None]
        np.add.at(yerr, tt, np.abs(ws) * ey)
        np.add.at(S, tt, np.abs(ws * y))
        np.add.at(out, tt, ws * y)
    if fused:
        return yerr + 2 * k * U_BF16 * S
    return yerr + k * U_F32 * S + U_BF16 * np.abs(out)


def assert_within_bound(got, ref, bound, rel=BF16_REL_L2, what=""):
    """|got - ref| <= bound element by element (plus a 1e-30 floor for exact zeros),
    and relative L2 <= rel overall."""
    got, ref = to_np(got), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - ref)
    lim = np.asarray(bound, np.float64) + 1e-30
    bad = d > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the bound, worst "
                           f"{float((d / lim).max()):.3f}x")
    r = rel_l2(got, ref)
    assert r <= rel, f"{what}: relative L2 {r:.3e} (<= {rel})"
    return float((d / lim).max()), r


def grad_bounds(c, ids, w, dout):
    """First-order error bounds of (dx, dw1, dw2, dtopk_weights) from the bf16 hand-offs,
    from absolute values of the exact intermediates (float32 accumulation over a length n
    adds n 2^-24 of the absolute sum)."""
    import moe_synth as S
    import oracle as O
    x, w1, w2 = (S.bf16_to_f32(t).astype(np.float64) for t in (c.x, c.w1, c.w2))
    ids = ids.cpu().numpy()
    w = w.cpu().numpy().astype(np.float64)
    dout = S.bf16_to_f32(dout).astype(np.float64)
    T, k = ids.shape
    L, H = w1.shape[0], x.shape[1]
    loc = O.local_expert(ids, c.num_experts, L, c.local_offset).reshape(T, k)
    bx, bw1, bw2 = np.zeros_like(x), np.zeros_like(w1), np.zeros_like(w2)
    bdw = np.zeros((T, k))
    ax = np.abs(x)
    for e in range(L):
        tt, ss = np.nonzero(loc == e)
        if tt.size == 0:
            continue
        lim = 7.0 if c.limits is None else float(c.limits[e])
        h = x[tt] @ w1[e].T
        a = O.activation(h, c.activation, lim)
        y = a @ w2[e].T
        dy = w[tt, ss][:, None] * dout[tt]
        da = dy @ w2[e]
        dh = O.activation_backward(h, da, c.activation, lim)
        # d dh / d da (dh is linear in da), applied to the error of da
        sens = np.abs(O.activation_backward(h, np.ones_like(da), c.activation, lim))
        eda = (U_BF16 + H * 2.0 ** -24) * (np.abs(dy) @ np.abs(w2[e]))
        bdh = sens * np.concatenate([eda, eda], axis=1) + U_BF16 * np.abs(dh)
        bw1[e] = bdh.T @ ax[tt] + U_BF16 * np.abs(dh.T @ x[tt])
        bw2[e] = 2 * U_BF16 * (np.abs(dy).T @ np.abs(a)) + U_BF16 * np.abs(dy.T @ a)
        np.add.at(bx, tt, bdh @ np.abs(w1[e]) + U_BF16 * np.abs(dh @ w1[e]))
        bdw[tt, ss] = (U_BF16 + H * 2.0 ** -24) * np.sum(np.abs(dout[tt]) * np.abs(y), axis=1)
    return bx, bw1, bw2, bdw


def check_grads(grads, ref, bounds, what):
    for name, g, r, b in zip(("dx", "dw1", "dw2", "dtopk_weights"), grads, ref, bounds):
        g = to_np(g).astype(np.float64)
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        d = np.abs(g - r)
        # the output's own rounding, and a floor for elements whose bound is 0
        lim = b + U_BF16 * np.abs(r) + 1e-30
        bad = d > lim
        assert not bad.any(), (f"{what} {name}: {bad.sum()} elements beyond the bound, worst "
                               f"{(d / lim).max():.3f}x")
        rl = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
        assert rl <= 1e-2, f"{what} {name}: relative L2 {rl:.3e}"


def mx_dequant_table(wfmt, codes, scales):
    """The oracle's MX dequantization (O.mx_dequant_fp4 / O.mx_dequant_fp8) computed
    through lookup tables of the oracle's own element and scale decoders over every
    code: the same float64 values (pinned by a CPU test), an order of magnitude faster
    on a full expert matrix."""
    import oracle as O
    tabs = _MX_TABLES.get("t")
    if tabs is None:
        tabs = _MX_TABLES["t"] = (O.e2m1_decode(np.arange(16)), O.e4m3_decode(np.arange(256)),
                                  O.ue8m0_decode(np.arange(256)))
    e2m1, e4m3, ue8m0 = tabs
    if wfmt == "mxfp4":
        elem = e2m1[O.unpack_e2m1(codes)]
    elif wfmt == "mxfp8":
        elem = e4m3[np.asarray(codes, np.uint8)]
    else:
        raise ValueError(wfmt)
    return elem * np.repeat(ue8m0[np.asarray(scales, np.uint8)], 32, axis=-1)


_MX_TABLES = {}
