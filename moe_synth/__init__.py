"""Seeded synthetic inputs for the routed-MoE expert layer.

This module is shared by the tests, the benchmark and the CPU oracle's
callers. It draws random numbers and casts them to the storage dtypes; it
holds none of the layer's arithmetic (no routing, sorting, products,
activations or combines).

Conventions
-----------
* ``N(0, v)`` means mean 0 and *variance* v, so weights of fan-in ``f`` are
  drawn with standard deviation ``sqrt(1/f)``.
* Every draw is float32 from ``numpy.random.default_rng``; bf16 tensors are
  the round-to-nearest-even cast done by ``torch.Tensor.to(torch.bfloat16)``.
* Routing logits, the per-expert logit bias, ``x`` and the clamp limits come
  from one generator seeded with ``seed``, drawn in that order. Expert ``e``'s
  rows of ``w1`` and ``w2`` come from generators seeded with
  ``[seed, 1, e]`` and ``[seed, 2, e]``, so banks of any size are drawn
  expert by expert (and in parallel) without holding an fp32 copy of the bank.
* The MX (MXFP8 / MXFP4) encoders here produce *inputs* only: block scales are
  powers of two chosen so the block maximum fits the element format, and the
  elements are rounded to nearest, ties to even. The per-tensor fp8 encoder
  takes scale = amax / 448 (float32) for the whole tensor (x) or expert matrix
  (w1[e], w2[e]); the static scale of the requantized FC1 output is a case
  parameter, not derived from any layer output.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = [
    "MoECase", "GroupedGemmCase", "moe_case", "tiny_moe", "mixtral_moe",
    "expert_shard_moe", "grouped_gemm_case", "dirichlet_group_sizes",
    "route_logits", "bf16_to_f32", "to_bf16", "mx_quant_e4m3", "mx_quant_e2m1", "W4A8Case",
    "w4a8_moe", "fp8_quant_per_tensor", "FP8_ACT_SCALE", "upstream_grad", "BgmvCase",
    "bgmv_case",
]

_THREADS = max(1, min(16, os.cpu_count() or 1))


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 numpy array -> bf16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_to_f32(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> fp32 numpy array; the widening is exact."""
    return t.detach().to("cpu", torch.float32).numpy()


def _normal_bank(shape, std: float, seed: int, stream: int) -> torch.Tensor:
    """bf16 bank [E, rows, cols]; expert e drawn from default_rng([seed, stream, e])."""
    E = shape[0]
    out = torch.empty(shape, dtype=torch.bfloat16)

    def fill(e: int) -> None:
        g = np.random.default_rng([seed, stream, e])
        a = g.standard_normal(shape[1:], dtype=np.float32)
        a *= np.float32(std)
        out[e].copy_(torch.from_numpy(a).to(torch.bfloat16))

    if E == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=min(_THREADS, E)) as ex:
            list(ex.map(fill, range(E)))
    return out


@dataclass
class MoECase:
    """One synthetic MoE-forward problem.

    logits:  float32 [T, E_g] router logits (per-expert bias already added)
    x:       bf16 [T, H]
    w1:      bf16 [L, 2I, H]; rows 0..I-1 are the up projection, I..2I-1 the gate
    w2:      bf16 [L, H, I]
    limits:  float32 [L] clamp limits for SwiGLUStep, or None
    """
    name: str
    T: int
    H: int
    I: int
    num_experts: int
    num_local: int
    local_offset: int
    top_k: int
    activation: str  # "swiglu" | "swiglu_step"
    logits: np.ndarray
    x: torch.Tensor
    w1: torch.Tensor
    w2: torch.Tensor
    limits: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)


def route_logits(g: np.random.Generator, T: int, E: int, bias_var: float = 0.0) -> np.ndarray:
    """logits ~ N(0,1) [T,E] float32, plus a per-expert bias ~ N(0, bias_var) if bias_var > 0."""
    logits = g.standard_normal((T, E), dtype=np.float32)
    if bias_var > 0.0:
        bias = g.standard_normal((E,), dtype=np.float32) * np.float32(math.sqrt(bias_var))
        logits = logits + bias[None, :]
    return np.ascontiguousarray(logits, dtype=np.float32)


def moe_case(name: str, T: int, H: int, I: int, num_experts: int, top_k: int, *,
             num_local: Optional[int] = None, local_offset: int = 0,
             activation: str = "swiglu", bias_var: float = 0.0, x_scale: float = 1.0,
             limit_range: Optional[tuple] = None, seed: int = 0,
             with_weights: bool = True) -> MoECase:
    """Generic MoE forward case; draw order logits -> bias -> x -> limits, then weights."""
    L = num_experts if num_local is None else num_local
    g = np.random.default_rng(seed)
    logits = route_logits(g, T, num_experts, bias_var)
    xa = g.standard_normal((T, H), dtype=np.float32)
    if x_scale != 1.0:
        xa *= np.float32(x_scale)
    x = to_bf16(xa)
    limits = None
    if limit_range is not None:
        lo, hi = limit_range
        limits = g.uniform(lo, hi, size=(L,)).astype(np.float32)
    if with_weights:
        w1 = _normal_bank((L, 2 * I, H), math.sqrt(1.0 / H), seed, 1)
        w2 = _normal_bank((L, H, I), math.sqrt(1.0 / I), seed, 2)
    else:
        w1 = torch.empty((0,), dtype=torch.bfloat16)
        w2 = torch.empty((0,), dtype=torch.bfloat16)
    return MoECase(name, T, H, I, num_experts, L, local_offset, top_k, activation,
                   logits, x, w1, w2, limits,
                   meta=dict(seed=seed, bias_var=bias_var, x_scale=x_scale,
                             limit_range=limit_range))


def tiny_moe(seed: int = 0) -> MoECase:
    """Tiny bf16 forward: T=32, H=128, I=256, E=8, top-2, SwiGLU."""
    return moe_case("tiny", 32, 128, 256, 8, 2, seed=seed)


def mixtral_moe(seed: int = 0, T: int = 4096, with_weights: bool = True) -> MoECase:
    """Mixtral-shaped forward: H=4096, I=14336, E=8, top-2, SwiGLU, logit bias N(0, 0.5)."""
    return moe_case("mixtral", T, 4096, 14336, 8, 2, bias_var=0.5, seed=seed,
                    with_weights=with_weights)


def expert_shard_moe(seed: int = 0, T: int = 8192, clamp_active: bool = False,
                     with_weights: bool = True) -> MoECase:
    """Fine-grained expert shard: H=7168, I=2048, 256 experts, 32 local from id 64,
    top-8, SwiGLUStep with per-expert limits ~ U[5, 9]. ``clamp_active`` scales x
    by 8 so that the clamp fires on a large share of the pre-activations."""
    return moe_case("expert_shard", T, 7168, 2048, 256, 8, num_local=32, local_offset=64,
                    activation="swiglu_step", x_scale=8.0 if clamp_active else 1.0,
                    limit_range=(5.0, 9.0), seed=seed, with_weights=with_weights)


def upstream_grad(seed: int, T: int, H: int, scale: float = 1.0) -> torch.Tensor:
    """Upstream gradient d loss / d out for the backward: bf16 [T, H], N(0, scale^2), drawn
    from default_rng([seed, 3]) (a stream of its own, so the forward case is unchanged)."""
    g = np.random.default_rng([seed, 3])
    a = g.standard_normal((T, H), dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return to_bf16(a)


def dirichlet_group_sizes(E: int = 16, total: int = 8192, alpha: float = 0.3,
                          seed: int = 0, tile: int = 64) -> np.ndarray:
    """Imbalanced group sizes that include one empty group, one 1-row group and no
    other size that is a multiple of ``tile``.

    1. p ~ Dirichlet(alpha), m = floor(total * p).
    2. The group with the smallest p gets 0 rows, the next smallest gets 1.
    3. Every other group gets at least 2 rows, and +1 if its size is a tile multiple.
    4. The remainder goes to the largest group; if that lands on a tile multiple,
       one row moves to the second largest.
    """
    g = np.random.default_rng(seed)
    p = g.dirichlet(np.full(E, alpha))
    m = np.floor(total * p).astype(np.int64)
    order = np.argsort(p, kind="stable")
    m[order[0]] = 0
    m[order[1]] = 1
    for e in order[2:]:
        m[e] = max(m[e], 2)
        if m[e] % tile == 0:
            m[e] += 1
    big, second = order[-1], order[-2]
    m[big] += total - int(m.sum())
    if m[big] % tile == 0:
        m[big] -= 1
        m[second] += 1
        if m[second] % tile == 0:
            m[second] += 1
            m[big] -= 1
    assert int(m.sum()) == total and m.min() >= 0
    return m.astype(np.int32)


@dataclass
class GroupedGemmCase:
    """Ragged grouped GEMM problem: groups are consecutive row ranges of X and G.

    sizes: int32 [E]; offs: int32 [E] cumulative ends
    x: bf16 [sum_m, K]; g: bf16 [sum_m, N]; w: bf16 [E, N, K]
    """
    sizes: np.ndarray
    offs: np.ndarray
    x: torch.Tensor
    g: torch.Tensor
    w: torch.Tensor

    @property
    def E(self) -> int:
        return int(self.sizes.shape[0])

    @property
    def sum_m(self) -> int:
        return int(self.offs[-1]) if self.offs.size else 0


def grouped_gemm_case(seed: int = 0, E: int = 16, sum_m: int = 8192, K: int = 2048,
                      N: int = 4096, sizes: Optional[np.ndarray] = None,
                      integer_valued: bool = False) -> GroupedGemmCase:
    """Ragged bf16 grouped GEMM inputs. X, G ~ N(0,1); W ~ N(0, 1/K).

    With ``integer_valued`` every operand is an integer in [-3, 3] (exact in
    bf16), so every fp32 partial sum is an exact integer at these sizes.
    """
    if sizes is None:
        sizes = dirichlet_group_sizes(E, sum_m, seed=seed)
    sizes = np.asarray(sizes, dtype=np.int32)
    offs = np.cumsum(sizes).astype(np.int32)
    M = int(offs[-1]) if offs.size else 0
    g = np.random.default_rng([seed, 7])
    if integer_valued:
        x = torch.from_numpy(g.integers(-3, 4, size=(M, K)).astype(np.float32)).to(torch.bfloat16)
        gg = torch.from_numpy(g.integers(-3, 4, size=(M, N)).astype(np.float32)).to(torch.bfloat16)
        w = torch.from_numpy(g.integers(-3, 4, size=(len(sizes), N, K)).astype(np.float32)).to(torch.bfloat16)
    else:
        x = to_bf16(g.standard_normal((M, K), dtype=np.float32))
        gg = to_bf16(g.standard_normal((M, N), dtype=np.float32))
        w = _normal_bank((len(sizes), N, K), math.sqrt(1.0 / K), seed, 3)
    return GroupedGemmCase(sizes, offs, x, gg, w)


# ---------------------------------------------------------------------------
# MX inputs (MXFP8 activations, MXFP4 weights) with UE8M0 block-32 scales.
# Scale exponent of a block: the smallest e with amax <= elem_max * 2^e (so the
# scaled block fits the element format); elements rounded to nearest, ties even.
# ---------------------------------------------------------------------------
def _block_exponent(amax: np.ndarray, elem_max: float) -> np.ndarray:
    """smallest integer e with amax <= elem_max * 2^e (amax > 0), checked exactly."""
    e = np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / elem_max))
    e = np.where(amax > elem_max * np.exp2(e), e + 1, e)
    e = np.where(amax <= elem_max * np.exp2(e - 1), e - 1, e)
    return np.where(amax > 0, e, -127.0)


def _block_scales(a: np.ndarray, elem_max: float, block: int):
    *lead, K = a.shape
    ab = a.reshape(*lead, K // block, block)
    e = _block_exponent(np.abs(ab).max(-1).astype(np.float64), elem_max)
    sc = np.clip(e + 127, 0, 254).astype(np.uint8)
    # dividing by a power of two is exact in float32 for these magnitudes
    inv = np.exp2(127.0 - sc.astype(np.float64)).astype(np.float32)
    return ab * inv[..., None], sc


def mx_quant_e4m3(a: np.ndarray, block: int = 32):
    """float32 [..., K] -> (e4m3fn codes uint8 [..., K], UE8M0 scales uint8 [..., K/32])."""
    a = np.asarray(a, dtype=np.float32)
    scaled, sc = _block_scales(a, 448.0, block)
    codes = torch.from_numpy(np.ascontiguousarray(scaled.reshape(a.shape))).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, sc


def mx_quant_e2m1(a: np.ndarray, block: int = 32):
    """float32 [..., K] -> (packed e2m1 uint8 [..., K/2] (element 2j in the low nibble),
    UE8M0 scales uint8 [..., K/32]). Magnitudes round to the nearest of
    {0, .5, 1, 1.5, 2, 3, 4, 6}; a value exactly between two takes the even code."""
    a = np.asarray(a, dtype=np.float32)
    scaled, sc = _block_scales(a, 6.0, block)
    m = np.abs(scaled)
    code = ((m > 0.25).astype(np.uint8) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5)
            + (m >= 3.5) + (m > 5.0)).astype(np.uint8)
    code = np.where((scaled < 0) & (code > 0), code | 8, code).astype(np.uint8).reshape(a.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, sc


def fp8_quant_per_tensor(a: np.ndarray):
    """float32 array -> (e4m3fn codes uint8, float32 scale) with scale = amax / 448
    (1.0 for an all-zero array); codes are torch's RNE cast of a / scale in float32."""
    a = np.asarray(a, dtype=np.float32)
    amax = float(np.abs(a).max()) if a.size else 0.0
    sc = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    codes = torch.from_numpy(np.ascontiguousarray(a / sc)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    return codes, sc


# Static FC1-output scale of the per-tensor fp8 cases: codes reach 448 * 0.0357 = 16,
# about 4 sigma of silu(gate) * up for unit-variance pre-activations; deliberately
# not a power of two, so that the float32 reciprocal matters.
FP8_ACT_SCALE = 0.0357


@dataclass
class W4A8Case:
    """MXFP8-activation / MX-weight MoE case (numpy arrays on the host).

    x, x_sf:   uint8 [T, H] e4m3fn codes, uint8 [T, H/32] UE8M0
    w1, w1_sf: uint8 [L, 2I, H/2] packed e2m1 (wfmt "mxfp4") or [L, 2I, H] e4m3fn codes
               (wfmt "mxfp8"), [up | gate] rows; uint8 [L, 2I, H/32]
    w2, w2_sf: uint8 [L, H, I/2] or [L, H, I], uint8 [L, H, I/32]
    wfmt "fp8" (per-tensor): x, w1, w2 e4m3fn codes as for "mxfp8"; x_sf float32 [1],
               w1_sf / w2_sf float32 [L]; act_scale float32 [1] (FC1 output scale)
    """
    T: int
    H: int
    I: int
    num_experts: int
    top_k: int
    logits: np.ndarray
    x: np.ndarray
    x_sf: np.ndarray
    w1: np.ndarray
    w1_sf: np.ndarray
    w2: np.ndarray
    w2_sf: np.ndarray
    wfmt: str = "mxfp4"
    act_scale: Optional[np.ndarray] = None

    @property
    def num_local(self) -> int:
        return self.num_experts


def w4a8_moe(seed: int = 0, T: int = 8192, H: int = 7168, I: int = 2048, E: int = 64,
             top_k: int = 8, x_scale: float = 1.0, wfmt: str = "mxfp4") -> W4A8Case:
    """fp8-activation MoE: logits N(0,1); x N(0,1); w1 N(0,1/H), w2 N(0,1/I), quantized
    expert by expert (draw order as in moe_case) to MXFP4 (wfmt "mxfp4", the W4A8 case;
    x MXFP8), MXFP8 (wfmt "mxfp8"; x MXFP8) or per-tensor fp8 (wfmt "fp8"; x too, and
    the FC1 output scale is FP8_ACT_SCALE)."""
    if wfmt not in ("mxfp4", "mxfp8", "fp8"):
        raise ValueError(wfmt)
    pt = wfmt == "fp8"
    quant = {"mxfp4": mx_quant_e2m1, "mxfp8": mx_quant_e4m3, "fp8": fp8_quant_per_tensor}[wfmt]
    per = 2 if wfmt == "mxfp4" else 1    # elements per byte
    g = np.random.default_rng(seed)
    logits = route_logits(g, T, E)
    xa = g.standard_normal((T, H), dtype=np.float32)
    if x_scale != 1.0:
        xa *= np.float32(x_scale)
    if pt:
        x, xs = fp8_quant_per_tensor(xa)
        x_sf = np.array([xs], np.float32)
    else:
        x, x_sf = mx_quant_e4m3(xa)
    w1 = np.empty((E, 2 * I, H // per), np.uint8)
    w1_sf = np.empty((E,), np.float32) if pt else np.empty((E, 2 * I, H // 32), np.uint8)
    w2 = np.empty((E, H, I // per), np.uint8)
    w2_sf = np.empty((E,), np.float32) if pt else np.empty((E, H, I // 32), np.uint8)

    def fill(e: int) -> None:
        a = np.random.default_rng([seed, 1, e]).standard_normal((2 * I, H), dtype=np.float32)
        a *= np.float32(math.sqrt(1.0 / H))
        w1[e], w1_sf[e] = quant(a)
        b = np.random.default_rng([seed, 2, e]).standard_normal((H, I), dtype=np.float32)
        b *= np.float32(math.sqrt(1.0 / I))
        w2[e], w2_sf[e] = quant(b)

    with ThreadPoolExecutor(max_workers=min(_THREADS, E)) as ex:
        list(ex.map(fill, range(E)))
    act_scale = np.array([FP8_ACT_SCALE], np.float32) if pt else None
    return W4A8Case(T, H, I, E, top_k, logits, x, x_sf, w1, w1_sf, w2, w2_sf, wfmt, act_scale)


# ---------------------------------------------------------------------------
# BGMV MoE-LoRA inputs: x N(0,1), LoRA-A N(0, 1/H), LoRA-B N(0, 1/rank) (bf16);
# per token top_k distinct experts drawn uniformly and Dirichlet(1) routing weights;
# LoRA index per token uniform in [0, num_loras) (a share of -1 = no adapter if
# asked). Pair order: "contiguous" (p = t * top_k + s), "expert" (stable by expert)
# or "random" (a permutation).
# ---------------------------------------------------------------------------
@dataclass
class BgmvCase:
    x: torch.Tensor            # [T, H] bf16
    lora_a: torch.Tensor       # [num_loras, E, rank, H] bf16
    lora_b: torch.Tensor       # [num_loras, E, feat_out, rank] bf16
    sorted_token_ids: np.ndarray   # [P] int32
    expert_ids: np.ndarray         # [P] int32
    lora_indices: np.ndarray       # [T] int32
    topk_weights: np.ndarray       # [P] float32
    num_experts: int


def bgmv_case(seed: int = 0, T: int = 2048, H: int = 3072, rank: int = 32, num_loras: int = 4,
              E: int = 8, top_k: int = 2, feat_out: Optional[int] = None, order: str = "contiguous",
              no_lora_share: float = 0.0) -> BgmvCase:
    g = np.random.default_rng(seed)
    N = H if feat_out is None else feat_out
    x = to_bf16(g.standard_normal((T, H), dtype=np.float32))
    a = g.standard_normal((num_loras, E, rank, H), dtype=np.float32) * np.float32(math.sqrt(1.0 / H))
    b = g.standard_normal((num_loras, E, N, rank), dtype=np.float32) * np.float32(math.sqrt(1.0 / rank))
    ex = np.stack([g.permutation(E)[:top_k] for _ in range(T)]).astype(np.int32)
    wt = g.dirichlet(np.ones(top_k), size=T).astype(np.float32)
    li = g.integers(0, num_loras, T).astype(np.int32)
    if no_lora_share > 0:
        li[g.random(T) < no_lora_share] = -1
    tok = np.repeat(np.arange(T, dtype=np.int32), top_k)
    ex, wt = ex.reshape(-1), wt.reshape(-1)
    if order == "expert":
        perm = np.argsort(ex, kind="stable")
    elif order == "random":
        perm = g.permutation(tok.shape[0])
    elif order == "contiguous":
        perm = np.arange(tok.shape[0])
    else:
        raise ValueError(order)
    return BgmvCase(x, to_bf16(a), to_bf16(b), tok[perm].copy(), ex[perm].copy(), li,
                    wt[perm].copy(), E)
