"""MI355X (gfx950) routed Mixture-of-Experts expert layer.

A thin ctypes binding over the HIP library ``libmoe_mi355x.so`` (built from
``csrc/`` by ``_build.py``). Every function here only marshals arguments:
PyTorch tensors provide device memory and the current HIP stream, and every
step of the computation runs in the library's kernels. If the library is
missing the functions raise; there is no fallback.

Entry points (same names as the C ABI in include/moe.h):
``moe_route``, ``moe_sort``, ``grouped_gemm_fwd``, ``grouped_gemm_dgrad``,
``grouped_gemm_wgrad``, ``moe_ffn_forward``, ``moe_finalize``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "MoeError", "lib", "library_path", "EXPORTS", "moe_route", "moe_sort", "grouped_gemm_fwd",
    "grouped_gemm_dgrad", "grouped_gemm_wgrad", "moe_ffn_forward", "moe_ffn_workspace_size",
    "moe_finalize", "moe_fc1", "moe_fc2", "status_string", "ACT", "FINALIZE", "WFMT",
    "moe_ffn_forward_mx", "moe_fc1_mx", "moe_fc2_mx", "moe_ffn_forward_fp8", "moe_fc1_fp8",
    "moe_fc2_fp8", "moe_ffn_forward_train", "moe_ffn_backward", "moe_route_backward", "MoEFunction",
    "moe_tune", "moe_tune_set", "moe_tune_clear", "moe_bgmv", "moe_bgmv_workspace_bytes",
    "moe_ffn_forward_noalloc", "NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmoe_mi355x.so")

ACT = {"swiglu": 0, "swiglu_step": 1}
FINALIZE = {"deterministic": 0, "fused": 1, "none": 2}
OFFS = {"ends": 0, "indptr": 1}
DTYPE = {torch.bfloat16: 0, torch.float32: 1}

_i32, _i64, _u64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
_sz = ctypes.c_size_t


WFMT = {"bf16": 0, "mxfp4": 1, "mxfp8": 2, "fp8": 3}
NOALLOC_SCRATCH_BYTES = 128 << 20   # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h


class MoeFfnDesc(ctypes.Structure):
    _fields_ = [("T", _i64), ("H", _i32), ("I", _i32), ("num_experts", _i32),
                ("num_local_experts", _i32), ("local_expert_offset", _i32), ("top_k", _i32),
                ("activation", _i32), ("finalize_mode", _i32), ("weight_format", _i32)]


class MoeFfnTensors(ctypes.Structure):
    _fields_ = [("x", _vp), ("topk_ids", _vp), ("topk_weights", _vp), ("w1", _vp), ("w2", _vp),
                ("clamp_limit", _vp), ("out", _vp), ("y", _vp), ("e2p", _vp),
                ("x_sf", _vp), ("w1_sf", _vp), ("w2_sf", _vp), ("act_scale", _vp)]


class MoeFfnGrads(ctypes.Structure):
    _fields_ = [("dout", _vp), ("dx", _vp), ("dw1", _vp), ("dw2", _vp), ("dtopk_weights", _vp),
                ("grad_dtype", _i32)]


class MoeBgmvDesc(ctypes.Structure):
    _fields_ = [("num_tokens", _i64), ("num_pairs", _i64), ("hidden", _i32), ("feat_out", _i32),
                ("rank", _i32), ("num_loras", _i32), ("num_experts", _i32), ("mode", _i32)]


# name -> (restype, argtypes)
EXPORTS = {
    "moe_status_string": (ctypes.c_char_p, [_i32]),
    "moe_version": (ctypes.c_char_p, []),
    "moe_route": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp, _vp]),
    "moe_sort_workspace_size": (_sz, [_i64, _i32, _i32]),
    "moe_sort": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "grouped_gemm_fwd": (_i32, [_vp, _vp, _vp, _i32, _i32, _i64, _i32, _i32, _vp, _vp, _sz, _vp]),
    "grouped_gemm_dgrad": (_i32, [_vp, _vp, _vp, _i32, _i32, _i64, _i32, _i32, _vp, _vp, _sz, _vp]),
    "grouped_gemm_wgrad_workspace_size": (_sz, [_i32, _i64, _i32, _i32, _i32]),
    "grouped_gemm_wgrad": (_i32, [_vp, _vp, _vp, _i32, _i32, _i64, _i32, _i32, _vp, _i32, _vp, _sz, _vp]),
    "moe_ffn_workspace_size": (_sz, [ctypes.POINTER(MoeFfnDesc)]),
    "moe_ffn_forward": (_i32, [ctypes.POINTER(MoeFfnDesc), ctypes.POINTER(MoeFfnTensors), _vp, _sz, _vp]),
    "moe_ffn_forward_noalloc": (_i32, [ctypes.POINTER(MoeFfnDesc), ctypes.POINTER(MoeFfnTensors), _vp]),
    "moe_finalize": (_i32, [_vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp]),
    "moe_gemm_split_workspace_size": (_sz, []),
    "moe_fc1": (_i32, [ctypes.POINTER(MoeFfnDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_fc2": (_i32, [ctypes.POINTER(MoeFfnDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_fc1_mx": (_i32, [ctypes.POINTER(MoeFfnDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_fc2_mx": (_i32, [ctypes.POINTER(MoeFfnDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_fc1_fp8": (_i32, [ctypes.POINTER(MoeFfnDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_fc2_fp8": (_i32, [ctypes.POINTER(MoeFfnDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_ffn_saved_size": (_sz, [ctypes.POINTER(MoeFfnDesc)]),
    "moe_ffn_forward_train": (_i32, [ctypes.POINTER(MoeFfnDesc), ctypes.POINTER(MoeFfnTensors), _vp,
                                     _sz, _vp]),
    "moe_ffn_backward_workspace_size": (_sz, [ctypes.POINTER(MoeFfnDesc)]),
    "moe_ffn_backward": (_i32, [ctypes.POINTER(MoeFfnDesc), ctypes.POINTER(MoeFfnTensors),
                                ctypes.POINTER(MoeFfnGrads), _vp, _sz, _vp, _sz, _vp]),
    "moe_route_backward": (_i32, [_vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp]),
    "moe_tune": (_i32, [ctypes.POINTER(MoeFfnDesc), ctypes.POINTER(MoeFfnTensors), _vp, _sz, _vp, _vp]),
    "moe_tune_clear": (None, []),
    "moe_tune_set": (_i32, [ctypes.POINTER(MoeFfnDesc), _i32, _i32]),
    "moe_bgmv_workspace_size": (_sz, [ctypes.POINTER(MoeBgmvDesc)]),
    "moe_bgmv": (_i32, [ctypes.POINTER(MoeBgmvDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                        _vp, _sz, _vp]),
}

_LIB: Optional[ctypes.CDLL] = None


class MoeError(RuntimeError):
    """A library call returned a non-zero moe_status."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is missing: build it with "
                              "`python -m mixture_experts_expert_softmax_amd._build`")
        h = ctypes.CDLL(library_path)
        for name, (res, args) in EXPORTS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _LIB = h
    return _LIB


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# --------------------------------------------------------------------------- routing
def moe_route(logits: torch.Tensor, top_k: int, topk_ids=None, topk_weights=None):
    """Renormalized top-k routing: logits [T, E] fp32 -> (ids [T,k] i32, weights [T,k] fp32)."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _check("moe_route", lib().moe_route(_ptr(logits), T, E, top_k, _ptr(topk_ids),
                                        _ptr(topk_weights), _stream()))
    return topk_ids, topk_weights


def moe_sort(topk_ids: torch.Tensor, num_experts: int, num_local_experts: Optional[int] = None,
             local_expert_offset: int = 0, workspace: Optional[torch.Tensor] = None,
             out: Optional[dict] = None):
    """Stable counting sort by local expert. Returns a dict of device tensors:
    offs [L], m_indptr [L+1], e2p [T*k], p2e [T*k] (valid below n_local), n_local [1].
    ``out`` may hold preallocated int32 tensors under those names (as returned by an
    earlier call with the same shape); they are written in place."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    L = num_experts if num_local_experts is None else num_local_experts
    dev = topk_ids.device
    h = lib()
    ws_bytes = h.moe_sort_workspace_size(T, k, L)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    need = dict(offs=L, m_indptr=L + 1, e2p=T * k, p2e=T * k, n_local=1)   # elements written
    if out is None:
        out = {n: torch.empty(max(sz, 1), dtype=torch.int32, device=dev) for n, sz in need.items()}
    else:
        for n, sz in need.items():
            t = out[n]
            if t.numel() < sz or t.dtype != torch.int32 or t.device != dev or not t.is_contiguous():
                raise ValueError(f"moe_sort: out[{n!r}] must be a contiguous int32 tensor of at "
                                 f"least {sz} elements on {dev}")
        out = dict(out)
    _check("moe_sort", h.moe_sort(_ptr(topk_ids), T, k, num_experts, L, local_expert_offset,
                                  _ptr(out["offs"]), _ptr(out["m_indptr"]), _ptr(out["e2p"]),
                                  _ptr(out["p2e"]), _ptr(out["n_local"]), _ptr(workspace),
                                  workspace.numel(), _stream()))
    out["e2p"] = out["e2p"][: T * k]
    return out


# --------------------------------------------------------------------------- grouped GEMM
def grouped_gemm_fwd(x: torch.Tensor, w: torch.Tensor, offs: torch.Tensor, out=None,
                     offs_kind: Optional[str] = None, workspace: Optional[torch.Tensor] = None):
    """y[rows of e] = x[rows of e] @ w[e].T; x [M,K], w [E,N,K], offs int32 ends [E] (or indptr).
    workspace (optional, >= moe_gemm_split_workspace_size() bytes) lets the last round of
    tiles be cut along K (fixed-order fp32 partial sums)."""
    _dev(x, torch.bfloat16, "x"), _dev(w, torch.bfloat16, "w")
    E, N, K = w.shape
    kind = offs_kind or ("ends" if offs.numel() == E else "indptr")
    _dev(offs, torch.int32, "offs")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    nws = 0 if workspace is None else workspace.numel()
    _check("grouped_gemm_fwd", lib().grouped_gemm_fwd(_ptr(x), _ptr(w), _ptr(offs), OFFS[kind], E, M,
                                                      N, K, _ptr(out), _ptr(workspace), nws,
                                                      _stream()))
    return out


def grouped_gemm_dgrad(g: torch.Tensor, w: torch.Tensor, offs: torch.Tensor, out=None,
                       offs_kind: Optional[str] = None, workspace: Optional[torch.Tensor] = None):
    """dx[rows of e] = g[rows of e] @ w[e]; g [M,N], w [E,N,K] -> dx [M,K] bf16 (workspace as
    grouped_gemm_fwd: the last round's tiles cut along N)."""
    _dev(g, torch.bfloat16, "g"), _dev(w, torch.bfloat16, "w")
    E, N, K = w.shape
    kind = offs_kind or ("ends" if offs.numel() == E else "indptr")
    _dev(offs, torch.int32, "offs")
    M = g.shape[0]
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=g.device)
    nws = 0 if workspace is None else workspace.numel()
    _check("grouped_gemm_dgrad", lib().grouped_gemm_dgrad(_ptr(g), _ptr(w), _ptr(offs), OFFS[kind], E,
                                                          M, N, K, _ptr(out), _ptr(workspace), nws,
                                                          _stream()))
    return out


def grouped_gemm_wgrad(g: torch.Tensor, x: torch.Tensor, offs: torch.Tensor, E: Optional[int] = None,
                       out=None, out_dtype=torch.bfloat16, offs_kind: Optional[str] = None):
    """dw[e] = g[rows of e].T @ x[rows of e] -> [E, N, K] in bf16 or fp32."""
    _dev(g, torch.bfloat16, "g"), _dev(x, torch.bfloat16, "x")
    _dev(offs, torch.int32, "offs")
    kind = offs_kind or "ends"
    if E is None:
        E = offs.numel() if kind == "ends" else offs.numel() - 1
    M, N = g.shape
    K = x.shape[1]
    if out is None:
        out = torch.empty((E, N, K), dtype=out_dtype, device=g.device)
    h = lib()
    ws = h.grouped_gemm_wgrad_workspace_size(E, M, N, K, DTYPE[out.dtype])
    wsb = torch.empty(max(ws, 16), dtype=torch.uint8, device=g.device) if ws else None
    _check("grouped_gemm_wgrad", h.grouped_gemm_wgrad(_ptr(g), _ptr(x), _ptr(offs), OFFS[kind], E, M, N,
                                                      K, _ptr(out), DTYPE[out.dtype], _ptr(wsb), ws,
                                                      _stream()))
    return out


# --------------------------------------------------------------------------- MoE layer
def _ffn_desc(T, H, I, num_experts, L, off, k, activation, finalize, wfmt="bf16"):
    return MoeFfnDesc(T, H, I, num_experts, L, off, k, ACT[activation], FINALIZE[finalize], WFMT[wfmt])


def moe_ffn_workspace_size(T, H, I, num_experts, top_k, num_local_experts=None,
                           local_expert_offset=0, activation="swiglu", finalize="deterministic",
                           weight_format="bf16"):
    L = num_experts if num_local_experts is None else num_local_experts
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, top_k, activation, finalize,
                  weight_format)
    return lib().moe_ffn_workspace_size(ctypes.byref(d))


def moe_ffn_forward(x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                    w1: torch.Tensor, w2: torch.Tensor, num_experts: int,
                    num_local_experts: Optional[int] = None, local_expert_offset: int = 0,
                    activation: str = "swiglu", clamp_limit: Optional[torch.Tensor] = None,
                    finalize: str = "deterministic", out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                    e2p: Optional[torch.Tensor] = None):
    """out[t] = sum_s topk_weights[t,s] * ffn(x[t]; topk_ids[t,s]) (foreign routes give 0).

    finalize="none" returns (y [T*k, H] rows in permuted order, e2p [T*k]) instead of out.
    """
    _dev(x, torch.bfloat16, "x"), _dev(w1, torch.bfloat16, "w1"), _dev(w2, torch.bfloat16, "w2")
    _dev(topk_ids, torch.int32, "topk_ids"), _dev(topk_weights, torch.float32, "topk_weights")
    if clamp_limit is not None:
        _dev(clamp_limit, torch.float32, "clamp_limit")
    T, H = x.shape
    L, twoI, _ = w1.shape
    I = twoI // 2
    k = topk_ids.shape[1]
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, k, activation, finalize)
    h = lib()
    ws_bytes = h.moe_ffn_workspace_size(ctypes.byref(d))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
    if finalize == "none":
        if y is None:
            y = torch.empty((max(T * k, 1), H), dtype=torch.bfloat16, device=x.device)
        if e2p is None:
            e2p = torch.empty(max(T * k, 1), dtype=torch.int32, device=x.device)
    elif out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    tens = MoeFfnTensors(x.data_ptr(), topk_ids.data_ptr(), topk_weights.data_ptr(), w1.data_ptr(),
                         w2.data_ptr(), None if clamp_limit is None else clamp_limit.data_ptr(),
                         None if out is None else out.data_ptr(), None if y is None else y.data_ptr(),
                         None if e2p is None else e2p.data_ptr(), None, None, None)
    _check("moe_ffn_forward", h.moe_ffn_forward(ctypes.byref(d), ctypes.byref(tens), _ptr(workspace),
                                                workspace.numel(), _stream()))
    if finalize == "none":
        return y, e2p[: T * k]
    return out


def moe_ffn_forward_noalloc(x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                            w1: torch.Tensor, w2: torch.Tensor, num_experts: int,
                            num_local_experts: Optional[int] = None, local_expert_offset: int = 0,
                            activation: str = "swiglu", clamp_limit: Optional[torch.Tensor] = None,
                            finalize: str = "deterministic", out: Optional[torch.Tensor] = None,
                            y: Optional[torch.Tensor] = None, e2p: Optional[torch.Tensor] = None,
                            weight_format: str = "bf16", x_sf: Optional[torch.Tensor] = None,
                            w1_sf: Optional[torch.Tensor] = None, w2_sf: Optional[torch.Tensor] = None,
                            act_scale: Optional[torch.Tensor] = None):
    """moe_ffn_forward with the library's fixed scratch memory instead of a workspace: the
    same layer and bits. Outputs (out, or y and e2p for finalize="none") must be passed in
    by a caller that cannot allocate; here they are created when omitted. weight_format
    "mxfp4" / "mxfp8" / "fp8" takes the operands of moe_ffn_forward_mx / _fp8 (x_sf, w1_sf,
    w2_sf hold x_scale, w1_scale, w2_scale for "fp8")."""
    wdt = torch.bfloat16 if weight_format == "bf16" else torch.uint8
    _dev(x, wdt, "x"), _dev(w1, wdt, "w1"), _dev(w2, wdt, "w2")
    _dev(topk_ids, torch.int32, "topk_ids"), _dev(topk_weights, torch.float32, "topk_weights")
    T, H = x.shape
    L, twoI, _ = w1.shape
    I = twoI // 2
    k = topk_ids.shape[1]
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, k, activation, finalize,
                  weight_format)
    if finalize == "none":
        if y is None:
            y = torch.empty((max(T * k, 1), H), dtype=torch.bfloat16, device=x.device)
        if e2p is None:
            e2p = torch.empty(max(T * k, 1), dtype=torch.int32, device=x.device)
    elif out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    p = lambda t_: None if t_ is None else t_.data_ptr()  # noqa: E731
    tens = MoeFfnTensors(p(x), p(topk_ids), p(topk_weights), p(w1), p(w2), p(clamp_limit), p(out),
                         p(y), p(e2p), p(x_sf), p(w1_sf), p(w2_sf), p(act_scale))
    _check("moe_ffn_forward_noalloc", lib().moe_ffn_forward_noalloc(ctypes.byref(d), ctypes.byref(tens),
                                                                    _stream()))
    if finalize == "none":
        return y, e2p[: T * k]
    return out


def _train_desc(x, topk_ids, w1, num_experts, num_local_experts, local_expert_offset, activation):
    _dev(x, torch.bfloat16, "x"), _dev(w1, torch.bfloat16, "w1")
    _dev(topk_ids, torch.int32, "topk_ids")
    T, H = x.shape
    L, twoI, _ = w1.shape
    if num_local_experts is not None and num_local_experts != L:
        raise ValueError("num_local_experts must equal w1.shape[0]")
    return _ffn_desc(T, H, twoI // 2, num_experts, L, local_expert_offset, topk_ids.shape[1],
                     activation, "deterministic")


def moe_ffn_forward_train(x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                          w1: torch.Tensor, w2: torch.Tensor, num_experts: int,
                          num_local_experts: Optional[int] = None, local_expert_offset: int = 0,
                          activation: str = "swiglu", clamp_limit: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, saved: Optional[torch.Tensor] = None):
    """The bf16 layer forward (deterministic finalize) that also keeps what the backward
    needs. Returns (out [T, H] bf16, saved): pass `saved` unchanged to moe_ffn_backward."""
    _dev(w2, torch.bfloat16, "w2"), _dev(topk_weights, torch.float32, "topk_weights")
    if clamp_limit is not None:
        _dev(clamp_limit, torch.float32, "clamp_limit")
    d = _train_desc(x, topk_ids, w1, num_experts, num_local_experts, local_expert_offset, activation)
    h = lib()
    nbytes = h.moe_ffn_saved_size(ctypes.byref(d))
    if saved is None:
        saved = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty(tuple(x.shape), dtype=torch.bfloat16, device=x.device)
    tens = MoeFfnTensors(x.data_ptr(), topk_ids.data_ptr(), topk_weights.data_ptr(), w1.data_ptr(),
                         w2.data_ptr(), None if clamp_limit is None else clamp_limit.data_ptr(),
                         out.data_ptr(), None, None, None, None, None)
    _check("moe_ffn_forward_train", h.moe_ffn_forward_train(ctypes.byref(d), ctypes.byref(tens),
                                                            _ptr(saved), saved.numel(), _stream()))
    return out, saved


def moe_ffn_backward(dout: torch.Tensor, saved: torch.Tensor, x: torch.Tensor,
                     topk_ids: torch.Tensor, topk_weights: torch.Tensor, w1: torch.Tensor,
                     w2: torch.Tensor, num_experts: int, num_local_experts: Optional[int] = None,
                     local_expert_offset: int = 0, activation: str = "swiglu",
                     clamp_limit: Optional[torch.Tensor] = None, grad_dtype=torch.bfloat16,
                     need_topk_grad: bool = True, workspace: Optional[torch.Tensor] = None):
    """Gradients of the layer for dout [T, H] bf16, with the tensors and `saved` of
    moe_ffn_forward_train. Returns (dx [T,H] bf16, dw1 [L,2I,H], dw2 [L,H,I] in grad_dtype,
    dtopk_weights [T,k] float32 or None)."""
    _dev(dout, torch.bfloat16, "dout"), _dev(w2, torch.bfloat16, "w2")
    _dev(topk_weights, torch.float32, "topk_weights"), _dev(saved, torch.uint8, "saved")
    d = _train_desc(x, topk_ids, w1, num_experts, num_local_experts, local_expert_offset, activation)
    h = lib()
    ws = h.moe_ffn_backward_workspace_size(ctypes.byref(d))
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=x.device)
    dx = torch.empty(tuple(x.shape), dtype=torch.bfloat16, device=x.device)
    dw1 = torch.empty(tuple(w1.shape), dtype=grad_dtype, device=x.device)
    dw2 = torch.empty(tuple(w2.shape), dtype=grad_dtype, device=x.device)
    dtw = torch.empty(tuple(topk_ids.shape), dtype=torch.float32, device=x.device) if need_topk_grad else None
    tens = MoeFfnTensors(x.data_ptr(), topk_ids.data_ptr(), topk_weights.data_ptr(), w1.data_ptr(),
                         w2.data_ptr(), None if clamp_limit is None else clamp_limit.data_ptr(),
                         None, None, None, None, None, None)
    grads = MoeFfnGrads(dout.data_ptr(), dx.data_ptr(), dw1.data_ptr(), dw2.data_ptr(),
                        None if dtw is None else dtw.data_ptr(), DTYPE[grad_dtype])
    _check("moe_ffn_backward", h.moe_ffn_backward(ctypes.byref(d), ctypes.byref(tens), ctypes.byref(grads),
                                                  _ptr(saved), saved.numel(), _ptr(workspace),
                                                  workspace.numel(), _stream()))
    return dx, dw1, dw2, dtw


def moe_route_backward(topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                       dtopk_weights: torch.Tensor, num_experts: int, dlogits=None):
    """d loss / d logits [T, E] float32 through the Renormalize weights of moe_route."""
    _dev(topk_ids, torch.int32, "topk_ids"), _dev(topk_weights, torch.float32, "topk_weights")
    _dev(dtopk_weights, torch.float32, "dtopk_weights")
    T, k = topk_ids.shape
    if dlogits is None:
        dlogits = torch.empty((T, num_experts), dtype=torch.float32, device=topk_ids.device)
    _check("moe_route_backward", lib().moe_route_backward(_ptr(topk_ids), _ptr(topk_weights),
                                                          _ptr(dtopk_weights), T, num_experts, k,
                                                          _ptr(dlogits), _stream()))
    return dlogits


class MoEFunction(torch.autograd.Function):
    """Autograd wrapper of the bf16 layer: out = MoEFunction.apply(x, topk_weights, w1, w2,
    topk_ids, num_experts, local_expert_offset, activation, clamp_limit). Gradients flow to
    x, topk_weights, w1 and w2 (bf16, like the parameters), each step in the library."""

    @staticmethod
    def forward(ctx, x, topk_weights, w1, w2, topk_ids, num_experts, local_expert_offset=0,
                activation="swiglu", clamp_limit=None):
        out, saved = moe_ffn_forward_train(x, topk_ids, topk_weights, w1, w2, num_experts,
                                           local_expert_offset=local_expert_offset,
                                           activation=activation, clamp_limit=clamp_limit)
        ctx.save_for_backward(x, topk_weights, w1, w2, topk_ids, saved)
        ctx.cfg = (num_experts, local_expert_offset, activation, clamp_limit)
        return out

    @staticmethod
    def backward(ctx, dout):
        x, topk_weights, w1, w2, topk_ids, saved = ctx.saved_tensors
        num_experts, off, activation, clamp_limit = ctx.cfg
        dx, dw1, dw2, dtw = moe_ffn_backward(
            dout.contiguous(), saved, x, topk_ids, topk_weights, w1, w2, num_experts,
            local_expert_offset=off, activation=activation, clamp_limit=clamp_limit,
            need_topk_grad=ctx.needs_input_grad[1])
        return dx, dtw, dw1, dw2, None, None, None, None, None


def _split_ws(split: bool, workspace: Optional[torch.Tensor], device):
    """(pointer, bytes) of the split-tile workspace of moe_fc1 / moe_fc2, or (None, 0)."""
    if not split:
        return None, 0
    if workspace is None:
        workspace = torch.empty(lib().moe_gemm_split_workspace_size(), dtype=torch.uint8,
                                device=device)
    return workspace, workspace.numel() * workspace.element_size()


def moe_fc1(x: torch.Tensor, w1: torch.Tensor, offs: torch.Tensor, p2e: torch.Tensor, top_k: int,
            num_experts: int, local_expert_offset: int = 0, activation: str = "swiglu",
            clamp_limit: Optional[torch.Tensor] = None, act: Optional[torch.Tensor] = None,
            split: bool = True, workspace: Optional[torch.Tensor] = None):
    """act[p] = activation(x[p2e[p] // top_k] @ w1[e].T) for the expert-sorted rows p.
    split: let a mostly idle last round of tiles be cut along K (workspace: optional
    moe_gemm_split_workspace_size() bytes, allocated here if None)."""
    _dev(x, torch.bfloat16, "x"), _dev(w1, torch.bfloat16, "w1")
    T, H = x.shape
    L, twoI, _ = w1.shape
    I = twoI // 2
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, top_k, activation, "deterministic")
    if act is None:
        act = torch.empty((max(T * top_k, 1), I), dtype=torch.bfloat16, device=x.device)
    ws, ws_bytes = _split_ws(split, workspace, x.device)
    _check("moe_fc1", lib().moe_fc1(ctypes.byref(d), _ptr(x), _ptr(w1), _ptr(clamp_limit), _ptr(offs),
                                    _ptr(p2e), _ptr(act), _ptr(ws), ws_bytes, _stream()))
    return act


def moe_fc2(act: torch.Tensor, w2: torch.Tensor, offs: torch.Tensor, T: int, top_k: int,
            num_experts: int, local_expert_offset: int = 0, finalize: str = "deterministic",
            p2e: Optional[torch.Tensor] = None, topk_weights: Optional[torch.Tensor] = None,
            dst: Optional[torch.Tensor] = None, split: bool = True,
            workspace: Optional[torch.Tensor] = None):
    """y[p] = act[p] @ w2[e].T (rows [T*k, H]); with finalize="fused" the scaled rows are
    added into a zeroed out [T, H] instead. split / workspace as for moe_fc1."""
    _dev(act, torch.bfloat16, "act"), _dev(w2, torch.bfloat16, "w2")
    L, H, I = w2.shape
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, top_k, "swiglu", finalize)
    if dst is None:
        rows = T if finalize == "fused" else max(T * top_k, 1)
        dst = torch.empty((rows, H), dtype=torch.bfloat16, device=act.device)
    ws, ws_bytes = _split_ws(split, workspace, act.device)
    _check("moe_fc2", lib().moe_fc2(ctypes.byref(d), _ptr(act), _ptr(w2), _ptr(offs), _ptr(p2e),
                                    _ptr(topk_weights), _ptr(dst), _ptr(ws), ws_bytes, _stream()))
    return dst


def _mx_format(last_dim: int, K: int, name: str) -> str:
    """Weight family of an MX bank from the bytes per row: K/2 (MXFP4) or K (MXFP8)."""
    if last_dim == K:
        return "mxfp8"
    if 2 * last_dim == K:
        return "mxfp4"
    raise ValueError(f"{name}: {last_dim} bytes per row fit neither MXFP4 ({K // 2}) nor MXFP8 ({K})")


def moe_ffn_forward_mx(x: torch.Tensor, x_sf: torch.Tensor, topk_ids: torch.Tensor,
                       topk_weights: torch.Tensor, w1: torch.Tensor, w1_sf: torch.Tensor,
                       w2: torch.Tensor, w2_sf: torch.Tensor, num_experts: int,
                       num_local_experts: Optional[int] = None, local_expert_offset: int = 0,
                       activation: str = "swiglu", clamp_limit: Optional[torch.Tensor] = None,
                       finalize: str = "deterministic", out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                       e2p: Optional[torch.Tensor] = None):
    """Block-scaled layer: x MXFP8 (uint8 e4m3 codes [T,H] + UE8M0 [T,H/32]); w1 / w2 either
    MXFP4 (packed uint8 [L,2I,H/2] / [L,H,I/2]) or MXFP8 (e4m3 codes [L,2I,H] / [L,H,I]), told
    apart by their last dimension, with UE8M0 scales [L,2I,H/32] / [L,H,I/32]; bf16 output."""
    for t_, n_ in [(x, "x"), (x_sf, "x_sf"), (w1, "w1"), (w1_sf, "w1_sf"), (w2, "w2"), (w2_sf, "w2_sf")]:
        _dev(t_, torch.uint8, n_)
    H = x.shape[1]
    I = w1.shape[1] // 2
    wfmt = _mx_format(w1.shape[2], H, "w1")
    if w2.shape[2] != (I if wfmt == "mxfp8" else I // 2):
        raise ValueError(f"w2 last dim {w2.shape[2]} does not match the {wfmt} w1")
    return _ffn_forward_fp8act(wfmt, x, x_sf, topk_ids, topk_weights, w1, w1_sf, w2, w2_sf, None,
                               num_experts, num_local_experts, local_expert_offset, activation,
                               clamp_limit, finalize, out, workspace, y, e2p)


def moe_ffn_forward_fp8(x: torch.Tensor, x_scale: torch.Tensor, topk_ids: torch.Tensor,
                        topk_weights: torch.Tensor, w1: torch.Tensor, w1_scale: torch.Tensor,
                        w2: torch.Tensor, w2_scale: torch.Tensor, act_scale: torch.Tensor,
                        num_experts: int, num_local_experts: Optional[int] = None,
                        local_expert_offset: int = 0, activation: str = "swiglu",
                        clamp_limit: Optional[torch.Tensor] = None, finalize: str = "deterministic",
                        out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        y: Optional[torch.Tensor] = None, e2p: Optional[torch.Tensor] = None):
    """fp8 per-tensor layer: x, w1 [L,2I,H], w2 [L,H,I] e4m3 codes (uint8); x_scale [1],
    w1_scale / w2_scale [L] and act_scale [1] (the static scale of the requantized FC1
    output) float32 device tensors; bf16 output."""
    for t_, n_ in [(x, "x"), (w1, "w1"), (w2, "w2")]:
        _dev(t_, torch.uint8, n_)
    for t_, n_ in [(x_scale, "x_scale"), (w1_scale, "w1_scale"), (w2_scale, "w2_scale"),
                   (act_scale, "act_scale")]:
        _dev(t_, torch.float32, n_)
    L, twoI, H = w1.shape
    if H != x.shape[1] or tuple(w2.shape) != (L, H, twoI // 2):
        raise ValueError("fp8: w1 must be [L, 2I, H] and w2 [L, H, I] e4m3 codes")
    if w1_scale.numel() != L or w2_scale.numel() != L or x_scale.numel() < 1 or act_scale.numel() < 1:
        raise ValueError("fp8: x_scale / act_scale need one value, w1_scale / w2_scale one per expert")
    return _ffn_forward_fp8act("fp8", x, x_scale, topk_ids, topk_weights, w1, w1_scale, w2, w2_scale,
                               act_scale, num_experts, num_local_experts, local_expert_offset,
                               activation, clamp_limit, finalize, out, workspace, y, e2p)


def _ffn_forward_fp8act(wfmt, x, x_sf, topk_ids, topk_weights, w1, w1_sf, w2, w2_sf, act_scale,
                        num_experts, num_local_experts, local_expert_offset, activation,
                        clamp_limit, finalize, out, workspace, y, e2p):
    _dev(topk_ids, torch.int32, "topk_ids"), _dev(topk_weights, torch.float32, "topk_weights")
    if clamp_limit is not None:
        _dev(clamp_limit, torch.float32, "clamp_limit")
    T, H = x.shape
    L, twoI, _ = w1.shape
    I = twoI // 2
    k = topk_ids.shape[1]
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, k, activation, finalize, wfmt)
    h = lib()
    ws_bytes = h.moe_ffn_workspace_size(ctypes.byref(d))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
    if finalize == "none":
        if y is None:
            y = torch.empty((max(T * k, 1), H), dtype=torch.bfloat16, device=x.device)
        if e2p is None:
            e2p = torch.empty(max(T * k, 1), dtype=torch.int32, device=x.device)
    elif out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    tens = MoeFfnTensors(x.data_ptr(), topk_ids.data_ptr(), topk_weights.data_ptr(), w1.data_ptr(),
                         w2.data_ptr(), None if clamp_limit is None else clamp_limit.data_ptr(),
                         None if out is None else out.data_ptr(), None if y is None else y.data_ptr(),
                         None if e2p is None else e2p.data_ptr(), x_sf.data_ptr(), w1_sf.data_ptr(),
                         w2_sf.data_ptr(), None if act_scale is None else act_scale.data_ptr())
    _check("moe_ffn_forward", h.moe_ffn_forward(ctypes.byref(d), ctypes.byref(tens), _ptr(workspace),
                                                workspace.numel(), _stream()))
    if finalize == "none":
        return y, e2p[: T * k]
    return out


def moe_tune(x, topk_ids, topk_weights, w1, w2, num_experts, num_local_experts=None,
             local_expert_offset=0, activation="swiglu", clamp_limit=None, x_sf=None, w1_sf=None,
             w2_sf=None, act_scale=None, workspace=None):
    """Times both tile families of the layer's FC1 / FC2 on these inputs and records the
    faster one for this shape and token bucket (synchronises). bf16 operands (x bf16) or
    the operands of moe_ffn_forward_mx (x_sf, w1_sf, w2_sf) / moe_ffn_forward_fp8 (x_sf,
    w1_sf, w2_sf holding x_scale, w1_scale, w2_scale, plus act_scale). Returns the (fc1,
    fc2) picks: 1 = the smaller family (128-row bf16 tile or 32-row streaming tile), 0 =
    the 256-row tile."""
    T, H = x.shape
    L, twoI, _ = w1.shape
    I = twoI // 2
    if x.dtype == torch.bfloat16:
        wfmt = "bf16"
    else:
        wfmt = "fp8" if act_scale is not None else _mx_format(w1.shape[2], H, "w1")
    k = topk_ids.shape[1]
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, k, activation, "deterministic", wfmt)
    h = lib()
    if workspace is None:
        workspace = torch.empty(max(h.moe_ffn_workspace_size(ctypes.byref(d)), 16), dtype=torch.uint8,
                                device=x.device)
    p = lambda t_: None if t_ is None else t_.data_ptr()  # noqa: E731
    tens = MoeFfnTensors(p(x), p(topk_ids), p(topk_weights), p(w1), p(w2), p(clamp_limit), None, None,
                         None, p(x_sf), p(w1_sf), p(w2_sf), p(act_scale))
    choice = (ctypes.c_int32 * 2)(-1, -1)
    _check("moe_tune", h.moe_tune(ctypes.byref(d), ctypes.byref(tens), _ptr(workspace),
                                  workspace.numel(), _stream(), choice))
    return int(choice[0]), int(choice[1])


def moe_tune_set(T, H, I, num_experts, top_k, stage, choice, num_local_experts=None,
                 local_expert_offset=0, weight_format="bf16"):
    """Record a tile family for one stage (1 = FC1, 2 = FC2) of this shape and token
    bucket, as moe_tune would after timing: 1 = the smaller family, 0 = the 256-row tile."""
    L = num_experts if num_local_experts is None else num_local_experts
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, top_k, "swiglu", "deterministic",
                  weight_format)
    _check("moe_tune_set", lib().moe_tune_set(ctypes.byref(d), stage, choice))


def moe_tune_clear():
    """Forget every tile choice recorded by moe_tune / moe_tune_set."""
    lib().moe_tune_clear()


def moe_fc1_mx(x, x_sf, w1, w1_sf, offs, p2e, top_k, num_experts, local_expert_offset=0,
               activation="swiglu", clamp_limit=None, act=None, act_sf=None):
    """act (MXFP8 codes [T*k, I] + UE8M0 [T*k, I/32]) = requant(activation(FC1)) per permuted row;
    w1 MXFP4 or MXFP8 (see moe_ffn_forward_mx)."""
    T, H = x.shape
    L, twoI, _ = w1.shape
    I = twoI // 2
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, top_k, activation,
                  "deterministic", _mx_format(w1.shape[2], H, "w1"))
    if act is None:
        act = torch.empty((max(T * top_k, 1), I), dtype=torch.uint8, device=x.device)
    if act_sf is None:
        act_sf = torch.empty((max(T * top_k, 1), I // 32), dtype=torch.uint8, device=x.device)
    _check("moe_fc1_mx", lib().moe_fc1_mx(ctypes.byref(d), _ptr(x), _ptr(x_sf), _ptr(w1), _ptr(w1_sf),
                                          _ptr(clamp_limit), _ptr(offs), _ptr(p2e), _ptr(act),
                                          _ptr(act_sf), _stream()))
    return act, act_sf


def moe_fc2_mx(act, act_sf, w2, w2_sf, offs, T, top_k, num_experts, local_expert_offset=0, y=None):
    """y [T*k, H] bf16 = act @ w2[e].T for the permuted rows (MXFP8 act, MXFP4 or MXFP8 w2)."""
    L, H, _ = w2.shape
    I = act.shape[1]
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, top_k, "swiglu", "deterministic",
                  _mx_format(w2.shape[2], I, "w2"))
    if y is None:
        y = torch.empty((max(T * top_k, 1), H), dtype=torch.bfloat16, device=act.device)
    _check("moe_fc2_mx", lib().moe_fc2_mx(ctypes.byref(d), _ptr(act), _ptr(act_sf), _ptr(w2), _ptr(w2_sf),
                                          _ptr(offs), _ptr(y), _stream()))
    return y


def moe_fc1_fp8(x, x_scale, w1, w1_scale, act_scale, offs, p2e, top_k, num_experts,
                local_expert_offset=0, activation="swiglu", clamp_limit=None, act=None):
    """act (e4m3 codes [T*k, I]) = per-tensor requant(activation(FC1)) per permuted row."""
    T, H = x.shape
    L, twoI, _ = w1.shape
    I = twoI // 2
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, top_k, activation,
                  "deterministic", "fp8")
    if act is None:
        act = torch.empty((max(T * top_k, 1), I), dtype=torch.uint8, device=x.device)
    _check("moe_fc1_fp8", lib().moe_fc1_fp8(ctypes.byref(d), _ptr(x), _ptr(x_scale), _ptr(w1),
                                            _ptr(w1_scale), _ptr(act_scale), _ptr(clamp_limit),
                                            _ptr(offs), _ptr(p2e), _ptr(act), _stream()))
    return act


def moe_fc2_fp8(act, act_scale, w2, w2_scale, offs, T, top_k, num_experts, local_expert_offset=0,
                y=None):
    """y [T*k, H] bf16 = act_scale * w2_scale[e] * (act @ w2[e].T) for the permuted rows."""
    L, H, I = w2.shape
    d = _ffn_desc(T, H, I, num_experts, L, local_expert_offset, top_k, "swiglu", "deterministic",
                  "fp8")
    if y is None:
        y = torch.empty((max(T * top_k, 1), H), dtype=torch.bfloat16, device=act.device)
    _check("moe_fc2_fp8", lib().moe_fc2_fp8(ctypes.byref(d), _ptr(act), _ptr(act_scale), _ptr(w2),
                                            _ptr(w2_scale), _ptr(offs), _ptr(y), _stream()))
    return y


def moe_bgmv_workspace_bytes(T: int, P: int, H: int, feat_out: int, rank: int, num_loras: int,
                             num_experts: int, grouped: Optional[bool] = None) -> int:
    """Workspace bytes moe_bgmv needs for these sizes (grouped as in moe_bgmv)."""
    d = MoeBgmvDesc(T, P, H, feat_out, rank, num_loras, num_experts,
                    0 if grouped is None else (2 if grouped else 1))
    return int(lib().moe_bgmv_workspace_size(ctypes.byref(d)))


def moe_bgmv(x: torch.Tensor, lora_a: torch.Tensor, lora_b: torch.Tensor,
             sorted_token_ids: torch.Tensor, expert_ids: torch.Tensor, lora_indices: torch.Tensor,
             topk_weights: torch.Tensor, num_experts: int, shrink_out: Optional[torch.Tensor] = None,
             y_accum: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             grouped: Optional[bool] = None):
    """BGMV MoE-LoRA shrink + expand. x [T,H] bf16, lora_a [nl,E,rank,H], lora_b [nl,E,N,rank]
    bf16, sorted_token_ids / expert_ids [P] int32, lora_indices [T] int32, topk_weights [P]
    float32. grouped: None lets the library choose the pipeline, True / False force the
    grouped / per-pair one. Returns (y_accum [T, N] float32 (or the given, possibly
    strided, view), shrink [P, rank] bf16)."""
    _dev(x, torch.bfloat16, "x"), _dev(lora_a, torch.bfloat16, "lora_a"), _dev(lora_b, torch.bfloat16, "lora_b")
    for t_, n_ in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                   (lora_indices, "lora_indices")):
        _dev(t_, torch.int32, n_)
    _dev(topk_weights, torch.float32, "topk_weights")
    T, H = x.shape
    nl, E, r, H2 = lora_a.shape
    N = lora_b.shape[2]
    if H2 != H or tuple(lora_b.shape) != (nl, E, N, r) or E != num_experts:
        raise ValueError("bgmv: lora_a must be [nl, E, rank, H] and lora_b [nl, E, N, rank]")
    P = sorted_token_ids.numel()
    d = MoeBgmvDesc(T, P, H, N, r, nl, num_experts, 0 if grouped is None else (2 if grouped else 1))
    h = lib()
    if workspace is None:
        workspace = torch.empty(max(h.moe_bgmv_workspace_size(ctypes.byref(d)), 16), dtype=torch.uint8,
                                device=x.device)
    if shrink_out is None:
        shrink_out = torch.empty((max(P, 1), r), dtype=torch.bfloat16, device=x.device)
    if y_accum is None:
        y_accum = torch.empty((T, N), dtype=torch.float32, device=x.device)
    if y_accum.dtype != torch.float32 or y_accum.shape != (T, N) or y_accum.stride(1) != 1:
        raise ValueError("bgmv: y_accum must be float32 [T, feat_out] with unit column stride")
    _check("moe_bgmv", h.moe_bgmv(ctypes.byref(d), _ptr(x), _ptr(lora_a), _ptr(lora_b), _ptr(sorted_token_ids),
                                  _ptr(expert_ids), _ptr(lora_indices), _ptr(topk_weights), _ptr(shrink_out),
                                  _ptr(y_accum), y_accum.stride(0), _ptr(workspace), workspace.numel(),
                                  _stream()))
    return y_accum, shrink_out[:P]


def moe_finalize(y: torch.Tensor, e2p: torch.Tensor, topk_weights: torch.Tensor, out=None):
    """Deterministic combine: out[t] = bf16(sum_s w[t,s] * y[e2p[t*k+s]]) in fp32, s ascending."""
    _dev(y, torch.bfloat16, "y"), _dev(e2p, torch.int32, "e2p")
    _dev(topk_weights, torch.float32, "topk_weights")
    T, k = topk_weights.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check("moe_finalize", lib().moe_finalize(_ptr(y), _ptr(e2p), _ptr(topk_weights), T, k, H,
                                              _ptr(out), _stream()))
    return out
