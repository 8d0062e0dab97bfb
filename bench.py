"""Benchmark: the Mixtral-shaped routed-MoE expert layer on one MI355X.

One step = one pass of the whole hot path over a resident synthetic batch:
route (top-2 of 8 from fp32 logits) -> sort -> FC1 + SwiGLU -> FC2 -> the
deterministic finalize, at T=4096, H=4096, I=14336, E=8, top_k=2 (bf16
operands, fp32 accumulation). The same step with the fused finalize is timed
as well. Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer TFLOP/s + tokens/s (T=4096, Mixtral shape); % of MFMA peak"
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (the e2m1 x e4m3 MFMA runs at this rate)
FC1_KERNEL = "k_gemm_nt<1, true, 256>"  # FC1 grouped GEMM, SwiGLU epilogue, full-K path, 256-row tiles
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fc1_mixtral_traffic.json")
KERNEL_SOURCES = ["mixture_experts_expert_softmax_amd/csrc/gemm_bf16.hip",
                  "mixture_experts_expert_softmax_amd/csrc/common.h"]


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic():
    """HBM bytes per FC1 launch from committed rocprofv3 counter runs, valid only
    while the kernel source is unchanged since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(case, ids, w, n_tokens, n_experts):
    """Time the CPU oracle on a bounded sample of the same workload: the first
    n_tokens tokens, evaluated on the shard of the first n_experts experts (routes
    to other experts are skipped by the oracle's shard rule)."""
    import numpy as np
    import moe_synth as S
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    x = S.bf16_to_f32(case.x[:n_tokens])
    w1 = S.bf16_to_f32(case.w1[:n_experts])
    w2 = S.bf16_to_f32(case.w2[:n_experts])
    ids_n, w_n = ids[:n_tokens], w[:n_tokens].astype(np.float64)
    routes = int(np.count_nonzero(ids_n < n_experts))
    t0 = time.perf_counter()
    O.moe_forward(x, ids_n, w_n, w1, w2, num_experts=case.num_experts, local_offset=0)
    dt = time.perf_counter() - t0
    flops = 6.0 * case.H * case.I * routes
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    # tokens/s scaled from routes/s: a token carries top_k routes
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "tokens_per_s": routes / case.top_k / dt, "seconds": dt, "routes": routes,
            "sample": f"{routes} routes: first {n_tokens} of {case.T} tokens on the shard of experts "
                      f"0..{n_experts - 1} of {case.num_experts}; numpy float64 oracle incl. "
                      f"per-expert weight widening; {cpu}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--cpu-experts", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary rows (grouped GEMMs, expert shard, large route/sort/finalize)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy (3x): the known-size "
                         "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--profile", choices=sorted(PROFILE_WORKLOADS),
                    help="only run one workload a few times (3 warm-up, 5 measured calls), for "
                         "rocprofv3 kernel traces and counters; prints its mean event time")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        import torch
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return

    if args.profile:
        profile_workload(args.profile)
        return

    import numpy as np
    import torch
    import mixture_experts_expert_softmax_amd as M
    import moe_synth as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    M.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    progress("generating the synthetic Mixtral-shaped batch")
    case = S.mixtral_moe(seed=0)
    T, H, I, E, k = case.T, case.H, case.I, case.num_experts, case.top_k
    logits = torch.from_numpy(case.logits).to(dev)
    x, w1, w2 = case.x.to(dev), case.w1.to(dev), case.w2.to(dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    sort_ws = torch.empty(max(M.lib().moe_sort_workspace_size(T, k, E), 16), dtype=torch.uint8, device=dev)
    offs = torch.empty(E, dtype=torch.int32, device=dev)
    e2p = torch.empty(T * k, dtype=torch.int32, device=dev)
    p2e = torch.empty(T * k, dtype=torch.int32, device=dev)
    nloc = torch.empty(1, dtype=torch.int32, device=dev)
    act = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    out_fused = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    lib = M.lib()
    P = M._ptr
    # the GEMM stages' split-tile workspace (the layer call keeps one in its own workspace)
    split_ws = torch.empty(lib.moe_gemm_split_workspace_size(), dtype=torch.uint8, device=dev)

    def route():
        M._check("moe_route", lib.moe_route(P(logits), T, E, k, P(ids), P(wts), M._stream()))

    def sort():
        M._check("moe_sort", lib.moe_sort(P(ids), T, k, E, E, 0, P(offs), None, P(e2p), P(p2e), P(nloc),
                                          P(sort_ws), sort_ws.numel(), M._stream()))

    def fc1():
        M.moe_fc1(x, w1, offs, p2e, k, E, act=act, workspace=split_ws)

    def fc2(fused=False):
        if fused:
            M.moe_fc2(act, w2, offs, T, k, E, finalize="fused", p2e=p2e, topk_weights=wts, dst=out_fused,
                      workspace=split_ws)
        else:
            M.moe_fc2(act, w2, offs, T, k, E, dst=y, workspace=split_ws)

    def finalize():
        M.moe_finalize(y, e2p, wts, out=out)

    stages = [("route", route), ("sort", sort), ("fc1", fc1), ("fc2", fc2), ("finalize", finalize)]
    stages_fused = [("route", route), ("sort", sort), ("fc1", fc1), ("fc2_fused", lambda: fc2(True))]

    def run(stage_list, steps, warmup):
        for _ in range(warmup):
            for _, f in stage_list:
                f()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stage_list) + 1)] for _ in range(steps)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for s in range(steps):
            ev[s][0].record()
            for j, (_, f) in enumerate(stage_list):
                f()
                ev[s][j + 1].record()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total_ms = start.elapsed_time(end) / steps
        per_stage = {name: float(np.mean([ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(steps)]))
                     for j, (name, _) in enumerate(stage_list)}
        return total_ms, per_stage, wall

    progress("timing the deterministic-finalize step")
    ms, per_stage, wall = run(stages, args.steps, args.warmup)
    progress("timing the fused-finalize step")
    ms_f, per_stage_f, _ = run(stages_fused, args.steps, args.warmup)
    n_local = int(nloc.item())
    flops = 6.0 * H * I * n_local            # FC1 (4HI) + FC2 (2HI) per local route
    fc1_flops = 4.0 * H * I * n_local
    tflops = flops / (ms * 1e-3) / 1e12
    fc1_tflops = fc1_flops / (per_stage["fc1"] * 1e-3) / 1e12
    fc2_tflops = 2.0 * H * I * n_local / (per_stage["fc2"] * 1e-3) / 1e12
    # finalize: reads n_local y rows + ids/weights, writes T output rows (bf16)
    fin_bytes = n_local * H * 2 + T * H * 2 + T * k * 8
    traffic = load_traffic()
    cpu = None
    if not args.no_cpu_baseline:
        progress("timing the CPU oracle sample")
        cpu = cpu_baseline(case, ids.cpu().numpy(), wts.cpu().numpy(), args.cpu_tokens, args.cpu_experts)
    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mixtral_moe_forward", "T": T, "H": H, "I": I, "num_experts": E,
                   "top_k": k, "activation": "swiglu", "finalize": "deterministic",
                   "logit_bias_var": 0.5, "seed": 0, "n_local_routes": n_local},
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "mfma_frac_layer": round(tflops / BF16_PEAK_TFLOPS, 4),
        "stage_ms": {k_: round(v, 4) for k_, v in per_stage.items()},
        "fc2_tflops": round(fc2_tflops, 2),
        "finalize_gbs": round(fin_bytes / (per_stage["finalize"] * 1e-3) / 1e9, 1),
        "fused_finalize": {"ms_per_step": round(ms_f, 4),
                           "value": round(flops / (ms_f * 1e-3) / 1e12, 2),
                           "tokens_per_s": round(T / (ms_f * 1e-3), 1),
                           "stage_ms": {k_: round(v, 4) for k_, v in per_stage_f.items()}},
        "roofline": {"kernel": FC1_KERNEL, "bound": "mfma", "achieved": round(fc1_tflops, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fc1_tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_secondary:
        progress("timing the training forward and the backward at the same shape")
        line["training"] = _training(x, w1, w2, ids, wts, E, n_local)
        del x, w1, w2, act, y, out, out_fused
        torch.cuda.empty_cache()
        line["secondary"] = secondary_measurements(progress)
    print(json.dumps(line), flush=True)


def _capture(fn):
    """fn captured into a graph (after a warm-up run on a side stream)."""
    import torch
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fn()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _training(x, w1, w2, ids, wts, E, n_local):
    """The bf16 layer's training forward (which also keeps h, act, y) and its backward
    (dx, dw1, dw2 in bf16, routing-weight gradients) on the benchmark batch; the upstream
    gradient is seeded N(0, 1). Backward work: dgrad + wgrad of both grouped products,
    12 H I flop per local route."""
    import ctypes
    import torch
    import mixture_experts_expert_softmax_amd as M
    import moe_synth as S
    T, H = x.shape
    I = w2.shape[2]
    dout = S.upstream_grad(0, T, H).to(x.device)
    out_t, saved = M.moe_ffn_forward_train(x, ids, wts, w1, w2, E)
    d = M._train_desc(x, ids, w1, E, None, 0, "swiglu")
    bws = torch.empty(max(M.lib().moe_ffn_backward_workspace_size(ctypes.byref(d)), 16),
                      dtype=torch.uint8, device=x.device)
    ms_f = _time(lambda: M.moe_ffn_forward_train(x, ids, wts, w1, w2, E, out=out_t, saved=saved))
    ms_b = _time(lambda: M.moe_ffn_backward(dout, saved, x, ids, wts, w1, w2, E, workspace=bws))
    fl_b = 12.0 * H * I * n_local
    return {"fwd_train_ms": round(ms_f, 4), "bwd_ms": round(ms_b, 4),
            "bwd_tflops": round(fl_b / (ms_b * 1e-3) / 1e12, 1),
            "bwd_mfma_frac": round(fl_b / (ms_b * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "step_ms": round(ms_f + ms_b, 4), "timing": "mean of 10 back to back"}


def _time(fn, reps=10, warmup=3, flush=None):
    """Milliseconds of fn() on the current stream: the mean over reps back to back, or,
    with flush (a >= 512 MB device buffer), the median of reps each timed alone after
    the buffer is read through, so that a working set smaller than the 256 MB
    Infinity Cache (MALL) is read from HBM as in a real layer call."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if flush is None:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps
    times = []
    for r in range(reps):
        # evict by reading (a write flush would leave dirty lines whose write-back
        # then competes with the timed kernel)
        torch.sum(flush, dtype=torch.int64)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e))
    times.sort()
    return times[len(times) // 2]


def _mx_sweep(wfmt, flush, dev):
    """fp8-activation layer (MXFP4 or MXFP8 weights with MXFP8 activations, or fp8 with
    per-tensor scales) at H=7168, I=2048, 64 experts, top-8 over decode and prefill token
    counts, plus its two GEMM stages."""
    import numpy as np
    import torch
    import mixture_experts_expert_softmax_amd as M
    import moe_synth as S
    cw = S.w4a8_moe(seed=0, T=8192, wfmt=wfmt)
    pt = wfmt == "fp8"
    keys = ("x", "x_sf", "w1", "w1_sf", "w2", "w2_sf") + (("act_scale",) if pt else ())
    dw = {k_: torch.from_numpy(np.ascontiguousarray(getattr(cw, k_))).to(dev) for k_ in keys}
    lgw = torch.from_numpy(cw.logits).to(dev)
    per_expert_bytes = (dw["w1"][0].numel() + dw["w2"][0].numel()
                        + (0 if pt else dw["w1_sf"][0].numel() + dw["w2_sf"][0].numel()))
    sweep = {}
    for Tw in (1, 16, 128, 1024, 8192):
        idsw, wtsw = M.moe_route(lgw[:Tw], cw.top_k)
        outw = torch.empty((Tw, cw.H), dtype=torch.bfloat16, device=dev)
        wsw = torch.empty(M.moe_ffn_workspace_size(Tw, cw.H, cw.I, cw.num_experts, cw.top_k,
                                                   weight_format=wfmt), dtype=torch.uint8, device=dev)

        def mx_step():
            M.moe_route(lgw[:Tw], cw.top_k, idsw, wtsw)
            if pt:
                M.moe_ffn_forward_fp8(dw["x"][:Tw], dw["x_sf"], idsw, wtsw, dw["w1"], dw["w1_sf"],
                                      dw["w2"], dw["w2_sf"], dw["act_scale"], cw.num_experts,
                                      out=outw, workspace=wsw)
            else:
                M.moe_ffn_forward_mx(dw["x"][:Tw], dw["x_sf"][:Tw], idsw, wtsw, dw["w1"], dw["w1_sf"],
                                     dw["w2"], dw["w2_sf"], cw.num_experts, out=outw, workspace=wsw)
        touched = int(torch.unique(idsw).numel())
        small = touched * per_expert_bytes < (512 << 20)
        reps = 50 if small else (20 if Tw < 1024 else 10)
        ms_ = _time(mx_step, reps=reps, flush=flush if small else None)
        ms_graph = None
        if Tw <= 128:   # the same step captured once and replayed (prepared launches)
            g = _capture(mx_step)
            ms_graph = _time(g.replay, reps=reps, flush=flush if small else None)
        fl = 6.0 * cw.H * cw.I * Tw * cw.top_k
        wb = touched * per_expert_bytes
        sweep[str(Tw)] = {"ms": round(ms_, 4), "tflops": round(fl / (ms_ * 1e-3) / 1e12, 2),
                          "tokens_per_s": round(Tw / (ms_ * 1e-3), 1), "experts_touched": touched,
                          "timing": "median of 50, MALL flushed" if small else "mean",
                          "weight_gbs": round(wb / (ms_ * 1e-3) / 1e9, 1),
                          "hbm_frac_weights": round(wb / (ms_ * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "fp8_mfma_frac": round(fl / (ms_ * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)}
        if ms_graph is not None:
            sweep[str(Tw)]["graph_ms"] = round(ms_graph, 4)
        # the per-bucket tuner: time both tile families of FC1 / FC2 on this batch
        choice = M.moe_tune(dw["x"][:Tw], idsw, wtsw, dw["w1"], dw["w2"], cw.num_experts,
                            x_sf=dw["x_sf"] if pt else dw["x_sf"][:Tw], w1_sf=dw["w1_sf"],
                            w2_sf=dw["w2_sf"], act_scale=dw["act_scale"] if pt else None,
                            workspace=wsw)
        sweep[str(Tw)]["tuned_ms"] = round(_time(mx_step, reps=reps, flush=flush if small else None), 4)
        sweep[str(Tw)]["tuned_tiles"] = ["streaming" if ch else "256-row" for ch in choice]
        M.moe_tune_clear()
    # the two GEMM stages at T=8192 on their own
    srt = M.moe_sort(idsw, cw.num_experts)
    act = torch.empty((8192 * cw.top_k, cw.I), dtype=torch.uint8, device=dev)
    act_sf = torch.empty((8192 * cw.top_k, cw.I // 32), dtype=torch.uint8, device=dev)
    yw = torch.empty((8192 * cw.top_k, cw.H), dtype=torch.bfloat16, device=dev)
    if pt:
        ms1 = _time(lambda: M.moe_fc1_fp8(dw["x"], dw["x_sf"], dw["w1"], dw["w1_sf"], dw["act_scale"],
                                          srt["offs"], srt["p2e"], cw.top_k, cw.num_experts, act=act))
        ms2 = _time(lambda: M.moe_fc2_fp8(act, dw["act_scale"], dw["w2"], dw["w2_sf"], srt["offs"], 8192,
                                          cw.top_k, cw.num_experts, y=yw))
    else:
        ms1 = _time(lambda: M.moe_fc1_mx(dw["x"], dw["x_sf"], dw["w1"], dw["w1_sf"], srt["offs"],
                                         srt["p2e"], cw.top_k, cw.num_experts, act=act, act_sf=act_sf))
        ms2 = _time(lambda: M.moe_fc2_mx(act, act_sf, dw["w2"], dw["w2_sf"], srt["offs"], 8192,
                                         cw.top_k, cw.num_experts, y=yw))
    R = 8192 * cw.top_k
    sweep["8192_stages"] = {"fc1_ms": round(ms1, 4), "fc1_tflops": round(4.0 * cw.H * cw.I * R / (ms1 * 1e-3) / 1e12, 1),
                            "fc2_ms": round(ms2, 4), "fc2_tflops": round(2.0 * cw.H * cw.I * R / (ms2 * 1e-3) / 1e12, 1),
                            "peak_tflops_fp8": FP8_PEAK_TFLOPS}
    del dw, act, act_sf, yw
    return sweep


def _bgmv_points(flush, dev):
    """BGMV MoE-LoRA shrink + expand at the page's measured shape (hidden 3072, rank 32,
    top-2 contiguous pairs, 4 LoRAs x 8 experts) for 16, 2048 and 8192 tokens (the
    library's automatic choice of pipeline: per pair at 16, grouped by bin at 2048 and 8192). Bytes: the
    LoRA weights of the touched (LoRA, expert) pairs once, x read, y written (float32);
    per-pair weight bytes (every pair reads its A and B slices, mostly from cache)
    are reported beside them."""
    import numpy as np
    import torch
    import mixture_experts_expert_softmax_amd as M
    import moe_synth as S
    out = {}
    for T in (16, 2048, 8192):
        c = S.bgmv_case(seed=0, T=T, H=3072, rank=32, num_loras=4, E=8, top_k=2)
        d = [c.x.to(dev), c.lora_a.to(dev), c.lora_b.to(dev)] + [
            torch.from_numpy(v).to(dev) for v in (c.sorted_token_ids, c.expert_ids, c.lora_indices,
                                                  c.topk_weights)]
        y = torch.empty((T, 3072), dtype=torch.float32, device=dev)
        P = c.sorted_token_ids.shape[0]
        ws = torch.empty(M.moe_bgmv_workspace_bytes(T, P, 3072, 3072, 32, 4, 8), dtype=torch.uint8,
                         device=dev)
        fn = lambda: M.moe_bgmv(*d, c.num_experts, y_accum=y, workspace=ws)
        ms_ = _time(fn, reps=50, flush=flush)
        pairs = {(int(c.lora_indices[t]), int(e)) for t, e in zip(c.sorted_token_ids, c.expert_ids)}
        wbytes = len(pairs) * 2 * (32 * 3072 * 2)
        alg = wbytes + T * 3072 * 2 + T * 3072 * 4
        out[str(T)] = {"ms": round(ms_, 4), "pairs_per_s": round(P / (ms_ * 1e-3), 1),
                       "algorithmic_gbs": round(alg / (ms_ * 1e-3) / 1e9, 1),
                       "hbm_frac": round(alg / (ms_ * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "per_pair_weight_gbs": round(P * 2 * 32 * 3072 * 2 / (ms_ * 1e-3) / 1e9, 1),
                       "timing": "median of 50, MALL flushed"}
    return out


def secondary_measurements(progress):
    """The other hot-path rows at their own workloads (not the headline step):
    the standalone grouped GEMMs, the expert-shard forward, and routing / sort /
    finalize at sizes large enough to load HBM."""
    import numpy as np
    import torch
    import mixture_experts_expert_softmax_amd as M
    import moe_synth as S
    dev = "cuda"
    res = {}
    # read through between timed reps wherever the touched data is under ~0.5 GB
    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev)

    progress("secondary: tiny layer T=32 H=128 I=256 E=8 top-2")
    ct = S.tiny_moe(seed=0)
    lgt = torch.from_numpy(ct.logits).to(dev)
    xt, w1t, w2t = ct.x.to(dev), ct.w1.to(dev), ct.w2.to(dev)
    idt, wtt = M.moe_route(lgt, ct.top_k)
    outt = torch.empty((ct.T, ct.H), dtype=torch.bfloat16, device=dev)
    wst = torch.empty(M.moe_ffn_workspace_size(ct.T, ct.H, ct.I, ct.num_experts, ct.top_k),
                      dtype=torch.uint8, device=dev)

    def tiny_step():
        M.moe_route(lgt, ct.top_k, idt, wtt)
        M.moe_ffn_forward(xt, idt, wtt, w1t, w2t, ct.num_experts, out=outt, workspace=wst)
    ms_t = _time(tiny_step, reps=50)
    res["tiny"] = {"ms": round(ms_t, 4), "tokens_per_s": round(ct.T / (ms_t * 1e-3), 1),
                   "timing": "mean of 50 back to back (launch-latency bound)"}
    del xt, w1t, w2t

    progress("secondary: grouped GEMM E=16 sum_m=8192 K=2048 N=4096")
    c = S.grouped_gemm_case(seed=0)
    x, g, w = c.x.to(dev), c.g.to(dev), c.w.to(dev)
    offs = torch.from_numpy(c.offs).to(dev)
    Mr, K, N, E = c.sum_m, 2048, 4096, c.E
    fl = 2.0 * Mr * K * N
    yb = torch.empty((Mr, N), dtype=torch.bfloat16, device=dev)
    dxb = torch.empty((Mr, K), dtype=torch.bfloat16, device=dev)
    dwb = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    dwf = torch.empty((E, N, K), dtype=torch.float32, device=dev)
    gg = {}
    sws = torch.empty(M.lib().moe_gemm_split_workspace_size(), dtype=torch.uint8, device=dev)
    for name, fn in [("fwd", lambda: M.grouped_gemm_fwd(x, w, offs, out=yb, workspace=sws)),
                     ("dgrad", lambda: M.grouped_gemm_dgrad(g, w, offs, out=dxb, workspace=sws)),
                     ("wgrad_bf16", lambda: M.grouped_gemm_wgrad(g, x, offs, out=dwb)),
                     ("wgrad_f32", lambda: M.grouped_gemm_wgrad(g, x, offs, out=dwf))]:
        ms_ = _time(fn, reps=20, flush=flush)  # ~370 MB of operands
        gg[name] = {"ms": round(ms_, 4), "tflops": round(fl / (ms_ * 1e-3) / 1e12, 1),
                    "mfma_frac": round(fl / (ms_ * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    gg["group_sizes"] = c.sizes.tolist()
    gg["timing"] = "median of 20, MALL flushed; fwd / dgrad with the split workspace"
    del sws
    res["grouped_gemm"] = gg
    del x, g, w, yb, dxb, dwb, dwf

    progress("secondary: expert shard T=8192 H=7168 I=2048, 32 of 256 experts, top-8, SwiGLUStep")
    cs = S.expert_shard_moe(seed=0)
    lg = torch.from_numpy(cs.logits).to(dev)
    xs, w1s, w2s = cs.x.to(dev), cs.w1.to(dev), cs.w2.to(dev)
    lim = torch.from_numpy(cs.limits).to(dev)
    ids, wts = M.moe_route(lg, cs.top_k)
    outs = torch.empty((cs.T, cs.H), dtype=torch.bfloat16, device=dev)
    ws_bytes = M.moe_ffn_workspace_size(cs.T, cs.H, cs.I, cs.num_experts, cs.top_k, cs.num_local,
                                        cs.local_offset, "swiglu_step")
    wsp = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def shard_step():
        M.moe_route(lg, cs.top_k, ids, wts)
        M.moe_ffn_forward(xs, ids, wts, w1s, w2s, cs.num_experts, cs.num_local, cs.local_offset,
                          "swiglu_step", lim, out=outs, workspace=wsp)
    ms_ = _time(shard_step)
    srt = M.moe_sort(ids, cs.num_experts, cs.num_local, cs.local_offset)
    n_loc = int(srt["n_local"].item())
    fl = 6.0 * cs.H * cs.I * n_loc
    wbytes = (w1s.numel() + w2s.numel()) * 2
    res["expert_shard"] = {"ms": round(ms_, 4), "tflops": round(fl / (ms_ * 1e-3) / 1e12, 1),
                           "tokens_per_s": round(cs.T / (ms_ * 1e-3), 1), "n_local_routes": n_loc,
                           "weight_gbs": round(wbytes / (ms_ * 1e-3) / 1e9, 1)}
    del xs, w1s, w2s, wsp, outs

    for wfmt, key in (("mxfp4", "w4a8"), ("mxfp8", "mxfp8_weights"), ("fp8", "fp8_per_tensor")):
        progress(f"secondary: {wfmt} weights, MXFP8 activations, H=7168 I=2048 64 experts top-8")
        res[key] = _mx_sweep(wfmt, flush, dev)

    progress("secondary: BGMV MoE-LoRA H=3072 rank 32, 4 LoRAs x 8 experts, top-2")
    res["bgmv"] = _bgmv_points(flush, dev)

    progress("secondary: route + sort at T=262144, 256 experts, top-8")
    T2, E2, k2 = 262144, 256, 8
    lg2 = torch.from_numpy(S.route_logits(np.random.default_rng(1), T2, E2)).to(dev)
    ids2 = torch.empty((T2, k2), dtype=torch.int32, device=dev)
    w2t = torch.empty((T2, k2), dtype=torch.float32, device=dev)
    ms_r = _time(lambda: M.moe_route(lg2, k2, ids2, w2t))
    ws2 = torch.empty(M.lib().moe_sort_workspace_size(T2, k2, E2), dtype=torch.uint8, device=dev)
    so2 = M.moe_sort(ids2, E2, workspace=ws2)
    ms_s = _time(lambda: M.moe_sort(ids2, E2, workspace=ws2, out=so2), reps=20, flush=flush)  # 34 MB
    del flush
    route_bytes = T2 * E2 * 4 + T2 * k2 * 8
    sort_bytes = T2 * k2 * 4 * 2 + T2 * k2 * 8   # ids read twice, e2p + p2e written
    res["route_large"] = {"ms": round(ms_r, 4), "gbs": round(route_bytes / (ms_r * 1e-3) / 1e9, 1),
                          "hbm_frac": round(route_bytes / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    res["sort_large"] = {"ms": round(ms_s, 4), "gbs": round(sort_bytes / (ms_s * 1e-3) / 1e9, 1),
                         "hbm_frac": round(sort_bytes / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "note": "outputs preallocated; count, scan and scatter launches; median of 20, MALL flushed"}

    progress("secondary: finalize at T=65536, H=7168, top-8")
    T3, H3, k3 = 65536, 7168, 8
    e2p = torch.randperm(T3 * k3, device=dev).to(torch.int32)
    yr = torch.randn((T3 * k3, H3), device=dev).to(torch.bfloat16)
    w3 = torch.rand((T3, k3), device=dev)
    o3 = torch.empty((T3, H3), dtype=torch.bfloat16, device=dev)
    ms_f = _time(lambda: M.moe_finalize(yr, e2p, w3, out=o3))
    fb = T3 * k3 * H3 * 2 + T3 * H3 * 2 + T3 * k3 * 8
    res["finalize_large"] = {"ms": round(ms_f, 4), "gbs": round(fb / (ms_f * 1e-3) / 1e9, 1),
                             "hbm_frac": round(fb / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return res


def _profile_calls(name):
    """(description, list of (label, fn)) of one profiling workload; every fn is one
    library call (or a short chain) on inputs resident on the device."""
    import numpy as np
    import torch
    import mixture_experts_expert_softmax_amd as M
    import moe_synth as S
    dev = "cuda"
    if name in ("layer", "backward"):
        c = S.mixtral_moe(seed=0)
        x, w1, w2 = c.x.to(dev), c.w1.to(dev), c.w2.to(dev)
        lg = torch.from_numpy(c.logits).to(dev)
        ids, w = M.moe_route(lg, c.top_k)
        srt = M.moe_sort(ids, c.num_experts)
        ws = torch.empty(M.lib().moe_gemm_split_workspace_size(), dtype=torch.uint8, device=dev)
        act = M.moe_fc1(x, w1, srt["offs"], srt["p2e"], c.top_k, c.num_experts, workspace=ws)
        y = M.moe_fc2(act, w2, srt["offs"], c.T, c.top_k, c.num_experts, workspace=ws)
        out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=dev)
        if name == "backward":
            import ctypes
            dout = S.upstream_grad(0, c.T, c.H).to(dev)
            _, saved = M.moe_ffn_forward_train(x, ids, w, w1, w2, c.num_experts)
            d = M._train_desc(x, ids, w1, c.num_experts, None, 0, "swiglu")
            bws = torch.empty(M.lib().moe_ffn_backward_workspace_size(ctypes.byref(d)),
                              dtype=torch.uint8, device=dev)
            return ("Mixtral-shaped layer backward (T=4096, H=4096, I=14336, 8 experts, top-2)",
                    [("backward", lambda: M.moe_ffn_backward(dout, saved, x, ids, w, w1, w2,
                                                             c.num_experts, workspace=bws))])
        return ("Mixtral-shaped layer forward (T=4096, H=4096, I=14336, 8 experts, top-2)", [
            ("route", lambda: M.moe_route(lg, c.top_k, ids, w)),
            ("sort", lambda: M.moe_sort(ids, c.num_experts, out=srt)),
            ("fc1", lambda: M.moe_fc1(x, w1, srt["offs"], srt["p2e"], c.top_k, c.num_experts,
                                      act=act, workspace=ws)),
            ("fc2", lambda: M.moe_fc2(act, w2, srt["offs"], c.T, c.top_k, c.num_experts, dst=y,
                                      workspace=ws)),
            ("finalize", lambda: M.moe_finalize(y, srt["e2p"], w, out=out)),
            ("fc2_fused", lambda: M.moe_fc2(act, w2, srt["offs"], c.T, c.top_k, c.num_experts,
                                            finalize="fused", p2e=srt["p2e"], topk_weights=w,
                                            dst=out, workspace=ws))])
    if name == "grouped_gemm":
        c = S.grouped_gemm_case(seed=0)
        x, g, w = c.x.to(dev), c.g.to(dev), c.w.to(dev)
        offs = torch.from_numpy(c.offs).to(dev)
        ws = torch.empty(M.lib().moe_gemm_split_workspace_size(), dtype=torch.uint8, device=dev)
        yb = torch.empty((c.sum_m, 4096), dtype=torch.bfloat16, device=dev)
        dxb = torch.empty((c.sum_m, 2048), dtype=torch.bfloat16, device=dev)
        dwb = torch.empty((c.E, 4096, 2048), dtype=torch.bfloat16, device=dev)
        dwf = torch.empty((c.E, 4096, 2048), dtype=torch.float32, device=dev)
        return ("ragged grouped GEMM, 16 groups, sum_m=8192, K=2048, N=4096", [
            ("fwd", lambda: M.grouped_gemm_fwd(x, w, offs, out=yb, workspace=ws)),
            ("dgrad", lambda: M.grouped_gemm_dgrad(g, w, offs, out=dxb, workspace=ws)),
            ("wgrad_bf16", lambda: M.grouped_gemm_wgrad(g, x, offs, out=dwb)),
            ("wgrad_f32", lambda: M.grouped_gemm_wgrad(g, x, offs, out=dwf))])
    if name == "expert_shard":
        cs = S.expert_shard_moe(seed=0)
        lg = torch.from_numpy(cs.logits).to(dev)
        xs, w1s, w2s = cs.x.to(dev), cs.w1.to(dev), cs.w2.to(dev)
        lim = torch.from_numpy(cs.limits).to(dev)
        ids, wts = M.moe_route(lg, cs.top_k)
        outs = torch.empty((cs.T, cs.H), dtype=torch.bfloat16, device=dev)
        wsp = torch.empty(M.moe_ffn_workspace_size(cs.T, cs.H, cs.I, cs.num_experts, cs.top_k,
                                                   cs.num_local, cs.local_offset, "swiglu_step"),
                          dtype=torch.uint8, device=dev)
        return ("expert shard T=8192, H=7168, I=2048, experts 64..95 of 256, top-8, SwiGLUStep", [
            ("step", lambda: (M.moe_route(lg, cs.top_k, ids, wts),
                              M.moe_ffn_forward(xs, ids, wts, w1s, w2s, cs.num_experts, cs.num_local,
                                                cs.local_offset, "swiglu_step", lim, out=outs,
                                                workspace=wsp)))])
    if name.startswith("w4a8_"):
        Tw = int(name.split("_")[1])
        cw = S.w4a8_moe(seed=0, T=Tw, wfmt="mxfp4")
        dw = {k_: torch.from_numpy(np.ascontiguousarray(getattr(cw, k_))).to(dev)
              for k_ in ("x", "x_sf", "w1", "w1_sf", "w2", "w2_sf")}
        lgw = torch.from_numpy(cw.logits).to(dev)
        idsw, wtsw = M.moe_route(lgw, cw.top_k)
        outw = torch.empty((Tw, cw.H), dtype=torch.bfloat16, device=dev)
        wsw = torch.empty(M.moe_ffn_workspace_size(Tw, cw.H, cw.I, cw.num_experts, cw.top_k,
                                                   weight_format="mxfp4"), dtype=torch.uint8, device=dev)
        return (f"W4A8 layer T={Tw}, H=7168, I=2048, 64 experts, top-8 (MXFP4 weights, MXFP8 "
                "activations)", [
            ("step", lambda: (M.moe_route(lgw, cw.top_k, idsw, wtsw),
                              M.moe_ffn_forward_mx(dw["x"], dw["x_sf"], idsw, wtsw, dw["w1"],
                                                   dw["w1_sf"], dw["w2"], dw["w2_sf"], cw.num_experts,
                                                   out=outw, workspace=wsw)))])
    if name.startswith("bgmv_"):
        Tb = int(name.split("_")[1])
        c = S.bgmv_case(seed=0, T=Tb, H=3072, rank=32, num_loras=4, E=8, top_k=2)
        d = [c.x.to(dev), c.lora_a.to(dev), c.lora_b.to(dev)] + [
            torch.from_numpy(v).to(dev) for v in (c.sorted_token_ids, c.expert_ids, c.lora_indices,
                                                  c.topk_weights)]
        yb = torch.empty((Tb, 3072), dtype=torch.float32, device=dev)
        P = c.sorted_token_ids.shape[0]
        wsb = torch.empty(M.moe_bgmv_workspace_bytes(Tb, P, 3072, 3072, 32, 4, 8), dtype=torch.uint8,
                          device=dev)
        return (f"BGMV T={Tb}, hidden 3072, rank 32, top-2, 4 LoRAs x 8 experts", [
            ("bgmv", lambda: M.moe_bgmv(*d, c.num_experts, y_accum=yb, workspace=wsb))])
    if name == "route_sort":
        T2, E2, k2 = 262144, 256, 8
        lg2 = torch.from_numpy(S.route_logits(np.random.default_rng(1), T2, E2)).to(dev)
        ids2 = torch.empty((T2, k2), dtype=torch.int32, device=dev)
        w2t = torch.empty((T2, k2), dtype=torch.float32, device=dev)
        M.moe_route(lg2, k2, ids2, w2t)
        ws2 = torch.empty(M.lib().moe_sort_workspace_size(T2, k2, E2), dtype=torch.uint8, device=dev)
        so2 = M.moe_sort(ids2, E2, workspace=ws2)
        return ("route + sort, T=262144, 256 experts, top-8", [
            ("route", lambda: M.moe_route(lg2, k2, ids2, w2t)),
            ("sort", lambda: M.moe_sort(ids2, E2, workspace=ws2, out=so2))])
    if name == "finalize":
        T3, H3, k3 = 65536, 7168, 8
        e2p = torch.randperm(T3 * k3, device=dev).to(torch.int32)
        yr = torch.randn((T3 * k3, H3), device=dev).to(torch.bfloat16)
        w3 = torch.rand((T3, k3), device=dev)
        o3 = torch.empty((T3, H3), dtype=torch.bfloat16, device=dev)
        return ("finalize T=65536, H=7168, top-8", [
            ("finalize", lambda: M.moe_finalize(yr, e2p, w3, out=o3))])
    raise ValueError(name)


PROFILE_WORKLOADS = ("layer", "backward", "grouped_gemm", "expert_shard", "w4a8_1024", "w4a8_8192",
                     "route_sort", "finalize", "bgmv_2048")


def profile_workload(name, warmup=3, reps=5):
    """Run one workload's calls warmup + reps times and print their mean event times."""
    import torch
    torch.cuda.set_device(0)
    desc, calls = _profile_calls(name)
    res = {}
    for label, fn in calls:
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        res[label] = round(s.elapsed_time(e) / reps, 4)
    print(json.dumps({"profile": name, "workload": desc, "mean_ms": res}), flush=True)


if __name__ == "__main__":
    main()
