#!/usr/bin/env python3
"""Benchmark: one MoE layer forward pass on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input,
with every input already resident in HBM: route (top-k + renormalised
softmax) -> permute (group pairs by expert) -> gate/up projection with
SwiGLU, reading the token rows in place -> down projection -> combine: the
same kernels moe_forward launches.  Each stage is one C-ABI call of
libmoe.so on torch's current stream; HIP events on that stream bracket every
stage, so each stage's average duration is measured live over the timed
region.  The headline (value, ms_per_step) times the same K steps through the
fused entry point moe_forward, which launches these kernels back to back.

Prints ONE JSON line.  ``value`` = routed (token, expert) pairs per second of
the whole layer (moe_forward).  ``roofline`` describes the dominant kernel (the gate/up
grouped GEMM: algorithmic flops per launch / measured launch duration against
the MI355X dense bf16 MFMA peak).  ``cpu_baseline`` is the CPU oracle timed on
a bounded sample of the same workload on this host.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "routed token-expert pairs/sec per MoE layer; % bf16 MFMA peak; permute GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
GEMM_SOURCE = os.path.join(ROOT, "token_routing_expert_amd", "csrc", "grouped_ffn.hip")
STAGES = ["route", "permute", "gate_up", "down", "combine"]


def kernel_source_hash() -> str:
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic_record(workload: str):
    """Key/value lines ('key: value') of the counter summary for the gate/up
    kernel on this workload, or None.  The record carries the hash of the
    kernel source it was measured on; a changed kernel has no traffic."""
    path = os.path.join(PROFILES, f"gate_up_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.strip().lstrip("-* ")
        if ":" in line:
            k, v = line.split(":", 1)
            rec[k.strip().strip("`")] = v.strip().strip("`")
    return rec if "hbm_bytes_per_launch" in rec else None


def inp_seed(name: str) -> int:
    return int(workloads.CONFIGS[name]["seed"])


def to_device(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def algorithmic_work(inp, n_rows: int, live_experts: int):
    """Per-launch algorithmic bytes / flops of each stage (what the method must
    move or compute, not what a kernel happens to touch)."""
    T, d, E, k, I = inp.T, inp.d, inp.E, inp.k, inp.I
    s = 4 if inp.dtype == "f32" else 2
    P = T * k
    return {
        "route": {"bytes": (4 * T * E + 8 * P) if inp.logits is not None else 0},
        "permute": {"bytes": (T * d * s + n_rows * d * s if inp.dtype == "f32" else 0) + 16 * P},
        "gate_up": {"flops": 4 * n_rows * d * I,
                    "bytes": live_experts * 2 * d * I * s + n_rows * d * s + n_rows * I * s},
        "down": {"flops": 2 * n_rows * I * d,
                 "bytes": live_experts * d * I * s + n_rows * I * s + n_rows * d * s},
        "combine": {"bytes": n_rows * d * s + T * d * s + 8 * P},
    }


def cpu_baseline(inp, seconds: float):
    """Time the CPU oracle on a bounded sample of the workload."""
    import oracle
    threads = oracle.default_threads()
    rng = np.random.default_rng(12345)
    t0 = time.perf_counter()
    if inp.logits is not None:
        idx, w = oracle.route(inp.logits, inp.k)
    else:
        idx = inp.pair_expert.reshape(inp.T, inp.k)
        w = inp.pair_w.reshape(inp.T, inp.k).astype(np.float64)
    oracle.dispatch(idx.reshape(-1), inp.k, inp.E)
    t_index = time.perf_counter() - t0
    probe = rng.choice(inp.T, size=min(inp.T, max(threads, 4)), replace=False)
    t0 = time.perf_counter()
    oracle.moe_tokens(inp.x, idx, w, inp.w_gate_up, inp.w_down, tokens=probe, nthreads=threads)
    per_tok = (time.perf_counter() - t0) / len(probe)
    n = int(min(inp.T, max(len(probe), (seconds - t_index) / max(per_tok, 1e-9))))
    sample = np.sort(rng.choice(inp.T, size=n, replace=False))
    t0 = time.perf_counter()
    oracle.moe_tokens(inp.x, idx, w, inp.w_gate_up, inp.w_down, tokens=sample, nthreads=threads)
    t_ffn = time.perf_counter() - t0
    # the index work is charged in proportion to the sample
    t_total = t_ffn + t_index * n / inp.T
    return {
        "value": n * inp.k / t_total,
        "unit": "pairs/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} of {inp.T} tokens ({n * inp.k} pairs) through experts+combine in float64, "
                  f"plus route+dispatch over all tokens charged pro rata; {t_total:.1f} s",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=workloads.ORDER[1], choices=workloads.ORDER)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="before the steps, run one plain device copy of this many MiB (a known-size "
                         "reference for HBM byte counters under rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer has no "
              "multi-GPU path in this build", file=sys.stderr)
        return 2

    import torch
    import token_routing_expert_amd as tre

    lib = tre.load()
    inp = workloads.make(args.workload)
    T, d, E, k, I = inp.T, inp.d, inp.E, inp.k, inp.I
    P = T * k
    dev_dtype = torch.float32 if inp.dtype == "f32" else torch.bfloat16
    dt = tre.MOE_F32 if inp.dtype == "f32" else tre.MOE_BF16

    x = to_device(inp.x, torch)
    wgu = to_device(inp.w_gate_up, torch)
    wd = to_device(inp.w_down, torch)
    if inp.logits is not None:
        logits = to_device(inp.logits, torch)
        topk_idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        topk_w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    else:
        logits = None
        topk_idx = to_device(inp.pair_expert.reshape(T, k), torch)
        topk_w = to_device(inp.pair_w.reshape(T, k), torch)
    gather_off = inp.dtype == "f32"
    x_perm = torch.empty((P, d), dtype=dev_dtype, device="cuda") if gather_off else None
    row_token = torch.empty(P, dtype=torch.int32, device="cuda")
    pair_row = torch.empty(P, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    h = torch.empty((P, I), dtype=dev_dtype, device="cuda")
    y_perm = torch.empty((P, d), dtype=dev_dtype, device="cuda")
    out = torch.empty((T, d), dtype=dev_dtype, device="cuda")
    pws_bytes = lib.moe_permute_workspace_size(T, k, E)
    pws = torch.empty(max(pws_bytes, 1), dtype=torch.uint8, device="cuda")
    fws_bytes = lib.moe_forward_workspace_size(T, d, E, k, I, dt)
    fws = torch.empty(max(fws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def ptr(t):
        return None if t is None else t.data_ptr()

    # raw C-ABI calls with the pointers marshalled once
    calls = {
        "route": (lambda: lib.moe_route_topk(ptr(logits), T, E, k, ptr(topk_idx), ptr(topk_w), sp))
        if logits is not None else (lambda: 0),
        # bf16: the index only, then the projection reads token rows in place
        # (what moe_forward does); float32: rows are moved
        "permute": lambda: lib.moe_permute(ptr(x), dt, T, d, k, ptr(topk_idx), E, ptr(x_perm) if gather_off else None,
                                           ptr(row_token), ptr(pair_row), ptr(offsets), ptr(pws), pws_bytes, sp),
        "gate_up": lambda: lib.moe_gate_up_swiglu(ptr(x_perm) if gather_off else ptr(x), ptr(offsets), P, E, d, I,
                                                  ptr(wgu), dt, None if gather_off else ptr(row_token), T, ptr(h), sp),
        "down": lambda: lib.moe_down_proj(ptr(h), ptr(offsets), P, E, d, I, ptr(wd), dt, ptr(y_perm), sp),
        "combine": lambda: lib.moe_combine(ptr(y_perm), P, ptr(pair_row), ptr(topk_w), T, k, d, dt, ptr(out), sp),
    }

    def fused():
        return lib.moe_forward(ptr(x), ptr(logits), T, d, E, k, I, ptr(wgu), ptr(wd), dt, ptr(topk_idx),
                               ptr(topk_w), None, None, None, ptr(out), ptr(fws), fws_bytes, sp)

    def run_step(events=None):
        for i, name in enumerate(STAGES):
            if events is not None:
                events[i].record(stream)
            st = calls[name]()
            if st != 0:
                raise RuntimeError(f"{name} failed with status {st}")
        if events is not None:
            events[len(STAGES)].record(stream)

    if args.copy_calibration_mb > 0:
        # a device-to-device copy of known size whose source is not cache
        # resident (a 1 GiB write in between evicts the 256 MB Infinity Cache)
        n = args.copy_calibration_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        flush.fill_(2)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, flush
    def run_fused():
        st = fused()
        if st != 0:
            raise RuntimeError(f"moe_forward failed with status {st}")

    for _ in range(args.warmup):
        run_step()
        run_fused()
    torch.cuda.synchronize()
    n_rows = int(offsets[E].item())
    counts = (offsets[1:] - offsets[:-1]).cpu().numpy()
    live = int((counts > 0).sum())

    # ---- timed region 1 (the headline): exactly K layer steps through the
    # fused entry point moe_forward ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_fused()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # ---- timed region 2: the same K steps as separate C-ABI calls with HIP
    # events on the stream around every stage (per-stage durations, roofline)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.steps):
        run_step(evs[st])
    torch.cuda.synchronize()
    staged_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    stage_ms = {name: float(np.mean([evs[st][i].elapsed_time(evs[st][i + 1]) for st in range(args.steps)]))
                for i, name in enumerate(STAGES)}
    gpu_ms = float(np.mean([evs[st][0].elapsed_time(evs[st][len(STAGES)]) for st in range(args.steps)]))

    # ---- timed region 2b: the same layer captured once as a HIP graph and
    # replayed K times (what a decode loop would do; the library records no
    # host work, so the whole layer is one graph) ----
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        st = lib.moe_forward(ptr(x), ptr(logits), T, d, E, k, I, ptr(wgu), ptr(wd), dt, ptr(topk_idx),
                             ptr(topk_w), None, None, None, ptr(out), ptr(fws), fws_bytes, cap.cuda_stream)
        if st != 0:
            raise RuntimeError(f"moe_forward (captured) failed with status {st}")
    for _ in range(args.warmup):
        graph.replay()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / args.steps
    del graph

    # ---- timed region 2c: the permutation with its row moves (moe_permute
    # with x_perm), the step as the benchmark defines it: each token row read
    # once and written to its k grouped rows, plus the index arrays.  The
    # fused bf16 layer skips the row copy (its gate/up reads token rows in
    # place), so this is reported beside the layer.
    xp_rows = torch.empty((P, d), dtype=dev_dtype, device="cuda")
    pr_tok = torch.empty(P, dtype=torch.int32, device="cuda")
    pr_row = torch.empty(P, dtype=torch.int32, device="cuda")
    pr_off = torch.empty(E + 1, dtype=torch.int32, device="cuda")

    def run_permute_rows():
        st = lib.moe_permute(ptr(x), dt, T, d, k, ptr(topk_idx), E, ptr(xp_rows), ptr(pr_tok), ptr(pr_row),
                             ptr(pr_off), ptr(pws), pws_bytes, sp)
        if st != 0:
            raise RuntimeError(f"moe_permute failed with status {st}")
    for _ in range(args.warmup):
        run_permute_rows()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    p0.record(stream)
    for _ in range(args.steps):
        run_permute_rows()
    p1.record(stream)
    torch.cuda.synchronize()
    pr_ms = p0.elapsed_time(p1) / args.steps
    s_elem = 4 if inp.dtype == "f32" else 2
    pr_bytes = T * d * s_elem * (1 + k) + 16 * P
    permute_rows = {"ms": round(pr_ms, 5), "bytes_per_call": pr_bytes,
                    "gbs": round(pr_bytes / (pr_ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(pr_bytes / (pr_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del xp_rows

    # ---- timed region 3 (reported beside the layer, not part of it): the
    # router projection fused with routing, x @ W_r^T then top-k, on the
    # workload's tokens and a seeded router weight [E, d] ----
    router = None
    if logits is not None:
        w_r = to_device(workloads.router_weight(inp), torch)
        r_idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        r_w = torch.empty((T, k), dtype=torch.float32, device="cuda")

        def run_router():
            st = lib.moe_route_project(ptr(x), ptr(w_r), dt, T, d, E, k, None, ptr(r_idx), ptr(r_w), sp)
            if st != 0:
                raise RuntimeError(f"moe_route_project failed with status {st}")
        for _ in range(args.warmup):
            run_router()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            run_router()
        ev1.record(stream)
        torch.cuda.synchronize()
        r_ms = ev0.elapsed_time(ev1) / args.steps
        s_el = 4 if inp.dtype == "f32" else 2
        r_bytes = T * d * s_el + E * d * s_el + 8 * T * k
        r_flops = 2 * T * d * E
        router = {"ms": round(r_ms, 5), "bound": "hbm", "bytes_per_launch": r_bytes,
                  "gbs": round(r_bytes / (r_ms * 1e-3) / 1e9, 1),
                  "hbm_frac": round(r_bytes / (r_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                  "tflops": round(r_flops / (r_ms * 1e-3) / 1e12, 2)}

    # ---- timed region 4 (reported beside the layer): the layer's backward
    # pass, moe_backward, which recomputes the forward it needs ----
    backward = None
    if inp.dtype == "bf16":
        rng = np.random.default_rng([inp_seed(args.workload), 99])
        dout = to_device(workloads.bf16_bits(rng.normal(size=(T, d)).astype(np.float32)), torch)
        gdx = torch.empty((T, d), dtype=dev_dtype, device="cuda")
        gwgu = torch.empty((E, d, 2 * I), dtype=dev_dtype, device="cuda")
        gwd = torch.empty((E, I, d), dtype=dev_dtype, device="cuda")
        gtw = torch.empty((T, k), dtype=torch.float32, device="cuda")
        glg = torch.empty((T, E), dtype=torch.float32, device="cuda") if logits is not None else None
        b_idx = torch.empty((T, k), dtype=torch.int32, device="cuda") if logits is not None else topk_idx
        b_w = torch.empty((T, k), dtype=torch.float32, device="cuda") if logits is not None else topk_w
        bws_bytes = lib.moe_backward_workspace_size(T, d, E, k, I, dt)
        bws = torch.empty(max(bws_bytes, 1), dtype=torch.uint8, device="cuda")

        def run_backward(recompute=1):
            st = lib.moe_backward(ptr(x), ptr(logits), T, d, E, k, I, ptr(wgu), ptr(wd), dt, ptr(b_idx), ptr(b_w),
                                  ptr(dout), ptr(gdx), ptr(gwgu), ptr(gwd), ptr(gtw), ptr(glg), recompute, ptr(bws),
                                  bws_bytes, sp)
            if st != 0:
                raise RuntimeError(f"moe_backward failed with status {st}")

        def run_forward_train():
            st = lib.moe_forward_train(ptr(x), ptr(logits), T, d, E, k, I, ptr(wgu), ptr(wd), dt, ptr(b_idx),
                                       ptr(b_w), ptr(gout), ptr(bws), bws_bytes, sp)
            if st != 0:
                raise RuntimeError(f"moe_forward_train failed with status {st}")
        gout = torch.empty((T, d), dtype=dev_dtype, device="cuda")

        def timed(fn, n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n
        for _ in range(args.warmup):
            run_backward()
        b_ms = timed(run_backward, args.steps)
        # a training step: the forward that keeps its intermediates, then the
        # backward from them (events around the pair, and around each)
        for _ in range(args.warmup):
            run_forward_train()
            run_backward(0)
        step_ms = timed(lambda: (run_forward_train(), run_backward(0)), args.steps)
        ft_ms = timed(run_forward_train, args.steps)
        bs_ms = timed(lambda: run_backward(0), args.steps)
        # matrix products per call: the recomputed forward (6 n d I) and the
        # gradients (dh 2, dW_down 2, dx 4, dW_gate_up 4: 12 n d I)
        b_flops = 18 * n_rows * d * I
        backward = {"ms": round(b_ms, 5), "flops_per_call": b_flops,
                    "tflops": round(b_flops / (b_ms * 1e-3) / 1e12, 1),
                    "mfma_frac": round(b_flops / (b_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "pairs_per_s": P / (b_ms * 1e-3),
                    # training step: 6 n d I (forward) + 12 n d I (gradients), no recompute
                    "training_step": {"ms": round(step_ms, 5), "forward_train_ms": round(ft_ms, 5),
                                      "backward_saved_ms": round(bs_ms, 5),
                                      "tflops": round(18 * n_rows * d * I / (step_ms * 1e-3) / 1e12, 1),
                                      "pairs_per_s": P / (step_ms * 1e-3)}}
        del gdx, gwgu, gwd, bws, gout

    work = algorithmic_work(inp, n_rows, live)
    peak_mm = PEAK_F32_TFLOPS if inp.dtype == "f32" else PEAK_BF16_TFLOPS
    kernels = {}
    for name in STAGES:
        ms = stage_ms[name]
        w = work[name]
        ent = {"ms": round(ms, 5)}
        if ms > 0 and w.get("bytes"):
            ent["gbs"] = round(w["bytes"] / (ms * 1e-3) / 1e9, 1)
            ent["hbm_frac"] = round(ent["gbs"] / PEAK_HBM_GBS, 4)
        if ms > 0 and w.get("flops"):
            ent["tflops"] = round(w["flops"] / (ms * 1e-3) / 1e12, 1)
            ent["mfma_frac"] = round(ent["tflops"] / peak_mm, 4)
        kernels[name] = ent

    gu = kernels["gate_up"]
    traffic = None
    rec = read_traffic_record(args.workload)
    if rec is not None and rec.get("source_sha256_16") == kernel_source_hash():
        traffic = float(rec["hbm_bytes_per_launch"])
    roofline = {
        "bound": "mfma",
        "kernel": "gate/up grouped GEMM + SwiGLU (dma::k_grouped_gemm<1, false, ...>, tile shape chosen per call)" if inp.dtype == "bf16"
                  else "gate/up grouped FFN (k_ffn_gate_up_f32)",
        "achieved": gu.get("tflops"),
        "peak": peak_mm,
        "unit": "TFLOP/s",
        "frac": gu.get("mfma_frac"),
        "traffic": traffic,
        "flops_per_launch": work["gate_up"]["flops"],
        "launch_ms": gu["ms"],
    }

    result = {
        "metric": METRIC,
        "value": P / (ms_per_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "d": d, "E": E, "k": k, "I": I, "pairs": P,
                   "routed_rows": n_rows, "live_experts": live},
        "roofline": roofline,
        "kernels": kernels,
        "staged_ms_per_step": staged_ms,
        "staged_gpu_ms_per_step": gpu_ms,
        "graph_ms_per_step": graph_ms,
        "permute_gbs": permute_rows["gbs"],
        "permute_rows": permute_rows,
        "router_projection": router,
        "backward": backward,
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
