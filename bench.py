#!/usr/bin/env python3
"""Benchmark: one MoE layer forward pass on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input,
with every input already resident in HBM: route (top-k + renormalised
softmax) -> permute (group pairs by expert) -> gate/up projection with
SwiGLU, reading the token rows in place -> down projection -> combine: the
kernels the fused entry point moe_forward launches.

Timing is HBM-honest: before every timed step a scratch buffer larger than
the 256 MB Infinity Cache (512 MiB by default) is read on the same stream,
so no operand of the step is served from a cache left warm by the step
before (a read, so that no dirty lines are left for the step to write
back); HIP events on the stream bracket the step itself (not the flush).
The headline (value, ms_per_step) is K such steps through moe_forward; the
same K steps run again as separate C-ABI calls with events between the
stages, which gives every kernel's average duration; a warm figure (steps
back to back, no flush) is reported beside it.

Prints ONE JSON line.  ``value`` = routed (token, expert) pairs per second of
the whole layer.  ``roofline`` describes the dominant kernel, the gate/up
grouped GEMM: its algorithmic bytes and flops per launch against its
measured launch duration, taken against the bound its arithmetic intensity
puts it under (HBM below the ridge point of 2500 TFLOP/s / 8 TB/s, MFMA
above), with the other fraction beside it.  ``cpu_baseline`` is the CPU
oracle timed on a bounded sample of the same workload on this host.

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


def host_cpu():
    """What the host offers the oracle: the CPU model, the logical CPUs the
    machine reports and the ones this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count() or 1
    return {"cpu_model": model, "host_cpus": os.cpu_count() or 1, "allowed_cpus": allowed}


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
    host = host_cpu()
    return {
        "value": n * inp.k / t_total,
        "unit": "pairs/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} of {inp.T} tokens ({n * inp.k} pairs) through experts+combine in float64, "
                  f"plus route+dispatch over all tokens charged pro rata; {t_total:.1f} s",
        **host,
        "thread_cap": f"{oracle.THREAD_CAP} threads at most: the CPU share one GPU is given on a shared "
                      f"multi-GPU host; here {threads} of {host['allowed_cpus']} allowed CPUs",
    }


class Layer:
    """One workload resident on the GPU, with raw C-ABI calls whose pointers
    are marshalled once."""

    def __init__(self, lib, tre, torch, inp):
        self.lib, self.torch, self.inp = lib, torch, inp
        T, d, E, k, I = inp.T, inp.d, inp.E, inp.k, inp.I
        P = T * k
        self.P = P
        dev_dtype = torch.float32 if inp.dtype == "f32" else torch.bfloat16
        self.dev_dtype = dev_dtype
        dt = tre.MOE_F32 if inp.dtype == "f32" else tre.MOE_BF16
        self.dt = dt
        self.x = to_device(inp.x, torch)
        self.wgu = to_device(inp.w_gate_up, torch)
        self.wd = to_device(inp.w_down, torch)
        if inp.logits is not None:
            self.logits = to_device(inp.logits, torch)
            self.topk_idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
            self.topk_w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        else:
            self.logits = None
            self.topk_idx = to_device(inp.pair_expert.reshape(T, k), torch)
            self.topk_w = to_device(inp.pair_w.reshape(T, k), torch)
        gather_off = inp.dtype == "f32"
        self.x_perm = torch.empty((P, d), dtype=dev_dtype, device="cuda") if gather_off else None
        self.row_token = torch.empty(P, dtype=torch.int32, device="cuda")
        self.pair_row = torch.empty(P, dtype=torch.int32, device="cuda")
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        self.h = torch.empty((P, I), dtype=dev_dtype, device="cuda")
        self.y_perm = torch.empty((P, d), dtype=dev_dtype, device="cuda")
        self.out = torch.empty((T, d), dtype=dev_dtype, device="cuda")
        self.pws_bytes = lib.moe_permute_workspace_size(T, k, E)
        self.pws = torch.empty(max(self.pws_bytes, 1), dtype=torch.uint8, device="cuda")
        self.fws_bytes = lib.moe_forward_workspace_size(T, d, E, k, I, dt)
        self.fws = torch.empty(max(self.fws_bytes, 1), dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.current_stream()
        sp = self.stream.cuda_stream
        ptr = self.ptr
        self.calls = {
            "route": (lambda: lib.moe_route_topk(ptr(self.logits), T, E, k, ptr(self.topk_idx), ptr(self.topk_w),
                                                 sp)) if self.logits is not None else (lambda: 0),
            # bf16: the index only, then the projection reads token rows in
            # place (what moe_forward does); float32: rows are moved
            "permute": lambda: lib.moe_permute(ptr(self.x), dt, T, d, k, ptr(self.topk_idx), E,
                                               ptr(self.x_perm) if gather_off else None, ptr(self.row_token),
                                               ptr(self.pair_row), ptr(self.offsets), ptr(self.pws), self.pws_bytes,
                                               sp),
            "gate_up": lambda: lib.moe_gate_up_swiglu(ptr(self.x_perm) if gather_off else ptr(self.x),
                                                      ptr(self.offsets), P, E, d, I, ptr(self.wgu), dt,
                                                      None if gather_off else ptr(self.row_token), T, ptr(self.h),
                                                      sp),
            "down": lambda: lib.moe_down_proj(ptr(self.h), ptr(self.offsets), P, E, d, I, ptr(self.wd), dt,
                                              ptr(self.y_perm), sp),
            "combine": lambda: lib.moe_combine(ptr(self.y_perm), P, ptr(self.pair_row), ptr(self.topk_w), T, k, d,
                                               dt, ptr(self.out), sp),
        }

    @staticmethod
    def ptr(t):
        return None if t is None else t.data_ptr()

    def fused(self, stream=None):
        inp, ptr = self.inp, self.ptr
        sp = (stream or self.stream).cuda_stream
        st = self.lib.moe_forward(ptr(self.x), ptr(self.logits), inp.T, inp.d, inp.E, inp.k, inp.I, ptr(self.wgu),
                                  ptr(self.wd), self.dt, ptr(self.topk_idx), ptr(self.topk_w), None, None, None,
                                  ptr(self.out), ptr(self.fws), self.fws_bytes, sp)
        if st != 0:
            raise RuntimeError(f"moe_forward failed with status {st}")

    def staged(self, events=None):
        for i, name in enumerate(STAGES):
            if events is not None:
                events[i].record(self.stream)
            st = self.calls[name]()
            if st != 0:
                raise RuntimeError(f"{name} failed with status {st}")
        if events is not None:
            events[len(STAGES)].record(self.stream)


class Flush:
    """Reads a scratch buffer larger than the Infinity Cache on the stream, so
    that the next step finds none of its operands in L2 or the Infinity Cache
    and reads them from HBM.  A read, not a write: a written buffer would
    leave the caches full of dirty lines whose write-back the next step would
    pay for."""

    def __init__(self, torch, mib: int):
        self.buf = None
        if mib > 0:
            self.buf = torch.zeros((mib << 20) // 4, dtype=torch.float32, device="cuda")
            torch.cuda.synchronize()

    def __call__(self):
        if self.buf is not None:
            self.buf.sum()


def time_layer(torch, layer, flush, steps: int, warmup: int):
    """Cold steps through moe_forward (flush, event, layer, event) and the
    same steps staged, with events between the kernels; then warm steps back
    to back.  Returns the timings in ms."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    stream = layer.stream
    for _ in range(warmup):
        flush()
        layer.staged()
        flush()
        layer.fused()
    torch.cuda.synchronize()

    # cold fused steps: exactly `steps` of them, synchronised on both sides
    pairs = [(ev(), ev()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in pairs:
        flush()
        a.record(stream)
        layer.fused()
        b.record(stream)
    torch.cuda.synchronize()
    wall_with_flush = (time.perf_counter() - t0) * 1e3 / steps
    cold = [a.elapsed_time(b) for a, b in pairs]

    # cold staged steps (per-kernel durations)
    evs = [[ev() for _ in range(len(STAGES) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for st in range(steps):
        flush()
        layer.staged(evs[st])
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([evs[st][i].elapsed_time(evs[st][i + 1]) for st in range(steps)]))
                for i, name in enumerate(STAGES)}
    staged_ms = float(np.mean([evs[st][0].elapsed_time(evs[st][len(STAGES)]) for st in range(steps)]))

    # warm steps back to back (operands partly cache-resident)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.fused()
    torch.cuda.synchronize()
    warm = (time.perf_counter() - t0) * 1e3 / steps
    return {"cold_ms": float(np.mean(cold)), "cold_min_ms": float(np.min(cold)),
            "cold_median_ms": float(np.median(cold)), "wall_ms_with_flush": wall_with_flush,
            "warm_ms": warm, "stage_ms": stage_ms, "staged_ms": staged_ms}


def kernel_table(inp, stage_ms, n_rows, live):
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
    return kernels, work, peak_mm


def roofline_of(inp, kernels, work, peak_mm, workload):
    """The dominant kernel (gate/up) against the bound its arithmetic
    intensity puts it under."""
    gu = kernels["gate_up"]
    w = work["gate_up"]
    ridge = peak_mm * 1e12 / (PEAK_HBM_GBS * 1e9)
    ai = w["flops"] / w["bytes"] if w["bytes"] else float("inf")
    traffic = None
    rec = read_traffic_record(workload)
    if rec is not None and rec.get("source_sha256_16") == kernel_source_hash():
        traffic = float(rec["hbm_bytes_per_launch"])
    kernel = ("gate/up grouped GEMM + SwiGLU (dma::k_grouped_gemm<1, false, ...>, tile shape chosen per call)"
              if inp.dtype == "bf16" else "gate/up grouped GEMM + SwiGLU, float32 MFMA (k_grouped_gemm_f32<true>)")
    common = {"kernel": kernel, "traffic": traffic, "flops_per_launch": w["flops"], "bytes_per_launch": w["bytes"],
              "arithmetic_intensity": round(ai, 1), "ridge": round(ridge, 1), "launch_ms": gu["ms"]}
    if ai < ridge:
        return {"bound": "hbm", "achieved": gu.get("gbs"), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gu.get("hbm_frac"), **common,
                "mfma": {"achieved": gu.get("tflops"), "peak": peak_mm, "unit": "TFLOP/s",
                         "frac": gu.get("mfma_frac")}}
    return {"bound": "mfma", "achieved": gu.get("tflops"), "peak": peak_mm, "unit": "TFLOP/s",
            "frac": gu.get("mfma_frac"), **common,
            "hbm": {"achieved": gu.get("gbs"), "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gu.get("hbm_frac")}}


def routed(torch, layer):
    E = layer.inp.E
    n_rows = int(layer.offsets[E].item())
    counts = (layer.offsets[1:] - layer.offsets[:-1]).cpu().numpy()
    return n_rows, int((counts > 0).sum())


def measure_extra(lib, tre, torch, name, flush, steps, warmup):
    """The layer and its kernels on another workload (cold), for the line."""
    inp = workloads.make(name)
    layer = Layer(lib, tre, torch, inp)
    t = time_layer(torch, layer, flush, steps, warmup)
    n_rows, live = routed(torch, layer)
    kernels, work, peak_mm = kernel_table(inp, t["stage_ms"], n_rows, live)
    res = {"ms_per_step": round(t["cold_ms"], 5), "pairs_per_s": layer.P / (t["cold_ms"] * 1e-3),
           "warm_ms_per_step": round(t["warm_ms"], 5), "roofline": roofline_of(inp, kernels, work, peak_mm, name),
           "kernels": kernels}
    del layer
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_e128", choices=workloads.ORDER,
                    help="the headline workload (default: the largest single-GPU one, the whole layer with "
                         "128 experts)")
    ap.add_argument("--extra", default="small_bf16",
                    help="comma-separated workloads measured beside the headline (cold layer and kernels), "
                         "or 'none'")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="MiB of scratch read before every timed step (0: no flush)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the router projection, permute-with-rows, graph, backward and tiled-weight "
                         "measurements")
    ap.add_argument("--extras", default="graph,permute,router,backward,tiled",
                    help="comma-separated measurements beside the layer (graph, permute, router, backward, "
                         "tiled); "
                         "--no-extras is the same as none")
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
    layer = Layer(lib, tre, torch, inp)
    stream = layer.stream
    sp = stream.cuda_stream
    dev_dtype, dt = layer.dev_dtype, layer.dt
    ptr = layer.ptr
    x, wgu, wd, logits = layer.x, layer.wgu, layer.wd, layer.logits
    topk_idx, topk_w = layer.topk_idx, layer.topk_w
    flush = Flush(torch, args.flush_mb)

    if args.copy_calibration_mb > 0:
        # a device-to-device copy of known size whose source is not cache
        # resident (a 1 GiB write in between evicts the 256 MB Infinity Cache)
        n = args.copy_calibration_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        big = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        big.fill_(2)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, big

    # ---- timed regions 1 and 2: K cold layer steps through moe_forward (the
    # headline), then the same K steps staged with events between kernels ----
    t = time_layer(torch, layer, flush, args.steps, args.warmup)
    ms_per_step = t["cold_ms"]
    n_rows, live = routed(torch, layer)
    kernels, work, peak_mm = kernel_table(inp, t["stage_ms"], n_rows, live)
    roofline = roofline_of(inp, kernels, work, peak_mm, args.workload)

    graph_ms = permute_rows = router = backward = tiled = None
    extras = set() if args.no_extras else {e for e in args.extras.split(",") if e and e != "none"}
    if extras:
        if "graph" in extras:
            # ---- timed region 3: the same layer captured once as a HIP graph and
            # replayed K times back to back (what a decode loop would do; the
            # library records no host work, so the whole layer is one graph) ----
            cap = torch.cuda.Stream()
            cap.wait_stream(stream)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=cap):
                layer.fused(stream=cap)
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

        def timed_cold(fn, n):
            # n cold calls: flush, event, call, event
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            torch.cuda.synchronize()
            for a, b in pairs:
                flush()
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            return float(np.mean([a.elapsed_time(b) for a, b in pairs]))

        if "permute" in extras:
            # ---- timed region 4: the permutation with its row moves (moe_permute
            # with x_perm), the step as the benchmark defines it: each token row
            # read once and written to its k grouped rows, plus the index arrays.
            # The fused bf16 layer skips the row copy (its gate/up reads token rows
            # in place), so this is reported beside the layer.
            xp_rows = torch.empty((P, d), dtype=dev_dtype, device="cuda")
            pr_tok = torch.empty(P, dtype=torch.int32, device="cuda")
            pr_row = torch.empty(P, dtype=torch.int32, device="cuda")
            pr_off = torch.empty(E + 1, dtype=torch.int32, device="cuda")

            def run_permute_rows():
                st = lib.moe_permute(ptr(x), dt, T, d, k, ptr(topk_idx), E, ptr(xp_rows), ptr(pr_tok), ptr(pr_row),
                                     ptr(pr_off), ptr(layer.pws), layer.pws_bytes, sp)
                if st != 0:
                    raise RuntimeError(f"moe_permute failed with status {st}")
            for _ in range(args.warmup):
                run_permute_rows()
            pr_ms = timed_cold(run_permute_rows, args.steps)
            s_elem = 4 if inp.dtype == "f32" else 2
            pr_bytes = T * d * s_elem * (1 + k) + 16 * P
            permute_rows = {"ms": round(pr_ms, 5), "bytes_per_call": pr_bytes,
                            "gbs": round(pr_bytes / (pr_ms * 1e-3) / 1e9, 1),
                            "hbm_frac": round(pr_bytes / (pr_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            del xp_rows

        # ---- timed region 5 (beside the layer, not part of it): the router
        # projection fused with routing, x @ W_r^T then top-k, on the
        # workload's tokens and a seeded router weight [E, d] ----
        if "router" in extras and logits is not None:
            w_r = to_device(workloads.router_weight(inp), torch)
            r_idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
            r_w = torch.empty((T, k), dtype=torch.float32, device="cuda")

            def run_router():
                st = lib.moe_route_project(ptr(x), ptr(w_r), dt, T, d, E, k, None, ptr(r_idx), ptr(r_w), sp)
                if st != 0:
                    raise RuntimeError(f"moe_route_project failed with status {st}")
            for _ in range(args.warmup):
                run_router()
            r_ms = timed_cold(run_router, args.steps)
            s_el = 4 if inp.dtype == "f32" else 2
            r_bytes = T * d * s_el + E * d * s_el + 8 * T * k
            r_flops = 2 * T * d * E
            router = {"ms": round(r_ms, 5), "bound": "hbm", "bytes_per_launch": r_bytes,
                      "gbs": round(r_bytes / (r_ms * 1e-3) / 1e9, 1),
                      "hbm_frac": round(r_bytes / (r_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "tflops": round(r_flops / (r_ms * 1e-3) / 1e12, 2)}

        # ---- timed region 6 (beside the layer): the layer's backward pass,
        # moe_backward, which recomputes the forward it needs, and a training
        # step (the forward that keeps its intermediates, then the backward
        # from them) ----
        if "backward" in extras:
            rng = np.random.default_rng([inp_seed(args.workload), 99])
            g32 = rng.normal(size=(T, d)).astype(np.float32)
            dout = to_device(g32 if inp.dtype == "f32" else workloads.bf16_bits(g32), torch)
            gdx = torch.empty((T, d), dtype=dev_dtype, device="cuda")
            gwgu = torch.empty((E, d, 2 * I), dtype=dev_dtype, device="cuda")
            gwd = torch.empty((E, I, d), dtype=dev_dtype, device="cuda")
            gtw = torch.empty((T, k), dtype=torch.float32, device="cuda")
            glg = torch.empty((T, E), dtype=torch.float32, device="cuda") if logits is not None else None
            b_idx = torch.empty((T, k), dtype=torch.int32, device="cuda") if logits is not None else topk_idx
            b_w = torch.empty((T, k), dtype=torch.float32, device="cuda") if logits is not None else topk_w
            bws_bytes = lib.moe_backward_workspace_size(T, d, E, k, I, dt)
            bws = torch.empty(max(bws_bytes, 1), dtype=torch.uint8, device="cuda")
            gout = torch.empty((T, d), dtype=dev_dtype, device="cuda")

            def run_backward(recompute=1):
                st = lib.moe_backward(ptr(x), ptr(logits), T, d, E, k, I, ptr(wgu), ptr(wd), dt, ptr(b_idx),
                                      ptr(b_w), ptr(dout), ptr(gdx), ptr(gwgu), ptr(gwd), ptr(gtw), ptr(glg),
                                      recompute, ptr(bws), bws_bytes, sp)
                if st != 0:
                    raise RuntimeError(f"moe_backward failed with status {st}")

            def run_forward_train():
                st = lib.moe_forward_train(ptr(x), ptr(logits), T, d, E, k, I, ptr(wgu), ptr(wd), dt, ptr(b_idx),
                                           ptr(b_w), ptr(gout), ptr(bws), bws_bytes, sp)
                if st != 0:
                    raise RuntimeError(f"moe_forward_train failed with status {st}")

            for _ in range(args.warmup):
                run_backward()
            b_ms = timed_cold(run_backward, args.steps)
            for _ in range(args.warmup):
                run_forward_train()
                run_backward(0)
            step_ms = timed_cold(lambda: (run_forward_train(), run_backward(0)), args.steps)
            ft_ms = timed_cold(run_forward_train, args.steps)
            bs_ms = timed_cold(lambda: run_backward(0), args.steps)
            # matrix products per call: the recomputed forward (6 n d I) and
            # the gradients (dh 2, dW_down 2, dx 4, dW_gate_up 4: 12 n d I)
            b_flops = 18 * n_rows * d * I
            backward = {"ms": round(b_ms, 5), "flops_per_call": b_flops,
                        "tflops": round(b_flops / (b_ms * 1e-3) / 1e12, 1),
                        "mfma_frac": round(b_flops / (b_ms * 1e-3) / 1e12 /
                                           (PEAK_F32_TFLOPS if inp.dtype == "f32" else PEAK_BF16_TFLOPS), 4),
                        "pairs_per_s": P / (b_ms * 1e-3),
                        # training step: 6 n d I (forward) + 12 n d I (gradients), no recompute
                        "training_step": {"ms": round(step_ms, 5), "forward_train_ms": round(ft_ms, 5),
                                          "backward_saved_ms": round(bs_ms, 5),
                                          "tflops": round(18 * n_rows * d * I / (step_ms * 1e-3) / 1e12, 1),
                                          "pairs_per_s": P / (step_ms * 1e-3)}}
            del gdx, gwgu, gwd, bws, gout

        # ---- timed region 7 (beside the layer): the same layer on the expert
        # weights in the column-tiled layout (moe_tile_weights, done once, then
        # moe_forward_tiled; bit-identical output) ----
        if "tiled" in extras and inp.dtype == "bf16":
            wgu_t, wd_t = torch.empty_like(wgu), torch.empty_like(wd)
            t_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            torch.cuda.synchronize()
            t_ev[0].record(stream)
            if lib.moe_tile_weights(ptr(wgu), ptr(wd), E, d, I, dt, ptr(wgu_t), ptr(wd_t), sp) != 0:
                raise RuntimeError("moe_tile_weights failed")
            t_ev[1].record(stream)
            torch.cuda.synchronize()
            tile_ms = t_ev[0].elapsed_time(t_ev[1])

            def run_tiled():
                st = lib.moe_forward_tiled(ptr(x), ptr(logits), T, d, E, k, I, ptr(wgu_t), ptr(wd_t), dt,
                                           ptr(layer.topk_idx), ptr(layer.topk_w), None, None, None, ptr(layer.out),
                                           ptr(layer.fws), layer.fws_bytes, sp)
                if st != 0:
                    raise RuntimeError(f"moe_forward_tiled failed with status {st}")
            for _ in range(args.warmup):
                run_tiled()
            tl_ms = timed_cold(run_tiled, args.steps)
            tiled = {"ms_per_step": round(tl_ms, 5), "pairs_per_s": P / (tl_ms * 1e-3),
                     "tile_weights_ms": round(tile_ms, 4),
                     "note": "moe_forward_tiled on weights laid out once by moe_tile_weights (a read and a write "
                             "of every weight, outside the steps); output bit-identical to moe_forward"}
            del wgu_t, wd_t

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
        "timing": {"headline": f"cold: {args.flush_mb} MiB scratch read before each step, HIP events around "
                               "moe_forward on its stream (the flush outside the events)",
                   "cold_min_ms": round(t["cold_min_ms"], 5), "cold_median_ms": round(t["cold_median_ms"], 5),
                   "wall_ms_per_step_with_flush": round(t["wall_ms_with_flush"], 5),
                   "warm_ms_per_step": round(t["warm_ms"], 5),
                   "warm_pairs_per_s": P / (t["warm_ms"] * 1e-3)},
        "roofline": roofline,
        "kernels": kernels,
        "hbm_targets": {"permute_rows_frac": permute_rows["hbm_frac"] if permute_rows else None,
                        "combine_frac": kernels["combine"].get("hbm_frac"), "target": 0.70},
        "staged_gpu_ms_per_step": t["staged_ms"],
        "graph_ms_per_step": graph_ms,
        "permute_gbs": permute_rows["gbs"] if permute_rows else None,
        "permute_rows": permute_rows,
        "router_projection": router,
        "backward": backward,
        "tiled_weights": tiled,
    }
    extras = [] if args.extra in ("", "none") else [w for w in args.extra.split(",") if w != args.workload]
    if extras:
        result["other_workloads"] = {w: measure_extra(lib, tre, torch, w, flush, args.steps, args.warmup)
                                     for w in extras}
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
