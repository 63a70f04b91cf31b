#!/usr/bin/env python3
"""Benchmark of the segmented multi-LoRA linear layer on one MI355X.

One step = one pass of the whole hot path over one batch: segment-metadata
build and shrink (H = X_a A_a^T; one launch for decode-sized batches,
lora_build_shrink), and the base GEMM with the LoRA expand fused into its
epilogue (``--path separate``: base GEMM, then expand + scatter-add;
``--path layer``: all of it in one call, lora_layer_fused, which is one
launch for batches of up to 512 rows).  By default every path is timed and
the fastest is the headline.  Inputs are resident in HBM before timing
starts.  Each step
uses the next of several copies of the layer's tensors (like consecutive
layers of a model), so that the 256 MB last-level cache cannot serve weights
read in the previous step.

Prints one JSON line (rank 0; one GPU):
  value      = token rows per second of the whole step (headline workload)
  roofline   = dominant kernel: algorithmic bytes (or flops) per launch over
               its mean HIP-event duration, against the MI355X peak
  kernels    = the same figures for every kernel of the step
  prefill    = the prefill workload's step (tokens/s, TFLOP/s, MFMA fraction)
  dora       = the same step with every slot a DoRA adapter (column factors
               in the epilogue), and the per-adapter factor preparation
  fp8_weight = the same step with the base weight in FP8 E4M3 (per-row scale)
  layer_70b  = the 70B-shaped layer's seven projections per step, one call
               pair each or with q|k|v and gate|up stacked
  cpu_baseline = the float64 CPU oracle on a bounded sample of the headline
               workload, on this host's cores

    python bench.py [--steps K] [--warmup W] [--workload decode] [--path fused]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
F32_TFLOPS = 157.3

WORKLOAD_NAMES = {
    "tiny_f32": "tiny fp32: d_in=d_out=512, 32 rows in 4 segments [0,8,12,28,32] (r 8/base/16/8)",
    "decode": "decode bf16: d_in=d_out=4096, 256 rows (1 token/request), 128 slots r=16, "
              "10% base-only",
    "prefill": "prefill bf16: d_in=4096 -> d_out=14336, 8 requests 512..4096 tokens, ranks 8..64, "
               "1 base-only",
    "skewed_decode": "skewed decode bf16: d=4096, 1024 rows, 1000 slots r in {8,16,32,64}, "
                     "Zipf(1.0) ids",
    "layer70b": "70B-shaped layer bf16: q/k/v/o/gate/up/down, 2304 rows (2048 prefill + 256 "
                "decode), 64 slots r in {16, 64}",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode",
                   choices=["tiny_f32", "decode", "prefill", "skewed_decode"])
    p.add_argument("--path", choices=["auto", "fused", "separate", "overlap", "layer"],
                   default="auto",
                   help="auto: time every step variant and report the fastest; overlap = "
                        "separate with the base GEMM on a second stream beside build+shrink; "
                        "layer = the whole layer in one call (one launch up to 512 rows)")
    p.add_argument("--policy", choices=["exact", "two_buckets", "padded"], default="exact")
    p.add_argument("--rotate-mb", type=float, default=600.0,
                   help="total size of the rotated copies of the layer tensors")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dora", action="store_true",
                   help="skip the DoRA variant (column factors in the epilogue)")
    p.add_argument("--no-fp8w", action="store_true",
                   help="skip the FP8-weight variant of the base product")
    p.add_argument("--no-skewed", action="store_true",
                   help="skip the skewed large-pool decode entry (three rank policies)")
    p.add_argument("--no-layer", action="store_true",
                   help="skip the 70B-shaped layer (seven projections, separate vs stacked)")
    p.add_argument("--no-vendor", action="store_true",
                   help="skip timing the base product through torch.matmul for comparison")
    p.add_argument("--eager", action="store_true",
                   help="launch every call from Python instead of replaying a captured HIP graph")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    p.add_argument("--kernel-loops", type=int, default=None,
                   help="launches per kernel in the per-kernel timing (default: steps)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (true ranks; base-only rows carry no LoRA work)
# ---------------------------------------------------------------------------
def work_figures(w):
    e = 2 if w.dtype == "bf16" else 4
    keys = [int(a) for a in w.row_slot]
    lora_rows = [(i, a) for i, a in enumerate(keys)
                 if 0 <= a < w.n_slots and 0 < int(w.slot_rank[a]) <= w.r_max]
    distinct = sorted({a for _, a in lora_rows})
    sum_r_distinct = sum(int(w.slot_rank[a]) for a in distinct)
    sum_r_rows = sum(int(w.slot_rank[a]) for _, a in lora_rows)
    n_lora = len(lora_rows)
    n, di, do = w.n, w.d_in, w.d_out
    f = {
        "n_lora_rows": n_lora,
        "distinct_adapters": len(distinct),
        "bytes": {
            "build": n * 4 + 2 * n * 4 + 2 * w.n_slots * 4,
            "build_shrink": (n * 4 + 2 * n * 4 + 2 * w.n_slots * 4) + sum_r_distinct * di * e
                            + n_lora * di * e + sum_r_rows * 4,
            "shrink": sum_r_distinct * di * e + n_lora * di * e + sum_r_rows * 4,
            "expand": sum_r_distinct * do * e + sum_r_rows * 4 + 2 * n_lora * do * e,
            "base": do * di * e + n * di * e + n * do * e,
            "fused": do * di * e + n * di * e + n * do * e + sum_r_distinct * do * e + sum_r_rows * 4,
            # the whole layer in one launch: the fused product's bytes plus
            # the metadata, the distinct A rows and H written once
            "layer": (n * 4 + 2 * n * 4 + 2 * w.n_slots * 4) + do * di * e + n * di * e
                     + n * do * e + sum_r_distinct * (di + do) * e + 2 * sum_r_rows * 4,
            # FP8 base weight: one byte per weight plus a float32 scale per row
            "base_fp8w": do * di + do * 4 + n * di * e + n * do * e,
            "fused_fp8w": do * di + do * 4 + n * di * e + n * do * e + sum_r_distinct * do * e
                          + sum_r_rows * 4,
            "layer_fp8w": (n * 4 + 2 * n * 4 + 2 * w.n_slots * 4) + do * di + do * 4
                          + n * di * e + n * do * e + sum_r_distinct * (di + do) * e
                          + 2 * sum_r_rows * 4,
        },
        "flops": {
            "shrink": 2 * sum_r_rows * di,
            "build_shrink": 2 * sum_r_rows * di,
            "expand": 2 * sum_r_rows * do,
            "base": 2 * n * di * do,
            "fused": 2 * n * di * do + 2 * sum_r_rows * do,
            "layer": 2 * n * di * do + 2 * sum_r_rows * (di + do),
            "base_fp8w": 2 * n * di * do,
            "fused_fp8w": 2 * n * di * do + 2 * sum_r_rows * do,
            "layer_fp8w": 2 * n * di * do + 2 * sum_r_rows * (di + do),
        },
    }
    return f


def workload_stats(w, seed):
    """The batch's structure as the bench ran it: seed, segments (one per
    distinct slot key, base-only included), their length histogram and the
    ranks of the adapters used (counted on the host from the mapping)."""
    keys, counts = np.unique(np.asarray(w.row_slot), return_counts=True)
    bins = [(1, 1), (2, 3), (4, 7), (8, 15), (16, 63), (64, 255), (256, 1023), (1024, 1 << 30)]
    hist = {(f"{a}" if a == b else (f"{a}-{b}" if b < (1 << 30) else f"{a}+")):
            int(np.sum((counts >= a) & (counts <= b))) for a, b in bins}
    used = [int(k) for k in keys if 0 <= k < w.n_slots]
    ranks = np.asarray([int(w.slot_rank[k]) for k in used], dtype=np.int64)
    return {"seed": f"numpy SeedSequence({seed})", "rows": int(w.n), "segments": int(len(keys)),
            "base_only_rows": int(np.sum(np.asarray(w.row_slot) < 0)),
            "segment_length_hist": {k: v for k, v in hist.items() if v},
            "longest_segment": int(counts.max()) if counts.size else 0,
            "adapter_rank_hist": {str(r): int(np.sum(ranks == r)) for r in sorted(set(ranks.tolist()))}}


# ---------------------------------------------------------------------------
# device state
# ---------------------------------------------------------------------------
DORA_SEED = 9
FP8_SEED = 11


def dora_magnitudes(w, device):
    """Seeded DoRA magnitudes for every slot (float32 [d_out] on device)."""
    import torch
    import workloads as wl
    mag = wl.make_magnitude(DORA_SEED, w.n_slots, w.d_out, 0.02 * np.sqrt(w.d_in), p_plain=0.0)
    return [torch.from_numpy(m).to(device) for m in mag]


class Layer:
    def __init__(self, w, policy, device, dora=False, fp8w=False):
        import torch
        import segmented_rank_gemm_segment_amd as srg
        import workloads as wl
        d = wl.device_tensors(w, device)
        self.X, self.W, self.row_slot = d["X"], d["W"], d["row_slot"]
        self.alpha = w.slot_alpha
        self.pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, policy, dora=dora)
        self.mag = dora_magnitudes(w, device) if dora else None
        if dora:
            for a, m in enumerate(self.mag):
                self.pool.dora_prepare(a, self.W, m)
        self.Wq = self.ws = None
        if fp8w:
            codes, scale = wl.make_fp8_weight(FP8_SEED, w.d_out, w.d_in)
            self.Wq = torch.from_numpy(codes).to(device)
            self.ws = torch.from_numpy(scale).to(device)
        self.seg = srg.Segments(w.n, w.n_slots, device)
        self.sync = srg.layer_sync(device)
        dt = self.X.dtype
        self.H = torch.zeros((w.n, w.r_max), dtype=torch.float32, device=device)
        self.Y = torch.empty((w.n, w.d_out), dtype=dt, device=device)
        self.nbytes = sum(t.numel() * t.element_size()
                          for t in (self.X, self.W, d["A"], d["Bt"], self.Y, self.H))

    def clone(self, device):
        import copy
        import torch
        import segmented_rank_gemm_segment_amd as srg
        c = copy.copy(self)
        c.X, c.W = self.X.clone(), self.W.clone()
        if self.Wq is not None:
            c.Wq, c.ws = self.Wq.clone(), self.ws.clone()
        p = self.pool
        c.row_slot = self.row_slot.clone()
        c.pool = srg.Pool(p.A.clone(), p.Bt.clone(), p.slot_rank.clone(), self.alpha,
                          p.rank_policy, dora=p.dora_scale is not None)
        if p.dora_scale is not None:
            c.pool.dora_scale.copy_(p.dora_scale)
        c.seg = srg.Segments(self.seg.n_rows, p.n_slots, device)
        c.sync = srg.layer_sync(device)
        c.H, c.Y = torch.zeros_like(self.H), torch.empty_like(self.Y)
        return c


def Layer_bytes_estimate(w):
    """Bytes of one copy of a layer's tensors (X, W, A, Bt, Y, H)."""
    e = 2 if w.dtype == "bf16" else 4
    return (w.n * w.d_in + w.d_out * w.d_in + w.n_slots * w.r_max * (w.d_in + w.d_out)
            + w.n * w.d_out) * e + w.n * w.r_max * 4


def k_build(L):
    import segmented_rank_gemm_segment_amd as srg
    srg.lora_build_segments(L.row_slot, L.pool, L.seg)


def k_shrink(L):
    import segmented_rank_gemm_segment_amd as srg
    srg.lora_shrink(L.X, L.seg, L.pool, L.H)


def k_build_shrink(L):
    import segmented_rank_gemm_segment_amd as srg
    srg.lora_build_shrink(L.row_slot, L.X, L.pool, L.seg, L.H)


def k_fused(L):
    import segmented_rank_gemm_segment_amd as srg
    srg.lora_linear_fused(L.X, L.W, L.H, L.seg, L.pool, L.Y)


def k_layer(L):
    import segmented_rank_gemm_segment_amd as srg
    srg.lora_layer_fused(L.row_slot, L.X, L.W, L.pool, L.seg, L.H, L.Y, L.sync)


def k_base(L):
    import segmented_rank_gemm_segment_amd as srg
    srg.lora_base_gemm(L.X, L.W, L.Y)


def k_expand(L):
    import segmented_rank_gemm_segment_amd as srg
    srg.lora_expand(L.H, L.seg, L.pool, L.Y)


def k_fused_fp8w(L):
    import segmented_rank_gemm_segment_amd as srg
    srg.lora_linear_fused_fp8w(L.X, L.Wq, L.ws, L.H, L.seg, L.pool, L.Y)


def k_layer_fp8w(L):
    import segmented_rank_gemm_segment_amd as srg
    srg.lora_layer_fused_fp8w(L.row_slot, L.X, L.Wq, L.ws, L.pool, L.seg, L.H, L.Y, L.sync)


def k_base_fp8w(L):
    import segmented_rank_gemm_segment_amd as srg
    srg.lora_base_gemm_fp8w(L.X, L.Wq, L.ws, L.Y)


def k_vendor_base(L):
    """The same X W^T through torch.matmul (the vendor BLAS): timed for
    comparison only, never part of a step."""
    import torch
    torch.matmul(L.X, L.W.t(), out=L.Y)


class _Overlap:
    """Base GEMM on a second stream, concurrent with build + shrink on the
    launch stream; the expand waits for both (fork/join through events, so
    it is captured into the same HIP graph as two branches)."""

    def __init__(self):
        import torch
        self.side = torch.cuda.Stream()          # default priority
        self.fork = torch.cuda.Event()
        self.join = torch.cuda.Event()

    def __call__(self, L):
        import torch
        main = torch.cuda.current_stream()
        self.fork.record(main)
        self.side.wait_event(self.fork)
        with torch.cuda.stream(self.side):
            k_base(L)
        self.join.record(self.side)
        k_build(L)
        k_shrink(L)
        main.wait_event(self.join)
        k_expand(L)


STEP = {"fused": (k_build_shrink, k_fused), "separate": (k_build_shrink, k_base, k_expand),
        "fused_fp8w": (k_build_shrink, k_fused_fp8w), "layer": (k_layer,),
        "layer_fp8w": (k_layer_fp8w,)}
PATHS = ("fused", "separate", "overlap", "layer")
KNAME = {k_build: "build", k_shrink: "shrink", k_build_shrink: "build_shrink", k_fused: "fused",
         k_base: "base", k_expand: "expand", k_fused_fp8w: "fused_fp8w", k_base_fp8w: "base_fp8w",
         k_layer: "layer", k_layer_fp8w: "layer_fp8w"}


def _graph(fn_seq, layers, count, start=0):
    """Capture `count` calls cycling through `layers` into one HIP graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            for fn in fn_seq:
                fn(layers[(start + i) % len(layers)])
    return g


def time_calls(fn_seq, layers, iters, warmup, use_graph):
    """Mean device time of one pass of fn_seq over `iters` passes cycling
    through `layers`, bracketed by HIP events on the launch stream.  With
    use_graph the passes are captured in one HIP graph (replayed once)."""
    import torch
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if use_graph:
        # one eager pass first, so that nothing a call sets up on first use
        # happens during capture
        for fn in fn_seq:
            fn(layers[0])
        torch.cuda.synchronize()
        gw = _graph(fn_seq, layers, max(1, warmup))
        gt = _graph(fn_seq, layers, iters, start=max(1, warmup))
        gw.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        ev0.record()
        gt.replay()
        ev1.record()
        torch.cuda.synchronize()
    else:
        for i in range(warmup):
            for fn in fn_seq:
                fn(layers[i % len(layers)])
        torch.cuda.synchronize()
        t = time.perf_counter()
        ev0.record()
        for i in range(iters):
            for fn in fn_seq:
                fn(layers[i % len(layers)])
        ev1.record()
        torch.cuda.synchronize()
    wall = time.perf_counter() - t
    return ev0.elapsed_time(ev1) * 1e-3 / iters, wall


def measure(w, paths, policy, steps, warmup, rotate_mb, kernel_loops, use_graph,
            device="cuda:0", vendor=False, dora=False, fp8w=False, kernels=None):
    import torch
    L0 = Layer(w, policy, device, dora=dora, fp8w=fp8w)
    copies = max(1, int(np.ceil(rotate_mb * 1e6 / L0.nbytes)))
    layers = [L0] + [L0.clone(device) for _ in range(copies - 1)]
    for L in layers:                      # metadata/H valid for per-kernel loops
        k_build(L)
        k_shrink(L)
    torch.cuda.synchronize()
    step = {}
    for p in paths:
        seq = (_Overlap(),) if p == "overlap" else STEP[p]
        step[p] = time_calls(seq, layers, steps, warmup, use_graph)
    kl = kernel_loops or steps
    per_kernel = {}
    if kernels is None:
        kernels = STEP["fused"] + STEP["separate"] + (k_build, k_shrink)
        if "layer" in paths:
            kernels += STEP["layer"]
    for fn in sorted(set(kernels), key=lambda f: KNAME[f]):
        per_kernel[KNAME[fn]], _ = time_calls((fn,), layers, kl, max(3, warmup // 4), use_graph)
    res = {"step": step, "per_kernel_s": per_kernel, "copies": copies, "layer_bytes": L0.nbytes}
    if dora:
        # DoRA column factors, one slot per call (a one-off per adapter load)
        turn = [0]

        def k_prepare(L):
            a = turn[0] % w.n_slots
            turn[0] += 1
            L.pool.dora_prepare(a, L.W, L.mag[a])
        res["prepare_s"], _ = time_calls((k_prepare,), layers, kl, max(3, warmup // 4), use_graph)
    if vendor:
        k_vendor_base(layers[0])          # library set-up outside any capture
        torch.cuda.synchronize()
        res["vendor_base_s"], _ = time_calls((k_vendor_base,), layers, kl, max(3, warmup // 4),
                                             use_graph)
    return res


def vendor_entry(fig, m):
    """Context: the base product through the vendor BLAS on the same operands."""
    if "vendor_base_s" not in m:
        return None
    t = m["vendor_base_s"]
    return {"what": "torch.matmul(X, W.t()) (hipBLASLt), same shape, operands and launch mode",
            "us": round(t * 1e6, 3), "TFLOP_s": round(fig["flops"]["base"] / t / 1e12, 2),
            "ours_base_us": round(m["per_kernel_s"]["base"] * 1e6, 3)}


def kernel_table(fig, per_kernel, dtype):
    out = {}
    for k, sec in per_kernel.items():
        b = fig["bytes"].get(k)
        fl = fig["flops"].get(k, 0)
        d = {"us": round(sec * 1e6, 3)}
        if b is not None:
            d["GB_s"] = round(b / sec / 1e9, 1)
            d["hbm_frac"] = round(b / sec / 1e9 / HBM_PEAK_GBS, 4)
            d["alg_bytes"] = int(b)
        if fl:
            d["TFLOP_s"] = round(fl / sec / 1e12, 2)
            peak = MFMA_BF16_TFLOPS if dtype == "bf16" else F32_TFLOPS
            d["mfma_frac"] = round(fl / sec / 1e12 / peak, 4)
        out[k] = d
    return out


def roofline_for(kernel, fig, sec, dtype):
    b = fig["bytes"][kernel]
    fl = fig["flops"].get(kernel, 0)
    peak_f = MFMA_BF16_TFLOPS if dtype == "bf16" else F32_TFLOPS
    ridge = peak_f * 1e12 / (HBM_PEAK_GBS * 1e9)
    if fl and fl / b > ridge:
        a = fl / sec / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": peak_f, "unit": "TFLOP/s",
                "frac": round(a / peak_f, 4), "traffic": None, "kernel": kernel}
    a = b / sec / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kernel}


def log(*a):
    """Progress of the run on stderr (the JSON line alone goes to stdout)."""
    print("[bench]", *a, file=sys.stderr, flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def _code_only(text):
    """C/C++ source without comments and blank space (comment edits do not
    change the kernels the counters were taken on)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_sha():
    """sha256 over the code (comments dropped) of the HIP sources and
    headers the kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "segmented_rank_gemm_segment_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


# The translation unit each timed kernel is compiled in.
KERNEL_UNIT = {"layer": "gemm.hip", "fused": "gemm.hip", "base": "gemm.hip",
               "fused_fp8w": "gemm.hip", "base_fp8w": "gemm.hip", "layer_fp8w": "gemm.hip",
               "shrink": "shrink_expand.hip", "shrink_mfma": "shrink_expand.hip",
               "expand": "shrink_expand.hip", "build": "build_segments.hip",
               "build_shrink": "build_segments.hip"}


def unit_source_sha(unit):
    """sha256 over the code (comments dropped) of one translation unit and
    every local header it includes, directly or not."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "segmented_rank_gemm_segment_amd", "csrc")
    seen, todo = [], [os.path.normpath(os.path.join(csrc, unit))]
    while todo:
        path = todo.pop()
        if path in seen:
            continue
        seen.append(path)
        with open(path, encoding="utf-8") as f:
            text = f.read()
        for inc in re.findall(r'^\s*#include\s+"([^"]+)"', text, flags=re.M):
            todo.append(os.path.normpath(os.path.join(os.path.dirname(path), inc)))
    h = hashlib.sha256()
    for path in sorted(seen):
        with open(path, encoding="utf-8") as f:
            h.update(os.path.relpath(path, ROOT).encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from rocprofv3 FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch, each scaled by the reading of a plain
    copy of known size), or None when no counters were taken for the current
    code of the kernel's translation unit (and the headers it includes)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    unit = KERNEL_UNIT.get(kernel)
    shas = t.get("unit_sha256", {})
    if unit is None or unit not in shas or shas[unit] != unit_source_sha(unit):
        return None
    k = t.get("workloads", {}).get(workload, {}).get(kernel)
    if not k:
        return None
    return int(round((k["fetch_kib"] * t["fetch_scale"] + k["write_kib"] * t["write_scale"]) * 1024))


def _oracle_rate(w, budget_s):
    import oracle
    runs, rows, t0 = 0, 0, time.perf_counter()
    while True:
        oracle.segment_metadata(w.row_slot, w.slot_rank, w.slot_alpha, w.r_max)
        oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha, w.r_max,
                            w.dtype)
        runs += 1
        rows += w.n
        el = time.perf_counter() - t0
        if el >= budget_s:
            return rows / el, runs, el


def cpu_baseline(w, budget_s=12.0, single_core_s=6.0):
    """The oracle as it stands, on the whole headline batch, repeated for
    about `budget_s` seconds of host time on every core the BLAS uses, then
    for about `single_core_s` seconds with one BLAS thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = len(os.sched_getaffinity(0))
    rate, runs, el = _oracle_rate(w, budget_s)
    out = {"value": round(rate, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{runs} full passes of the {w.n}-row batch (metadata + float64 row loop) in {el:.1f} s",
           "host_cpus": len(os.sched_getaffinity(0))}
    if threadpool_limits is not None and single_core_s > 0:
        with threadpool_limits(limits=1):
            r1, runs1, el1 = _oracle_rate(w, single_core_s)
        out["single_core"] = {"value": round(r1, 2), "unit": "tokens/s", "cores": 1,
                              "sample": f"{runs1} full passes in {el1:.1f} s"}
    return out


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def _oracle_layer_time(ws, rows, budget_s, min_runs=1, warmup=True):
    """Seconds per pass of the oracle over `rows` of every projection in ws
    (metadata built once per pass on the whole batch), median of the passes
    run within about budget_s (after one warm-up pass unless warmup=False)."""
    import oracle
    w0 = ws[0]

    def one():
        oracle.segment_metadata(w0.row_slot, w0.slot_rank, w0.slot_alpha, w0.r_max)
        for w in ws:
            oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                w.r_max, w.dtype, rows=rows)
    if warmup:
        one()
    times, t0 = [], time.perf_counter()
    while len(times) < min_runs or (time.perf_counter() - t0 < budget_s and len(times) < 7):
        a = time.perf_counter()
        one()
        times.append(time.perf_counter() - a)
    return float(np.median(times)), len(times)


def cpu_baselines(budget_s=3.0):
    """The float64 oracle on the tiny fp32, skewed-decode, prefill and
    70B-shaped workloads, on all BLAS threads and on one thread, median of
    the passes after a warm-up.  The tiny and skewed workloads run whole; the
    prefill and 70B-shaped ones run a seeded sample of rows and are
    extrapolated linearly to the batch, since rows are independent: 512 rows
    on all threads (the first and last row of every segment and every decode
    row of the 70B-shaped batch included), 128 (prefill) or 32 (70B-shaped)
    random rows on one thread (no warm-up pass: one 70B-shaped pass takes
    seconds).  A pass has a part that does not
    depend on the rows asked for (the metadata of the whole batch, decoding
    the whole X and W), timed by a pass over no rows: the batch time is
    t0 + (t_sample - t0) n / sample."""
    import workloads as wl
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    threads = int(_blas_threads())

    def sample(w, k, extra=(), ends=True):
        rows = set(int(x) for x in extra)
        if ends:
            _, first = np.unique(w.row_slot, return_index=True)
            last = w.n - 1 - np.unique(w.row_slot[::-1], return_index=True)[1]
            rows |= set(first.tolist()) | set(last.tolist())
        rng = np.random.default_rng(0)
        while len(rows) < min(k, w.n):
            rows.add(int(rng.integers(0, w.n)))
        return np.array(sorted(rows)[:max(k, len(rows))])

    out = {}
    for name in ("tiny_f32", "skewed_decode", "prefill", "layer70b"):
        if name == "layer70b":
            ws = [wl.layer70b_projection(p[0]) for p in wl.LAYER70B_PROJECTIONS]
        else:
            ws = [wl.make_workload(name)]
        n = ws[0].n
        entry = {"workload": WORKLOAD_NAMES[name], "seed": f"numpy SeedSequence({wl.SEEDS[name]})",
                 "rows": n}
        sampled = name in ("prefill", "layer70b")
        for label, k, lim in (("all_cores", 512, None),
                              ("single_core", 128 if name == "prefill" else 32, 1)):
            if lim == 1 and threadpool_limits is None:
                continue
            if sampled:
                extra = range(2048, 2304) if (name == "layer70b" and lim is None) else ()
                rows = sample(ws[0], k, extra, ends=lim is None)
            else:
                rows = None
            ctx = threadpool_limits(limits=lim) if lim else None
            if ctx:
                ctx.__enter__()
            try:
                warm = not (lim == 1 and rows is not None)
                t, runs = _oracle_layer_time(ws, rows, budget_s, warmup=warm)
                t0 = (_oracle_layer_time(ws, np.zeros(0, dtype=np.int64), 0.0, warmup=False)[0]
                      if rows is not None else 0.0)
            finally:
                if ctx:
                    ctx.__exit__(None, None, None)
            done = n if rows is None else len(rows)
            per_batch = t0 + max(t - t0, 0.0) * (n / done) if rows is not None else t
            entry[label] = {"value": round(n / per_batch, 2), "unit": "tokens/s",
                            "cores": threads if lim is None else 1, "kind": "oracle",
                            "extrapolated": rows is not None,
                            "sample": (f"median of {runs} passes over all {n} rows" if rows is None
                                       else f"median of {runs} passes over {done} seeded rows of "
                                            f"{n} ({t:.2f} s; {t0:.2f} s of it independent of "
                                            f"the rows), extrapolated linearly")}
        out[name] = entry
        del ws
    return out


def dora_entry(w, fig, m, paths, args):
    """The headline workload with every slot a DoRA adapter: step and kernel
    times against the plain pool's, and the column-factor preparation."""
    md = measure(w, paths, args.policy, args.steps, args.warmup, args.rotate_mb,
                 args.kernel_loops, not args.eager, dora=True)
    e = 2 if w.dtype == "bf16" else 4
    r_mean = float(np.mean(w.slot_rank))
    prep_bytes = (w.d_out * w.d_in * e + r_mean * (w.d_in + w.d_out) * e + 2 * w.d_out * 4)
    t = md["prepare_s"]
    return {
        "what": "same workload, every slot with DoRA column factors g = m / ||W0 + sBA||_c "
                "applied before the rounding",
        "step_us_by_path": {p: round(md["step"][p][0] * 1e6, 3) for p in paths},
        "step_vs_plain": {p: round(md["step"][p][0] / m["step"][p][0], 4) for p in paths},
        "kernels_us": {k: round(md["per_kernel_s"][k] * 1e6, 3) for k in ("fused", "expand")},
        "kernels_vs_plain": {k: round(md["per_kernel_s"][k] / m["per_kernel_s"][k], 4)
                             for k in ("fused", "expand")},
        "prepare": {"us_per_adapter": round(t * 1e6, 3), "alg_bytes": int(prep_bytes),
                    "GB_s": round(prep_bytes / t / 1e9, 1),
                    "hbm_frac": round(prep_bytes / t / 1e9 / HBM_PEAK_GBS, 4)},
    }


def fp8w_entry(w, fig, m, args):
    """The headline workload with the base weight in FP8 E4M3 (one float32
    scale per output row): the step on both paths (the one-call layer; build
    + shrink, then the fused GEMM) and the GEMM kernels, against the bf16
    weight's fastest step."""
    paths = ["layer_fp8w", "fused_fp8w"]
    mq = measure(w, paths, args.policy, args.steps, args.warmup, args.rotate_mb,
                 args.kernel_loops, not args.eager, fp8w=True,
                 kernels=(k_fused_fp8w, k_base_fp8w, k_layer_fp8w))
    kt = kernel_table(fig, mq["per_kernel_s"], w.dtype)
    best = min(paths, key=lambda p: mq["step"][p][0])
    st = mq["step"][best][0]
    bf16 = min(v[0] for v in m["step"].values()) if m["step"] else None
    main_k = "layer_fp8w" if best == "layer_fp8w" else "fused_fp8w"
    return {
        "what": "same workload, base weight as E4M3 codes with a float32 scale per output row "
                "(LoRA bf16 on the unquantized activations; paths add in fp32 before one rounding)",
        "path": best, "value": round(w.n / st, 1), "unit": "tokens/s",
        "step_us": round(st * 1e6, 3),
        "step_us_by_path": {p: round(v[0] * 1e6, 3) for p, v in mq["step"].items()},
        "step_vs_bf16": round(st / bf16, 4) if bf16 else None,
        "kernels": kt,
        "roofline": dict(roofline_for(main_k, fig, mq["per_kernel_s"][main_k], w.dtype),
                         traffic=measured_traffic(args.workload, main_k)),
    }


def layer_entry(args, device="cuda:0"):
    """The 70B-shaped layer (q, k, v, o, gate, up, down; 2304 rows: a 2048-row
    prefill chunk and 256 decode rows; 64 slots of rank 16 or 64).  q, k, v
    share one input, gate and up another.  One step computes all seven
    projections with one metadata build: either seven shrink + fused GEMM
    pairs, or four with q|k|v and gate|up stacked (one shrink and one GEMM
    over the concatenated weight each)."""
    import torch
    import segmented_rank_gemm_segment_amd as srg
    import workloads as wl
    names = [p[0] for p in wl.LAYER70B_PROJECTIONS]
    ws = {nm: wl.layer70b_projection(nm) for nm in names}
    for a, b in (("k_proj", "q_proj"), ("v_proj", "q_proj"), ("up_proj", "gate_proj")):
        ws[a].X = ws[b].X
    w0 = ws["q_proj"]
    n = w0.n
    row_slot = torch.from_numpy(np.ascontiguousarray(w0.row_slot, dtype=np.int32)).to(device)
    dev = {}
    for nm, w in ws.items():
        d = wl.device_tensors(w, device)
        dev[nm] = {"X": d["X"], "W": d["W"],
                   "pool": srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha)}
    seg = srg.Segments(n, w0.n_slots, device)

    def unit(X, W, pool):
        H = torch.empty((n, pool.r_max), dtype=torch.float32, device=device)
        Y = torch.empty((n, pool.d_out), dtype=torch.bfloat16, device=device)
        return {"X": X, "W": W, "pool": pool, "H": H, "Y": Y}

    sep = [unit(dev[nm]["X"], dev[nm]["W"], dev[nm]["pool"]) for nm in names]
    groups = (("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",))
    stk = []
    for g in groups:
        if len(g) == 1:
            stk.append(sep[names.index(g[0])])
        else:
            W = torch.cat([dev[nm]["W"] for nm in g], dim=0).contiguous()
            stk.append(unit(dev[g[0]]["X"], W, srg.Pool.stacked([dev[nm]["pool"] for nm in g])))

    def step(units):
        def fn(_):
            srg.lora_build_segments(row_slot, units[0]["pool"], seg)
            for u in units:
                srg.lora_shrink(u["X"], seg, u["pool"], u["H"])
                srg.lora_linear_fused(u["X"], u["W"], u["H"], seg, u["pool"], u["Y"])
        return fn

    st = max(3, args.steps // 20)
    t_sep, _ = time_calls((step(sep),), [None], st, 2, not args.eager)
    t_stk, _ = time_calls((step(stk),), [None], st, 2, not args.eager)
    flops = sum(2 * n * w.d_in * w.d_out for w in ws.values())
    out = {"workload": "70B-shaped layer: q/k/v/o/gate/up/down, 2304 rows (2048 prefill + 256 "
                       "decode), 64 slots r in {16, 64}",
           "batch": workload_stats(w0, 5),
           "separate": {"tokens_s": round(n / t_sep, 1), "ms": round(t_sep * 1e3, 4),
                        "TFLOP_s": round(flops / t_sep / 1e12, 1), "calls": 1 + 2 * len(sep),
                        "mfma_frac": round(flops / t_sep / 1e12 / MFMA_BF16_TFLOPS, 4)},
           "stacked": {"tokens_s": round(n / t_stk, 1), "ms": round(t_stk * 1e3, 4),
                       "TFLOP_s": round(flops / t_stk / 1e12, 1), "calls": 1 + 2 * len(stk),
                       "mfma_frac": round(flops / t_stk / 1e12 / MFMA_BF16_TFLOPS, 4)},
           "stacked_speedup": round(t_sep / t_stk, 4)}
    del dev, sep, stk
    torch.cuda.empty_cache()
    return out


def skewed_entry(args):
    """The skewed decode workload (1024 decode rows, 1000 resident slots of
    mixed rank, Zipf adapter ids) under each rank policy: per-rank buckets (exact), the
    two buckets {8,16} / {32,64}, and every slot padded to rank 64.  Step on
    each path (the fastest one named) and the shrink / fused GEMM per policy."""
    import workloads as wl
    w4 = wl.make_workload("skewed_decode")
    f4 = work_figures(w4)
    st = max(10, args.steps // 4)
    out = {"workload": WORKLOAD_NAMES["skewed_decode"], "rows": w4.n,
           "distinct_adapters": f4["distinct_adapters"],
           "batch": workload_stats(w4, wl.SEEDS["skewed_decode"]),
           "alg_bytes": {"shrink": int(f4["bytes"]["shrink"]), "expand": int(f4["bytes"]["expand"]),
                         "fused": int(f4["bytes"]["fused"])},
           "policies": {}}
    for pol in ("exact", "two_buckets", "padded"):
        m4 = measure(w4, ["fused", "separate"], pol, st, max(3, args.warmup // 4), args.rotate_mb,
                     st, not args.eager, kernels=(k_build_shrink, k_shrink, k_fused, k_expand))
        best = min(m4["step"], key=lambda p: m4["step"][p][0])
        pk = m4["per_kernel_s"]
        se = f4["bytes"]["shrink"] + f4["bytes"]["expand"]
        out["policies"][pol] = {
            "path": best, "tokens_s": round(w4.n / m4["step"][best][0], 1),
            "step_us_by_path": {p: round(v[0] * 1e6, 3) for p, v in m4["step"].items()},
            "us": {k: round(v * 1e6, 3) for k, v in pk.items()},
            # counters were taken with the exact policy
            "fused_gemm": dict(roofline_for("fused", f4, pk["fused"], "bf16"),
                               traffic=(measured_traffic("skewed_decode", "fused")
                                        if pol == "exact" else None)),
            "shrink_expand": {"GB_s": round(se / (pk["shrink"] + pk["expand"]) / 1e9, 1),
                              "hbm_frac": round(se / (pk["shrink"] + pk["expand"]) / 1e9 /
                                                HBM_PEAK_GBS, 4)}}
    ex, pad = out["policies"]["exact"], out["policies"]["padded"]
    out["padded_over_exact_step"] = round(ex["tokens_s"] / pad["tokens_s"], 4)
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this layer's kernels run on a single MI355X; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    import segmented_rank_gemm_segment_amd as srg
    import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        # reference for hardware byte counters: each copy reads and writes
        # exactly MIB MiB
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return
    srg.lib()

    w = wl.make_workload(args.workload)
    fig = work_figures(w)
    paths = list(PATHS) if args.path == "auto" else [args.path]
    log(f"{args.workload}: steps and kernels")
    m = measure(w, paths, args.policy, args.steps, args.warmup, args.rotate_mb,
                args.kernel_loops, not args.eager, vendor=not args.no_vendor and w.dtype == "bf16")
    path = min(paths, key=lambda p: m["step"][p][0])
    step_s, wall = m["step"][path]
    kt = kernel_table(fig, m["per_kernel_s"], w.dtype)
    cand = {"fused": ("build_shrink", "fused"), "layer": ("layer",)}.get(
        path, ("build_shrink", "base", "expand"))
    # (overlap: same kernels as separate, base GEMM concurrent with build + shrink)
    main_k = max(cand, key=lambda k: m["per_kernel_s"][k])
    roof = roofline_for(main_k, fig, m["per_kernel_s"][main_k], w.dtype)
    roof["traffic"] = measured_traffic(args.workload, main_k)
    sh, ex = m["per_kernel_s"]["shrink"], m["per_kernel_s"]["expand"]
    se_bytes = fig["bytes"]["shrink"] + fig["bytes"]["expand"]
    out = {
        "metric": "multi-LoRA layer tokens/s; shrink+expand HBM GB/s & % roofline (decode, prefill)",
        "value": round(w.n / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded normals; mapping per the workload recipe)",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "path": path,
                   "rank_policy": args.policy, "rows": w.n, "lora_rows": fig["n_lora_rows"],
                   "distinct_adapters": fig["distinct_adapters"],
                   "rotated_copies": m["copies"], "launch": "eager" if args.eager else "hip_graph",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "batch": workload_stats(w, wl.SEEDS[args.workload]),
        "shrink_expand": {"GB_s": round(se_bytes / (sh + ex) / 1e9, 1),
                          "hbm_frac": round(se_bytes / (sh + ex) / 1e9 / HBM_PEAK_GBS, 4),
                          "us": round((sh + ex) * 1e6, 3)},
        "kernels": kt,
        "step_us_by_path": {p: round(m["step"][p][0] * 1e6, 3) for p in paths},
        "host_wall_s": round(wall, 4),
    }
    if vendor_entry(fig, m):
        out["vendor_base_gemm"] = vendor_entry(fig, m)
    if not args.no_prefill and args.workload != "prefill":
        log("prefill")
        w3 = wl.make_workload("prefill")
        f3 = work_figures(w3)
        st3 = max(5, args.steps // 10)
        # two rotated copies (each ~0.75 GB): no call reads what the previous
        # one left in the 256 MB last-level cache
        rot3 = 2.0 * Layer_bytes_estimate(w3) / 1e6
        m3 = measure(w3, ["fused"], args.policy, st3, max(2, args.warmup // 4), rot3, st3,
                     not args.eager, vendor=not args.no_vendor)
        k3 = kernel_table(f3, m3["per_kernel_s"], "bf16")
        out["prefill"] = {
            "workload": WORKLOAD_NAMES["prefill"], "rows": w3.n, "rotated_copies": m3["copies"],
            "batch": workload_stats(w3, wl.SEEDS["prefill"]),
            "tokens_s": round(w3.n / m3["step"]["fused"][0], 1),
            "ms_per_step": round(m3["step"]["fused"][0] * 1e3, 4), "path": "fused",
            "fused_gemm": dict(roofline_for("fused", f3, m3["per_kernel_s"]["fused"], "bf16"),
                               traffic=measured_traffic("prefill", "fused")),
            "shrink_expand": {
                "GB_s": round((f3["bytes"]["shrink"] + f3["bytes"]["expand"]) /
                              (m3["per_kernel_s"]["shrink"] + m3["per_kernel_s"]["expand"]) / 1e9, 1),
                "hbm_frac": round((f3["bytes"]["shrink"] + f3["bytes"]["expand"]) /
                                  (m3["per_kernel_s"]["shrink"] + m3["per_kernel_s"]["expand"]) /
                                  1e9 / HBM_PEAK_GBS, 4),
                "us": round((m3["per_kernel_s"]["shrink"] + m3["per_kernel_s"]["expand"]) * 1e6, 3)},
            "kernels": k3,
        }
        if vendor_entry(f3, m3):
            out["prefill"]["vendor_base_gemm"] = vendor_entry(f3, m3)
        del w3
    if not args.no_dora:
        log("DoRA variant")
        out["dora"] = dora_entry(w, fig, m, paths, args)
        if "prefill" in out:
            w3 = wl.make_workload("prefill")
            st3 = max(5, args.steps // 10)
            md3 = measure(w3, ["fused"], args.policy, st3, max(2, args.warmup // 4), 0.0, st3,
                          not args.eager, dora=True)
            plain = out["prefill"]["kernels"]["fused"]["us"] * 1e-6
            out["prefill"]["dora"] = {
                "fused_us": round(md3["per_kernel_s"]["fused"] * 1e6, 3),
                "fused_vs_plain": round(md3["per_kernel_s"]["fused"] / plain, 4),
                "step_us": round(md3["step"]["fused"][0] * 1e6, 3)}
            del w3
    if not args.no_fp8w and w.dtype == "bf16":
        log("FP8-weight variant")
        out["fp8_weight"] = fp8w_entry(w, fig, m, args)
        if "prefill" in out:
            w3 = wl.make_workload("prefill")
            f3 = work_figures(w3)
            st3 = max(5, args.steps // 10)
            mq3 = measure(w3, ["fused_fp8w"], args.policy, st3, max(2, args.warmup // 4), 0.0, st3,
                          not args.eager, fp8w=True, kernels=(k_fused_fp8w,))
            out["prefill"]["fp8_weight"] = {
                "tokens_s": round(w3.n / mq3["step"]["fused_fp8w"][0], 1),
                "fused_gemm": roofline_for("fused_fp8w", f3, mq3["per_kernel_s"]["fused_fp8w"], "bf16"),
                "fused_us": round(mq3["per_kernel_s"]["fused_fp8w"] * 1e6, 3)}
            del w3
    if not args.no_skewed and args.workload == "decode":
        log("skewed decode, three rank policies")
        out["skewed_decode"] = skewed_entry(args)
    if not args.no_layer and args.workload == "decode":
        log("70B-shaped layer")
        out["layer_70b"] = layer_entry(args)
    if not args.no_cpu_baseline:
        log("CPU oracle baseline, headline workload")
        out["cpu_baseline"] = cpu_baseline(w)
        log("CPU oracle baselines: tiny fp32, skewed decode, prefill, 70B-shaped layer")
        out["cpu_baselines"] = cpu_baselines()
        if "prefill" in out:
            out["prefill"]["cpu_baseline"] = out["cpu_baselines"]["prefill"]["all_cores"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
