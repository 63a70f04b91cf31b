"""Helpers for the GPU parity tests: run the HIP path through the C ABI on a
workload and compare it with the oracle.  Imported by tests only."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import segmented_rank_gemm_segment_amd as srg
import workloads as wl

DEV = "cuda:0"
TOL = {"bf16": 1e-2, "f32": 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def normwise(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (0 when both are all zero)."""
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Run:
    """All outputs of the HIP path for one workload."""


def run_hip(w: wl.Workload, policy: str = "exact", d=None, separate: bool = True,
            fused: bool = True, natural_b: bool = True) -> Run:
    d = d or wl.device_tensors(w, DEV)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, policy, natural_b=natural_b)
    seg = srg.Segments(w.n, w.n_slots, DEV)
    out = Run()
    out.pool, out.seg, out.d = pool, seg, d
    srg.lora_build_segments(d["row_slot"], pool, seg)
    H = torch.full((w.n, w.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_shrink(d["X"], seg, pool, H)
    out.H = H
    if fused:
        Yf = torch.empty((w.n, w.d_out), dtype=dt, device=DEV)
        srg.lora_linear_fused(d["X"], d["W"], H, seg, pool, Yf)
        out.Yf = Yf
    if separate:
        Yb = torch.empty((w.n, w.d_out), dtype=dt, device=DEV)
        srg.lora_base_gemm(d["X"], d["W"], Yb)
        Ys = Yb.clone()
        srg.lora_expand(H, seg, pool, Ys)
        dY = torch.zeros((w.n, w.d_out), dtype=dt, device=DEV)
        srg.lora_expand(H, seg, pool, dY)
        out.Yb, out.Ys, out.dY = Yb, Ys, dY
    torch.cuda.synchronize()
    out.meta = seg.to_host()
    return out


def check_metadata(w: wl.Workload, run: Run) -> dict:
    ref = oracle.segment_metadata(w.row_slot, w.slot_rank, w.slot_alpha, w.r_max)
    m = run.meta
    assert m["num_segments"] == int(ref["num_segments"])
    for k in ("segment_offsets", "segment_slots", "segment_ranks", "token_indices", "row_segment"):
        assert np.array_equal(m[k], ref[k]), k
    assert np.array_equal(m["segment_scales"].view(np.uint32),
                          ref["segment_scales"].astype(np.float32).view(np.uint32))
    assert m["status"] == int(ref["status"])
    return ref


def check_values(w: wl.Workload, run: Run, rows=None, tol=None):
    """Compare H, Y (fused and separate) and dY with the oracle on `rows`
    (all rows by default).  Returns the error figures."""
    tol = TOL[w.dtype] if tol is None else tol
    Yr, dYr, Hr = oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                      w.r_max, w.dtype, rows=rows)
    idx = np.arange(w.n) if rows is None else np.asarray(rows)
    ti = torch.as_tensor(idx, device=DEV, dtype=torch.long)
    errs = {}
    # H: written entries are k < rank of the row's slot; everything else untouched (NaN)
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    Hg = to_f64(run.H[ti])
    mask = np.zeros_like(Hg, dtype=bool)
    for t, i in enumerate(idx):
        a = keys[i]
        if a >= 0:
            mask[t, :int(w.slot_rank[a])] = True
    assert np.all(np.isnan(Hg[~mask])), "shrink wrote outside [0, rank)"
    assert np.all(np.isfinite(Hg[mask]))
    errs["H"] = normwise(np.where(mask, Hg, 0.0), Hr)
    if hasattr(run, "Yf"):
        errs["Y_fused"] = normwise(to_f64(run.Yf[ti]), Yr)
    if hasattr(run, "Ys"):
        errs["Y_separate"] = normwise(to_f64(run.Ys[ti]), Yr)
        errs["dY"] = normwise(to_f64(run.dY[ti]), dYr)
        errs["Y_base"] = normwise(to_f64(run.Yb[ti]), Yr - dYr)
    for k, v in errs.items():
        assert v <= tol, (k, v, tol)
    return errs


def base_rows_bitwise(w: wl.Workload, run: Run):
    """Rows of base-only / rank-0 segments: fused output == base GEMM output
    bit for bit, and expand leaves them untouched."""
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    base = np.array([k < 0 or int(w.slot_rank[k]) == 0 for k in keys], dtype=bool)
    if not base.any():
        return 0
    ti = torch.as_tensor(np.nonzero(base)[0], device=DEV)
    if hasattr(run, "Yf") and hasattr(run, "Yb"):
        assert torch.equal(run.Yf[ti], run.Yb[ti])
    if hasattr(run, "Ys"):
        assert torch.equal(run.Ys[ti], run.Yb[ti])
        assert torch.count_nonzero(run.dY[ti].float()) == 0
    return int(base.sum())


def sample_rows(w: wl.Workload, meta_ref: dict, k: int = 512, seed: int = 0, extra=None):
    """>= k rows: first and last row of every segment, `extra`, then random."""
    ti = meta_ref["token_indices"]
    off = meta_ref["segment_offsets"]
    rows = set()
    for s in range(int(meta_ref["num_segments"])):
        rows.add(int(ti[off[s]]))
        rows.add(int(ti[off[s + 1] - 1]))
    if extra is not None:
        rows.update(int(x) for x in extra)
    rng = np.random.default_rng(seed)
    while len(rows) < min(k, w.n):
        rows.add(int(rng.integers(0, w.n)))
    return sorted(rows)
