"""GPU parity of stacked projections (adapter-batching page, "Adapter 不是一块
连续 Weight": fused QKV / stacked gate-up, each target with its own A and B):
one stacked pool and one concatenated weight give, for every projection,
the oracle's result for that projection alone (oracle.stacked_forward), on
both tile configurations (tiles straddling projection boundaries), the
long-segment MFMA shrink, fp32, both rank policies and both B layouts, with
DoRA factors and with an FP8 weight.  Tolerances as the plain layer."""
import math

import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_segment_amd as srg
import workloads as wl
from gpu_harness import DEV, TOL, normwise, sample_rows, say, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    srg.lib()
    yield
    torch.cuda.synchronize()


def _projections(seed, n, d_in, outs, n_slots, r_max, dtype="bf16", p_base=0.15, runs=True):
    base = wl.make_random(seed, n, d_in, outs[0], n_slots, r_max, p_base=p_base, dtype=dtype,
                          runs=runs)
    ws = [base]
    for p, d_out in enumerate(outs[1:], 1):
        w = wl.make_random(seed * 10 + p, n, d_in, d_out, n_slots, r_max, dtype=dtype,
                           ranks=list(base.slot_rank))
        w.X, w.row_slot = base.X, base.row_slot
        ws.append(w)
    return ws


def _stacked_pool(ws, policy="exact", natural_b=True, dora=False):
    pools = []
    for w in ws:
        d = wl.device_tensors(w, DEV)
        pools.append(srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, policy,
                              natural_b=False))
    return srg.Pool.stacked(pools, policy, natural_b=natural_b, dora=dora)


def _run(ws, pool, W=None, fp8=None, separate=True):
    b = ws[0]
    dt = torch.bfloat16 if b.dtype == "bf16" else torch.float32
    X = wl.to_torch(b.X, b.dtype, DEV)
    rs = torch.from_numpy(np.ascontiguousarray(b.row_slot, dtype=np.int32)).to(DEV)
    if W is None:
        W = torch.cat([wl.to_torch(w.W, w.dtype, DEV) for w in ws], dim=0).contiguous()
    seg = srg.Segments(b.n, b.n_slots, DEV)
    H = torch.full((b.n, pool.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_build_shrink(rs, X, pool, seg, H)
    out = {"H": H}
    Yf = torch.empty((b.n, pool.d_out), dtype=dt, device=DEV)
    if fp8 is None:
        srg.lora_linear_fused(X, W, H, seg, pool, Yf)
    else:
        srg.lora_linear_fused_fp8w(X, fp8[0], fp8[1], H, seg, pool, Yf)
    out["fused"] = Yf
    if separate:
        Ys = torch.empty_like(Yf)
        srg.lora_base_gemm(X, W, Ys)
        out["base"] = Ys.clone()
        srg.lora_expand(H, seg, pool, Ys)
        out["separate"] = Ys
    torch.cuda.synchronize()
    return out


def _check(ws, out, rows=None, ref=None):
    b = ws[0]
    if ref is None:
        ref = oracle.stacked_forward(b.X, [w.W for w in ws], [w.A for w in ws],
                                     [w.B for w in ws], b.row_slot, b.slot_rank, b.slot_alpha,
                                     b.r_max, b.dtype, rows=rows)
    Y, dY, Hr = ref
    idx = np.arange(b.n) if rows is None else np.asarray(rows)
    ti = torch.as_tensor(idx, device=DEV, dtype=torch.long)
    errs = {}
    for k in ("fused", "separate"):
        if k in out:
            errs[k] = normwise(to_f64(out[k][ti]), Y)
            assert errs[k] <= TOL[b.dtype], (k, errs[k])
    if "base" in out:
        errs["base"] = normwise(to_f64(out["base"][ti]), Y - dY)
        assert errs["base"] <= TOL[b.dtype]
    # H: projection q's ranks at [q rs, q rs + r); everything else untouched
    keys, _ = oracle.validate_rows(b.row_slot, b.slot_rank, b.r_max)
    Hg = to_f64(out["H"][ti])
    rs = b.r_max
    mask = np.zeros_like(Hg, dtype=bool)
    for t, i in enumerate(idx):
        a = keys[i]
        if a >= 0:
            for q in range(len(ws)):
                mask[t, q * rs:q * rs + int(b.slot_rank[a])] = True
    assert np.all(np.isnan(Hg[~mask])), "shrink wrote outside the projections' ranks"
    errs["H"] = normwise(np.where(mask, Hg, 0.0), Hr)
    assert errs["H"] <= TOL[b.dtype]
    return errs


CASES = [
    # seed, n, d_in, outs, n_slots, r_max, dtype
    (601, 96, 256, (64, 32, 32), 6, 16, "bf16"),       # small tiles, QKV-like
    (602, 300, 136, (136, 72, 200), 9, 32, "bf16"),    # small tiles, ragged projections
    (603, 700, 208, (136, 72, 200), 7, 16, "bf16"),    # large tiles straddling projections
    (604, 1100, 256, (512, 256, 256), 5, 64, "bf16"),  # large tiles on projection bounds
    (605, 2400, 192, (256, 64), 4, 16, "bf16"),        # long segments: MFMA shrink
    (606, 70, 64, (32, 16, 24), 4, 16, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
@pytest.mark.parametrize("policy", ["exact", "padded"])
def test_stacked_cases(case, policy):
    seed, n, d_in, outs, n_slots, r_max, dtype = case
    say("stacked", case, policy)
    ws = _projections(seed, n, d_in, outs, n_slots, r_max, dtype)
    if n_slots > 2:
        for w in ws:
            w.slot_rank[1] = 0
    out = _run(ws, _stacked_pool(ws, policy))
    e = _check(ws, out)
    say("stacked errors", e)


@pytest.mark.parametrize("n", [200, 900])
def test_stacked_b_layouts_give_identical_bits(n):
    ws = _projections(610, n, 136, (136, 72, 200), 8, 32)
    a = _run(ws, _stacked_pool(ws, natural_b=True), separate=False)
    b = _run(ws, _stacked_pool(ws, natural_b=False), separate=False)
    assert torch.equal(a["fused"], b["fused"])


def test_stacked_dora():
    ws = _projections(611, 260, 128, (64, 48), 5, 16)
    b = ws[0]
    pool = _stacked_pool(ws, dora=True)
    W = torch.cat([wl.to_torch(w.W, "bf16", DEV) for w in ws], dim=0).contiguous()
    mags = [wl.make_magnitude(611 + q, b.n_slots, w.d_out, 0.02 * math.sqrt(b.d_in), p_plain=0.25)
            for q, w in enumerate(ws)]
    for a in range(b.n_slots):
        if mags[0][a] is not None:
            m = np.concatenate([np.ones(w.d_out, np.float32) if mg[a] is None else mg[a]
                                for w, mg in zip(ws, mags)])
            pool.dora_prepare(a, W, torch.from_numpy(m).to(DEV))
    out = _run(ws, pool, W=W)
    # per projection: DoRA for the slots prepared above (a magnitude of ones
    # where that projection had none: still normalised), plain otherwise
    Ys = []
    for q, w in enumerate(ws):
        mq = [None if mags[0][a] is None else
              (np.ones(w.d_out, np.float32) if mags[q][a] is None else mags[q][a])
              for a in range(b.n_slots)]
        Ys.append(oracle.dora_forward(b.X, w.W, w.A, w.B, b.row_slot, b.slot_rank, b.slot_alpha,
                                      mq, b.r_max, "bf16"))
    Y = np.concatenate(Ys, axis=1)
    for k in ("fused", "separate"):
        e = normwise(to_f64(out[k]), Y)
        assert e <= TOL["bf16"], (k, e)


@pytest.mark.parametrize("n", [200, 900])
def test_stacked_fp8_weight(n):
    ws = _projections(612, n, 144, (144, 64, 80), 6, 32)
    b = ws[0]
    q8 = [wl.make_fp8_weight(612 + q, w.d_out, w.d_in) for q, w in enumerate(ws)]
    codes = np.concatenate([c for c, _ in q8], axis=0)
    scale = np.concatenate([s for _, s in q8])
    fp8 = (torch.from_numpy(codes).to(DEV), torch.from_numpy(scale).to(DEV))
    out = _run(ws, _stacked_pool(ws), fp8=fp8, separate=False)
    refs = [oracle.lora_forward_fp8w(b.X, c, s, w.A, w.B, b.row_slot, b.slot_rank, b.slot_alpha,
                                     b.r_max, "bf16") for (c, s), w in zip(q8, ws)]
    ref = tuple(np.concatenate([r[i] for r in refs], axis=1) for i in range(3))
    _check(ws, out, ref=ref)


def test_stacked_qkv_70b_shapes_sampled():
    """The 70B-shaped layer's q, k, v projections (8192 -> 8192 / 1024 / 1024,
    2304 rows, 64 slots with ranks 16 and 64) as one fused QKV call."""
    ws = [wl.layer70b_projection(p) for p in ("q_proj", "k_proj", "v_proj")]
    b = ws[0]
    for w in ws[1:]:
        w.X = b.X                       # one input for the three projections
    out = _run(ws, _stacked_pool(ws), separate=False)
    meta = oracle.segment_metadata(b.row_slot, b.slot_rank, b.slot_alpha, b.r_max)
    rows = sample_rows(b, meta, 96, extra=range(2048, 2304, 8))
    say("stacked qkv", _check(ws, out, rows=rows))
