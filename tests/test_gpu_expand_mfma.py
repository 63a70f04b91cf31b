"""GPU parity of the matrix-core expand: bf16 batches whose pool keeps B
d_out-major, large ones and decode-sized ones of rank 32 and more
(adapter-batching page, section "Segmented Kernel 需要哪些 Metadata":
Delta Y_a = s_a H_a B_a^T added back to the rows of segment a).

The increment alone (the expand onto Y = 0) is checked element by element
against the oracle's float64 Delta Y: the kernel rounds once to bf16 (at most
2^-8 relative) and feeds H as a bf16 high part plus a bf16 remainder, which
with the fp32 accumulation stays below 2^-14 of s_a sum_k |h_k b_jk|, so

    |got - ref| <= 2^-8 |ref| + 2^-14 |s_a| sum_k |h_k b_jk|

per element.  The same batch through the GEMV expand (the pool without the
d_out-major copy) must agree within one bf16 step (plus 2^-14 of the largest
magnitude, for sums that cancel), rows of base-only and
rank-0 segments must stay untouched, the rank policies must give identical
bits, and Y = base + increment must match the oracle normwise; DoRA and
stacked pools (projections on and off the 256-column blocks) likewise.
"""
import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_segment_amd as srg
import workloads as wl
from gpu_harness import DEV, TOL, normwise, say, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    srg.lib()
    yield
    torch.cuda.synchronize()


def expand_only(w, policy="exact", natural_b=True, d=None, pool=None):
    """H by the shrink, then the expand onto a zero Y and onto the base."""
    d = d or wl.device_tensors(w, DEV)
    pool = pool or srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, policy,
                            natural_b=natural_b)
    seg = srg.Segments(w.n, w.n_slots, DEV)
    srg.lora_build_segments(d["row_slot"], pool, seg)
    H = torch.full((w.n, pool.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_shrink(d["X"], seg, pool, H)
    dY = torch.zeros((w.n, pool.d_out), dtype=torch.bfloat16, device=DEV)
    srg.lora_expand(H, seg, pool, dY)
    Yb = torch.empty_like(dY)
    srg.lora_base_gemm(d["X"], d["W"], Yb)
    Ys = Yb.clone()
    srg.lora_expand(H, seg, pool, Ys)
    torch.cuda.synchronize()
    return dict(H=H, dY=dY, Yb=Yb, Ys=Ys, pool=pool)


def abs_bound(w, rows):
    """|s_a| sum_k |h_k b_jk| per (row, column), float64, from the oracle's H."""
    _, _, Hr = oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                   w.r_max, w.dtype, rows=rows)
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    out = np.zeros((len(rows), w.d_out))
    babs = {}
    for t, i in enumerate(rows):
        a = keys[i]
        if a < 0 or int(w.slot_rank[a]) == 0:
            continue
        r = int(w.slot_rank[a])
        if a not in babs:
            babs[a] = np.abs(oracle.decode(w.B[a, :, :r], w.dtype))
        out[t] = abs(float(w.slot_alpha[a]) / r) * (babs[a] @ np.abs(Hr[t, :r]))
    return out


def check_increment(w, out, rows=None):
    rows = np.arange(w.n) if rows is None else np.asarray(rows)
    Yr, dYr, _ = oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                     w.r_max, w.dtype, rows=rows)
    ti = torch.as_tensor(rows, device=DEV, dtype=torch.long)
    got = to_f64(out["dY"][ti])
    bound = 2.0 ** -8 * np.abs(dYr) + 2.0 ** -14 * abs_bound(w, rows)
    bad = np.abs(got - dYr) > bound
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5].tolist())
    e = normwise(to_f64(out["Ys"][ti]), Yr)
    assert e <= TOL[w.dtype], e
    # base-only and rank-0 rows: no increment, Y untouched
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    keys = np.asarray(keys)
    base = np.array([k < 0 or int(w.slot_rank[k]) == 0 for k in keys[rows]])
    if base.any():
        tb = torch.as_tensor(rows[base], device=DEV)
        assert torch.count_nonzero(out["dY"][tb].float()) == 0
        assert torch.equal(out["Ys"][tb], out["Yb"][tb])
    return e


def within_one_step(a, b):
    """bf16 tensors equal up to one step of the larger magnitude, plus 2^-14
    of the tensor's largest magnitude for sums that cancel (the two kernels
    add in different orders)."""
    fa, fb = a.float(), b.float()
    step = torch.maximum(fa.abs(), fb.abs()) * 2.0 ** -7 + fb.abs().max() * 2.0 ** -14
    assert bool(((fa - fb).abs() <= step).all()), float(((fa - fb).abs() - step).max())


CASES = [
    # seed, n, d_in, d_out, n_slots, r_max, p_base, runs
    (801, 2048, 256, 512, 6, 64, 0.1, True),      # ranks 8..64, base-only runs
    (802, 2100, 192, 1000, 9, 32, 0.05, True),    # ragged column block (1000 = 3 x 256 + 232)
    (803, 2304, 128, 264, 40, 16, 0.2, False),    # many short segments, rank-16 pool
    (804, 2500, 136, 776, 5, 8, 0.1, True),       # r_max 8: half of each K step masked
    (805, 4100, 64, 2056, 300, 64, 0.3, False),   # 300 slots, mostly single-row items
    # decode-sized batches that take the matrix-core expand by their rank
    # (rank >= 32 and rank x rows >= 32768), with items of each length class:
    (806, 700, 128, 776, 20, 64, 0.0, True),      # request runs: 64-row and partial items
    (807, 1100, 128, 520, 60, 32, 0.1, False),    # about 16 rows per segment: 9..32-row items
    (808, 600, 256, 1000, 200, 64, 0.2, False),   # 1..8-row items, ragged column block
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_increment_elementwise(case):
    seed, n, d_in, d_out, n_slots, r_max, p_base, runs = case
    say("expand mfma", case)
    w = wl.make_random(seed, n, d_in, d_out, n_slots, r_max, p_base=p_base, runs=runs)
    w.slot_rank[min(1, n_slots - 1)] = 0
    a = expand_only(w)
    assert a["pool"].B is not None
    rows = None if n * d_out <= 2100 * 1000 else np.unique(np.concatenate(
        [np.arange(0, n, 7), np.arange(n - 64, n)]))
    e = check_increment(w, a, rows)
    g = expand_only(w, natural_b=False)            # the GEMV expand
    within_one_step(a["dY"], g["dY"])
    within_one_step(a["Ys"], g["Ys"])
    say("error", e)


def test_policies_give_identical_bits():
    w = wl.make_random(810, 2200, 128, 512, 12, 64, p_base=0.1, runs=True)
    outs = [expand_only(w, p) for p in ("exact", "two_buckets", "padded")]
    for o in outs[1:]:
        assert torch.equal(o["dY"], outs[0]["dY"])
        assert torch.equal(o["Ys"], outs[0]["Ys"])
    check_increment(w, outs[0])


def test_dora_pool():
    w = wl.make_random(811, 2100, 256, 768, 10, 32, p_base=0.1, runs=True)
    mag = wl.make_magnitude(811, w.n_slots, w.d_out, 0.02 * np.sqrt(w.d_in), p_plain=0.25)
    outs = {}
    for nb in (True, False):
        d = wl.device_tensors(w, DEV)
        pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, "exact", natural_b=nb,
                        dora=True)
        for s_ in range(w.n_slots):
            if mag[s_] is not None:
                pool.dora_prepare(s_, d["W"], torch.from_numpy(mag[s_]).to(DEV))
        outs[nb] = expand_only(w, d=d, pool=pool)
    within_one_step(outs[True]["Ys"], outs[False]["Ys"])
    Yr = oracle.dora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha, mag,
                             w.r_max, w.dtype)
    e = normwise(to_f64(outs[True]["Ys"]), Yr)
    assert e <= TOL[w.dtype], e
    say("dora error", e)


@pytest.mark.parametrize("outs", [(512, 256, 256), (512, 200, 312)],
                         ids=["on_blocks", "off_blocks"])
def test_stacked_pool(outs):
    """Projections starting on 256-column blocks take the matrix-core expand;
    others take the GEMV expand; both match the oracle per projection."""
    ws = []
    for p, d_out in enumerate(outs):
        w = wl.make_random(812 + p, 2100, 128, d_out, 8, 16, p_base=0.1, runs=True,
                           ranks=None if p == 0 else list(ws[0].slot_rank))
        if p:
            w.X, w.row_slot = ws[0].X, ws[0].row_slot
        ws.append(w)
    b = ws[0]
    pools = []
    for w in ws:
        dw = wl.device_tensors(w, DEV)
        pools.append(srg.Pool(dw["A"], dw["Bt"], dw["slot_rank"], w.slot_alpha))
    st = srg.Pool.stacked(pools)
    X = wl.to_torch(b.X, "bf16", DEV)
    rs = torch.from_numpy(np.ascontiguousarray(b.row_slot)).to(DEV)
    seg = srg.Segments(b.n, b.n_slots, DEV)
    srg.lora_build_segments(rs, st, seg)
    H = torch.full((b.n, st.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_shrink(X, seg, st, H)
    dY = torch.zeros((b.n, st.d_out), dtype=torch.bfloat16, device=DEV)
    srg.lora_expand(H, seg, st, dY)
    torch.cuda.synchronize()
    _, dYr, _ = oracle.stacked_forward(b.X, [w.W for w in ws], [w.A for w in ws],
                                       [w.B for w in ws], b.row_slot, b.slot_rank, b.slot_alpha,
                                       b.r_max, b.dtype)
    c0 = 0
    for w in ws:
        c1 = c0 + w.d_out
        got = to_f64(dY[:, c0:c1])
        ref = dYr[:, c0:c1]
        e = normwise(got, ref)
        assert e <= TOL["bf16"], (c0, e)
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-3 * np.abs(ref).max())
        c0 = c1
