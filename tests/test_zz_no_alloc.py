"""GPU parity of the allocation-free layer call, lora_linear_fused_static:
its output must equal, bit for bit, lora_build_shrink followed by
lora_linear_fused on caller buffers (the same kernels), and the oracle
within the layer's tolerance.  Two calls in a row on one stream share the
static scratch, the second with a smaller batch (and another pool), so what
the first call left there must not leak into the second."""
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


def _with_buffers(w, d, pool):
    """The existing entry points on caller-owned metadata and H."""
    seg = srg.Segments(w.n, w.n_slots, DEV)
    H = torch.zeros((w.n, pool.r_max), dtype=torch.float32, device=DEV)
    srg.lora_build_shrink(d["row_slot"], d["X"], pool, seg, H)
    Y = torch.empty((w.n, w.d_out), dtype=d["X"].dtype, device=DEV)
    srg.lora_linear_fused(d["X"], d["W"], H, seg, pool, Y)
    return Y


CASES = [
    # (first call, second smaller call): seed, n, d_in, d_out, n_slots, r_max, dtype, runs
    ((901, 2300, 256, 520, 12, 64, "bf16", True), (902, 200, 256, 520, 12, 64, "bf16", False)),
    ((903, 700, 136, 1032, 40, 32, "bf16", False), (904, 33, 200, 264, 7, 16, "bf16", True)),
    ((905, 300, 128, 136, 9, 32, "f32", True), (906, 32, 128, 136, 9, 32, "f32", False)),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0][0]}" for c in CASES])
def test_static_call_matches_buffered_call(case):
    ws, ds, pools, outs = [], [], [], []
    for seed, n, d_in, d_out, n_slots, r_max, dtype, runs in case:
        w = wl.make_random(seed, n, d_in, d_out, n_slots, r_max, p_base=0.1, dtype=dtype,
                           runs=runs)
        w.slot_rank[1] = 0
        d = wl.device_tensors(w, DEV)
        pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha)
        ws.append(w)
        ds.append(d)
        pools.append(pool)
        outs.append(torch.full((n, d_out), float("nan"), dtype=d["X"].dtype, device=DEV))
    say("static call", [c[:2] for c in case])
    # two calls in a row on one stream, the second smaller: same scratch
    for w, d, pool, Y in zip(ws, ds, pools, outs):
        srg.lora_linear_fused_static(d["row_slot"], d["X"], d["W"], pool, Y)
    torch.cuda.synchronize()
    for w, d, pool, Y in zip(ws, ds, pools, outs):
        ref = _with_buffers(w, d, pool)
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), w.name
        Yr, _, _ = oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                       w.r_max, w.dtype)
        e = normwise(to_f64(Y), Yr)
        assert e <= TOL[w.dtype], (w.name, e)
        say("static", w.name, w.n, e)


def test_static_call_repeated_and_empty():
    """A call after a larger one, then an empty batch (no-op), then the first
    again: the same bits each time."""
    w = wl.make_random(907, 400, 192, 264, 20, 16, p_base=0.2)
    d = wl.device_tensors(w, DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha)
    big = wl.make_random(908, 1500, 192, 264, 20, 16, p_base=0.2, runs=True)
    db = wl.device_tensors(big, DEV)
    Yb = torch.empty((big.n, big.d_out), dtype=torch.bfloat16, device=DEV)
    srg.lora_linear_fused_static(db["row_slot"], db["X"], db["W"], pool, Yb)
    Y1 = torch.empty((w.n, w.d_out), dtype=torch.bfloat16, device=DEV)
    srg.lora_linear_fused_static(d["row_slot"], d["X"], d["W"], pool, Y1)
    e = torch.empty((0, w.d_out), dtype=torch.bfloat16, device=DEV)
    srg.lora_linear_fused_static(torch.empty(0, dtype=torch.int32, device=DEV),
                                 torch.empty((0, w.d_in), dtype=torch.bfloat16, device=DEV),
                                 d["W"], pool, e)
    Y2 = torch.empty_like(Y1)
    srg.lora_linear_fused_static(d["row_slot"], d["X"], d["W"], pool, Y2)
    torch.cuda.synchronize()
    ref = _with_buffers(w, d, pool)
    torch.cuda.synchronize()
    assert torch.equal(Y1, ref) and torch.equal(Y2, ref)
    assert torch.equal(Yb, _with_buffers(big, db, pool))


def test_static_call_stacked_pool():
    """A stacked pool (two projections of one input, B stored once per
    column): the same bits as the buffered calls, and the oracle per
    projection."""
    ws = []
    for p, d_out in enumerate((200, 136)):
        w = wl.make_random(910 + p, 600, 128, d_out, 10, 32, p_base=0.1, runs=True,
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
    d = wl.device_tensors(b, DEV)
    d["W"] = torch.cat([wl.to_torch(w.W, "bf16", DEV) for w in ws], dim=0).contiguous()
    Y = torch.full((b.n, st.d_out), float("nan"), dtype=torch.bfloat16, device=DEV)
    srg.lora_linear_fused_static(d["row_slot"], d["X"], d["W"], st, Y)
    # the buffered calls on the same stacked pool
    seg = srg.Segments(b.n, b.n_slots, DEV)
    H = torch.zeros((b.n, st.r_max), dtype=torch.float32, device=DEV)
    srg.lora_build_shrink(d["row_slot"], d["X"], st, seg, H)
    ref = torch.empty_like(Y)
    srg.lora_linear_fused(d["X"], d["W"], H, seg, st, ref)
    torch.cuda.synchronize()
    assert torch.equal(Y, ref)
    Yr, _, _ = oracle.stacked_forward(b.X, [w.W for w in ws], [w.A for w in ws],
                                      [w.B for w in ws], b.row_slot, b.slot_rank, b.slot_alpha,
                                      b.r_max, b.dtype)
    e = normwise(to_f64(Y), Yr)
    assert e <= TOL["bf16"], e
    say("static stacked", b.n, e)


def test_static_call_rejects_oversize_batch():
    w = wl.make_random(909, 16, 64, 64, 3, 64)
    d = wl.device_tensors(w, DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha)
    n = srg.STATIC_MAX_H // 64 + 1
    rs = torch.full((n,), -1, dtype=torch.int32, device=DEV)
    X = torch.zeros((n, 64), dtype=torch.bfloat16, device=DEV)
    Y = torch.zeros((n, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(srg.LoraError) as ei:
        srg.lora_linear_fused_static(rs, X, d["W"], pool, Y)
    assert ei.value.code == -9
    torch.cuda.synchronize()
    assert torch.count_nonzero(Y.float()) == 0          # nothing was launched
