"""GPU tests of the pool set-up calls, which keep the method's scale and the
pool's layouts inside the library (LoRA/QLoRA 多租户GPU推理服务化实战, sections
1.1-1.2: one preallocated buffer of uniform slots, the alpha / r scaling in
the kernel library; adapter-batching page, "Adapter 不是一块连续 Weight": each
target projection has its own A and B):

* lora_pool_set_scales: slot_scale = alpha / r rounded once to float32, for
  alphas that make the quotient inexact too;
* lora_pool_write_b: the d_out-major B is exactly Bt transposed;
* lora_pool_pack_slot on a stacked pool: per-projection sources in either B
  layout give the stacked layout (A: each projection's own rank rows; Bt and
  B: each column's own projection in one projection's rank rows, zeros past
  the rank) and the oracle's outputs per projection.
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


def test_set_scales_rounds_alpha_over_rank_once():
    ranks = [8, 3, 0, 64, 5, 16, 7, 1]
    alphas = [16.0, 10.0, 12.0, 0.1, 7.3, 32.0, 1e-3, 3.0]
    A = torch.zeros((8, 64, 64), dtype=torch.bfloat16, device=DEV)
    Bt = torch.zeros((8, 64, 72), dtype=torch.bfloat16, device=DEV)
    pool = srg.Pool(A, Bt, torch.tensor(ranks, dtype=torch.int32), alphas)
    torch.cuda.synchronize()
    want = np.array([np.float32(a / r) if r > 0 else np.float32(0) for a, r in zip(alphas, ranks)],
                    dtype=np.float32)
    got = pool.slot_scale.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (got, want)


@pytest.mark.parametrize("dtype,r_max,d_out", [("bf16", 64, 200), ("f32", 16, 72),
                                               ("bf16", 8, 4104)])
def test_write_b_is_bt_transposed(dtype, r_max, d_out):
    w = wl.make_random(70 + r_max, 10, 64, d_out, 5, r_max, dtype=dtype)
    d = wl.device_tensors(w, DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha)
    torch.cuda.synchronize()
    # bit patterns (NaN padding included) compared as integers
    it = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(pool.B.view(it), d["Bt"].view(it).transpose(1, 2).contiguous())


def _proj_workloads(seed, n, d_in, outs, n_slots, r_max, dtype="bf16"):
    ws = []
    for p, d_out in enumerate(outs):
        w = wl.make_random(seed * 10 + p, n, d_in, d_out, n_slots, r_max, p_base=0.15,
                           dtype=dtype, runs=True, pad="zero",
                           ranks=None if p == 0 else list(ws[0].slot_rank))
        if p:
            w.X, w.row_slot = ws[0].X, ws[0].row_slot
        ws.append(w)
    return ws


@pytest.mark.parametrize("b_layout", ["rows", "rank_rows"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_stacked_pool(b_layout, dtype):
    outs = (136, 72, 200)
    ws = _proj_workloads(75, 300, 128, outs, 6, 32, dtype)
    b = ws[0]
    b.slot_rank[2] = 0
    for w in ws[1:]:
        w.slot_rank[:] = b.slot_rank
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pool = srg.Pool.empty(b.n_slots, 32, b.d_in, 0, dtype=tdt, device=DEV, proj_outs=outs)
    assert pool.r_max == 96 and pool.d_out == sum(outs)
    for a in range(b.n_slots):
        r = int(b.slot_rank[a])
        As = [wl.to_torch(w.A[a, :r], dtype, DEV) for w in ws]
        if b_layout == "rows":
            Bs = [wl.to_torch(np.ascontiguousarray(w.B[a, :, :r]), dtype, DEV) for w in ws]
        else:
            Bs = [wl.to_torch(w.Bt[a, :r], dtype, DEV) for w in ws]
        pool.pack(a, As, Bs, 16.0, b_layout=b_layout)
    torch.cuda.synchronize()
    # layout: projection q's A rows at [32 q, 32 q + r); B^T in rank rows
    # [0, r) over projection q's own columns (each column holds its own
    # projection, so Bt and B take one projection's 32 rank rows), zeros past
    # the rank; the d_out-major copy likewise
    assert tuple(pool.Bt.shape) == (b.n_slots, 32, sum(outs))
    assert tuple(pool.B.shape) == (b.n_slots, sum(outs), 32)
    it = torch.int16 if dtype == "bf16" else torch.int32
    cols = np.cumsum((0,) + outs)
    Aref = torch.zeros_like(pool.A)
    Btref = torch.zeros_like(pool.Bt)
    for q, w in enumerate(ws):
        dq = wl.device_tensors(w, DEV)
        for a in range(b.n_slots):
            r = int(b.slot_rank[a])
            Aref[a, 32 * q:32 * q + r] = dq["A"][a, :r]
            Btref[a, :r, cols[q]:cols[q + 1]] = dq["Bt"][a, :r]
    assert torch.equal(pool.A.view(it), Aref.view(it))
    assert torch.equal(pool.Bt.view(it), Btref.view(it))
    assert torch.equal(pool.B.view(it), Btref.view(it).transpose(1, 2).contiguous())
    exp_scale = np.array([np.float32(16.0 / r) if r else 0 for r in b.slot_rank], np.float32)
    assert np.array_equal(pool.slot_scale.cpu().numpy(), exp_scale)
    # the same pool as Pool.stacked builds from per-projection pools
    pools = []
    for w in ws:
        dw = wl.device_tensors(w, DEV)
        pools.append(srg.Pool(dw["A"], dw["Bt"], dw["slot_rank"], w.slot_alpha))
    st = srg.Pool.stacked(pools)
    torch.cuda.synchronize()
    assert torch.equal(st.A.view(it), pool.A.view(it)) and torch.equal(st.Bt.view(it), pool.Bt.view(it))
    assert torch.equal(st.B.view(it), pool.B.view(it))
    assert torch.equal(st.slot_scale, pool.slot_scale)
    # outputs per projection against the oracle
    X = wl.to_torch(b.X, dtype, DEV)
    rs = torch.from_numpy(np.ascontiguousarray(b.row_slot)).to(DEV)
    W = torch.cat([wl.to_torch(w.W, dtype, DEV) for w in ws], dim=0).contiguous()
    seg = srg.Segments(b.n, b.n_slots, DEV)
    H = torch.full((b.n, pool.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_build_shrink(rs, X, pool, seg, H)
    Y = torch.empty((b.n, pool.d_out), dtype=tdt, device=DEV)
    srg.lora_linear_fused(X, W, H, seg, pool, Y)
    torch.cuda.synchronize()
    Yr, _, _ = oracle.stacked_forward(b.X, [w.W for w in ws], [w.A for w in ws], [w.B for w in ws],
                                      b.row_slot, b.slot_rank, b.slot_alpha, b.r_max, dtype)
    e = normwise(to_f64(Y), Yr)
    say("packed stacked", b_layout, dtype, e)
    assert e <= TOL[dtype]


def test_repack_stacked_slot_and_empty_it():
    outs = (64, 48)
    ws = _proj_workloads(77, 120, 64, outs, 4, 16)
    b = ws[0]
    pool = srg.Pool.empty(4, 16, 64, 0, device=DEV, proj_outs=outs)
    for a in range(4):
        r = int(b.slot_rank[a])
        pool.pack(a, [wl.to_torch(w.A[a, :r], "bf16", DEV) for w in ws],
                  [wl.to_torch(w.Bt[a, :r], "bf16", DEV) for w in ws], 16.0, b_layout="rank_rows")
    # empty slot 1: its rows become base-only, its blocks zero
    pool.pack(1, [torch.zeros((0, 64), dtype=torch.bfloat16)] * 2,
              [torch.zeros((0, 64)), torch.zeros((0, 48))], 16.0, b_layout="rank_rows")
    torch.cuda.synchronize()
    assert int(pool.slot_rank[1]) == 0 and float(pool.slot_scale[1]) == 0.0
    assert torch.count_nonzero(pool.A[1].float()) == 0 and torch.count_nonzero(pool.Bt[1].float()) == 0
    assert torch.count_nonzero(pool.B[1].float()) == 0
