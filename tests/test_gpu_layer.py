"""GPU parity of the one-call layer lora_layer_fused (adapter-batching page,
Multi-LoRA Serving, sections "一个混合 Batch 的数学形式" and "Segmented Kernel
需要哪些 Metadata"): segment build, shrink and fused product, in one launch
for bf16 batches of up to 512 rows.  Against the oracle:

* the segment metadata bit for bit, H on the written entries [0, rank)
  (and nothing outside them: H starts as NaN), Y within the bf16 tolerance,
  base-only rows bit-identical to the base GEMM;
* the same with no sync buffer (every tile computes its rows' H itself) and
  with many more rows than tiles (workgroups that only compute a row);
* repeated calls on one sync buffer with new inputs each time, eagerly and
  as replays of one captured HIP graph, so a flag left by an earlier call
  can never stand for the current one;
* stacked projections, DoRA, rank policies (identical bits), invalid rows,
  and the two-launch fallback (fp32 pools, more than 512 rows).
"""
import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_segment_amd as srg
import workloads as wl
from gpu_harness import (DEV, TOL, Run, base_rows_bitwise, check_metadata, check_values, normwise,
                         say, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    srg.lib()
    yield
    torch.cuda.synchronize()


def run_layer(w, policy="exact", sync=True, d=None, pool=None, base=True, sync_buf=None):
    d = d or wl.device_tensors(w, DEV)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    pool = pool or srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, policy)
    seg = srg.Segments(w.n, w.n_slots, DEV)
    H = torch.full((w.n, pool.r_max), float("nan"), dtype=torch.float32, device=DEV)
    Y = torch.empty((w.n, pool.d_out), dtype=dt, device=DEV)
    sy = sync_buf if sync_buf is not None else (srg.layer_sync(DEV) if sync else None)
    srg.lora_layer_fused(d["row_slot"], d["X"], d["W"], pool, seg, H, Y, sy)
    out = Run()
    out.pool, out.seg, out.d, out.H, out.Yf, out.sync = pool, seg, d, H, Y, sy
    if base:
        Yb = torch.empty_like(Y)
        srg.lora_base_gemm(d["X"], d["W"], Yb)
        out.Yb = Yb
    torch.cuda.synchronize()
    out.meta = seg.to_host()
    return out


def full_check(w, r):
    check_metadata(w, r)
    e = check_values(w, r)
    base_rows_bitwise(w, r)
    return e


def test_decode_configuration():
    """Decode workload (256 rows, d 4096, 128 slots of rank 16): one launch."""
    w = wl.make_workload("decode")
    r = run_layer(w)
    say("layer decode", full_check(w, r))
    # the same product as the two calls, up to the order of H's additions
    d = r.d
    seg = srg.Segments(w.n, w.n_slots, DEV)
    H2 = torch.full_like(r.H, float("nan"))
    Y2 = torch.empty_like(r.Yf)
    srg.lora_build_shrink(d["row_slot"], d["X"], r.pool, seg, H2)
    srg.lora_linear_fused(d["X"], d["W"], H2, seg, r.pool, Y2)
    torch.cuda.synchronize()
    assert normwise(to_f64(r.H.nan_to_num(0)), to_f64(H2.nan_to_num(0))) < 1e-5
    diff = (r.Yf.float() - Y2.float()).abs().max().item()
    say("layer vs two calls, max |dY|", diff)
    assert normwise(to_f64(r.Yf), to_f64(Y2)) < 1e-2


CASES = [
    # seed, n, d_in, d_out, n_slots, r_max, p_base, runs
    (601, 1, 64, 72, 3, 8, 0.0, False),
    (602, 7, 136, 200, 5, 16, 0.3, False),
    (603, 64, 512, 4096, 40, 64, 0.1, False),     # rank 64: four passes of 16 rank rows
    (604, 300, 520, 264, 40, 64, 0.1, False),     # 25 tiles, 300 rows: row-only workgroups
    (605, 333, 256, 384, 6, 32, 0.2, True),
    (606, 257, 96, 88, 300, 16, 0.5, False),
    (607, 512, 256, 4104, 60, 32, 0.1, False),    # more tiles than CUs (two-stage tiles), N tail
    (608, 512, 4104, 1024, 20, 16, 0.1, False),   # d_in past one chunk per thread, K tail
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
@pytest.mark.parametrize("sync", [True, False], ids=["handoff", "local"])
def test_random_cases(case, sync):
    seed, n, d_in, d_out, n_slots, r_max, p_base, runs = case
    say("layer", case, sync)
    w = wl.make_random(seed, n, d_in, d_out, n_slots, r_max, p_base=p_base, runs=runs)
    w.slot_rank[min(2, n_slots - 1)] = 0
    r = run_layer(w, sync=sync)
    say("errors", full_check(w, r))


def test_ranks_not_multiples_of_eight():
    w = wl.make_random(610, 200, 256, 512, 12, 32, ranks=[1, 3, 5, 7, 9, 13, 17, 31, 32, 0, 2, 8],
                       p_base=0.1)
    r = run_layer(w)
    say("odd ranks", full_check(w, r))


def test_invalid_rows_are_base_and_counted():
    w = wl.make_random(611, n=200, d_in=64, d_out=64, n_slots=10, r_max=16)
    w.slot_rank[3] = 40            # > r_max: every row on slot 3 is demoted
    w.row_slot[5] = 10             # >= n_slots
    w.row_slot[6] = -2
    w.row_slot[7] = 1 << 20
    r = run_layer(w)
    ref = check_metadata(w, r)
    assert ref["status"] >= 3 and r.meta["status"] == ref["status"]
    check_values(w, r)
    base_rows_bitwise(w, r)


def test_all_rows_one_adapter_and_all_base():
    w = wl.make_random(612, n=130, d_in=128, d_out=96, n_slots=5, r_max=64)
    w.row_slot[:] = 2
    r = run_layer(w)
    assert int(check_metadata(w, r)["num_segments"]) == 1
    check_values(w, r)
    w.row_slot[:] = -1
    r = run_layer(w)
    check_metadata(w, r)
    assert torch.equal(r.Yf, r.Yb)


def test_policies_give_identical_bits():
    w = wl.make_random(613, n=300, d_in=256, d_out=192, n_slots=30, r_max=64)
    outs = [run_layer(w, p) for p in ("exact", "two_buckets", "padded")]
    check_values(w, outs[0])
    for o in outs[1:]:
        assert torch.equal(o.H.nan_to_num(0), outs[0].H.nan_to_num(0))
        assert torch.equal(o.Yf, outs[0].Yf)


def test_handoff_and_local_give_identical_bits():
    """Whether a row's H comes from another workgroup or is computed by the
    tile itself, it is the same sum, so the outputs are the same bits."""
    w = wl.make_random(614, n=256, d_in=1024, d_out=2048, n_slots=50, r_max=16)
    a = run_layer(w, sync=True)
    b = run_layer(w, sync=False, d=a.d)
    assert torch.equal(a.H.nan_to_num(0), b.H.nan_to_num(0))
    assert torch.equal(a.Yf, b.Yf)


def test_fingerprint_mapping_exact():
    """Every row must pick up its own slot's adapter: with fingerprint
    adapters (A_a row 0 the unit vector at a mod d_in) H[i][0] of a LoRA row
    is exactly x_i[a mod d_in], and Y is within tolerance of the oracle."""
    w = wl.make_fingerprint(615, 400, 512, 256, 200, 16)
    r = run_layer(w)
    check_metadata(w, r)
    say("fingerprint", check_values(w, r))
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    H = r.H.cpu().numpy()
    Xf = w.as_f32("X")
    for i in range(w.n):
        a = keys[i]
        if a >= 0 and w.slot_rank[a] > 0:
            assert H[i, 0] == np.float32(Xf[i, a % w.d_in]), i


@pytest.mark.parametrize("graph", [False, True], ids=["eager", "graph"])
def test_repeated_calls_see_fresh_inputs(graph):
    """One sync buffer, many calls with new X and a new mapping in place
    each time: every call's outputs match the oracle for its own inputs (a
    flag from an earlier call never stands for the current one).  As graph
    replays, with eager work and synchronisation between them."""
    n, d_in, d_out, n_slots, r_max = 256, 512, 2048, 40, 16
    ws = [wl.make_random(620 + k, n, d_in, d_out, n_slots, r_max, p_base=0.1) for k in range(4)]
    base = ws[0]
    for w in ws[1:]:                   # one pool and W; new X and mapping per call
        w.A, w.Bt, w.W, w.slot_rank, w.slot_alpha = base.A, base.Bt, base.W, base.slot_rank, \
            base.slot_alpha
    d = wl.device_tensors(base, DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], base.slot_alpha)
    seg = srg.Segments(n, n_slots, DEV)
    H = torch.full((n, r_max), float("nan"), dtype=torch.float32, device=DEV)
    Y = torch.empty((n, d_out), dtype=torch.bfloat16, device=DEV)
    sy = srg.layer_sync(DEV)
    X, rs = d["X"], d["row_slot"]

    def call():
        srg.lora_layer_fused(rs, X, d["W"], pool, seg, H, Y, sy)

    if graph:
        call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
    for rep in range(2):
        for k, w in enumerate(ws):
            dk = wl.device_tensors(w, DEV)
            X.copy_(dk["X"])
            rs.copy_(dk["row_slot"])
            H.fill_(float("nan"))
            torch.cuda.synchronize()
            if graph:
                g.replay()
            else:
                call()
            torch.cuda.synchronize()
            r = Run()
            r.H, r.Yf, r.seg = H, Y, seg
            r.meta = seg.to_host()
            check_metadata(w, r)
            e = check_values(w, r)
            say("repeat", graph, rep, k, e)
            _ = (Y.float() * 2).sum().item()          # eager work between calls


def test_stacked_projections():
    """q|k|v-shaped stacked pool: every projection's output and H columns."""
    outs = (512, 128, 128)
    ws = []
    for p, d_out in enumerate(outs):
        w = wl.make_random(630 + p, 200, 512, d_out, 12, 16, p_base=0.1, pad="zero",
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
    W = torch.cat([wl.to_torch(w.W, "bf16", DEV) for w in ws], dim=0).contiguous()
    d = {"X": wl.to_torch(b.X, "bf16", DEV), "W": W,
         "row_slot": torch.from_numpy(np.ascontiguousarray(b.row_slot)).to(DEV)}
    seg = srg.Segments(b.n, b.n_slots, DEV)
    H = torch.full((b.n, st.r_max), float("nan"), dtype=torch.float32, device=DEV)
    Y = torch.empty((b.n, st.d_out), dtype=torch.bfloat16, device=DEV)
    srg.lora_layer_fused(d["row_slot"], d["X"], W, st, seg, H, Y, srg.layer_sync(DEV))
    torch.cuda.synchronize()
    Yr, _, _ = oracle.stacked_forward(b.X, [w.W for w in ws], [w.A for w in ws],
                                      [w.B for w in ws], b.row_slot, b.slot_rank, b.slot_alpha,
                                      b.r_max, "bf16")
    e = normwise(to_f64(Y), Yr)
    say("stacked", e)
    assert e <= TOL["bf16"]


def test_dora_pool():
    w = wl.make_random(640, 256, 256, 512, 20, 32, p_base=0.15)
    w.slot_rank[2] = 0
    mag = wl.make_magnitude(640, w.n_slots, w.d_out, 0.02 * np.sqrt(w.d_in), p_plain=0.25)
    d = wl.device_tensors(w, DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, "exact", dora=True)
    for a in range(w.n_slots):
        if mag[a] is not None:
            pool.dora_prepare(a, d["W"], torch.from_numpy(mag[a]).to(DEV))
    r = run_layer(w, d=d, pool=pool)
    Yr = oracle.dora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha, mag,
                             w.r_max, w.dtype)
    e = normwise(to_f64(r.Yf), Yr)
    say("dora", e)
    assert e <= TOL["bf16"]
    check_metadata(w, r)


@pytest.mark.parametrize("kind", ["f32", "rows_past_one_launch"])
def test_two_call_fallback(kind):
    if kind == "f32":
        w = wl.make_random(650, 70, 64, 64, 4, 64, p_base=0.1, dtype="f32")
    else:
        w = wl.make_random(651, 600, 256, 264, 30, 32, p_base=0.1)
    r = run_layer(w)
    say("fallback", kind, full_check(w, r))


def test_empty_batch():
    w = wl.make_random(652, n=0, d_in=64, d_out=64, n_slots=3, r_max=8)
    r = run_layer(w, base=False)
    assert r.meta["num_segments"] == 0 and r.meta["status"] == 0
