"""GPU parity of the row-by-row LoRA epilogue of the 128 x 128, 192 x 256 and
256 x 256 tiles of the fused layer (adapter-batching page, Multi-LoRA Serving, section
"一个混合 Batch 的数学形式": every row gets its own adapter's term).  Such a
tile switches from one staged MFMA increment per segment to the row
epilogue when its rows hold more than a few LoRA runs (decode rows, each of
its own adapter), so the cases here put many short runs, a run count on
either side of that switch, and prefill runs mixed with decode rows into
tiles of both sizes, and decode rows at either end of a grid of several
waves (where the end tile with more runs is scheduled first).  Same
tolerances and bitwise properties as the plain layer; DoRA factors and an
FP8 weight through the same epilogue."""
import math

import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_segment_amd as srg
import workloads as wl
from gpu_harness import (DEV, TOL, base_rows_bitwise, check_metadata, check_values, normwise,
                         run_hip, say, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    srg.lib()
    yield
    torch.cuda.synchronize()


def _mapped(seed, row_slot, d_in, d_out, ranks, dtype="bf16"):
    """A workload with the given row -> slot mapping (-1: base only)."""
    return wl.build_workload(f"mapped_s{seed}", dtype, np.random.SeedSequence(seed), len(row_slot),
                             d_in, d_out, row_slot, ranks, 64, 1.0, 0.02, 0.02)


def _runs_per_tile(tile_rows, n_tiles, n_slots, rng, base_run=True):
    """Tile t of `tile_rows` rows split into t + 1 runs of distinct slots
    (one of them base-only in every third tile when base_run)."""
    out = []
    for t in range(n_tiles):
        k = t + 1
        cuts = np.sort(rng.choice(np.arange(1, tile_rows), size=k - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [tile_rows]]))
        slots = rng.choice(n_slots, size=k, replace=False)
        if base_run and t % 3 == 2:
            slots[k // 2] = -1
        for L, s in zip(lens, slots):
            out.extend([int(s)] * int(L))
    return np.array(out, dtype=np.int32)


# ---------------------------------------------------------------- many short runs
MANY = [
    # seed, n, d_in, d_out, n_slots, p_base: random rows (one run per row or so)
    (701, 1024, 256, 1032, 50, 0.1),     # 128 x 128 tiles, ragged N
    (702, 1100, 200, 8200, 40, 0.1),     # 192 x 256 tiles, K tail, ragged M and N
    (703, 600, 136, 11008, 70, 0.3),     # 192 x 256 tiles, ragged M
    (708, 2040, 200, 7944, 40, 0.1),     # 256 x 256 tiles, K tail, ragged M and N
    (709, 2100, 200, 8200, 40, 0.1),     # split: 256 x 256 tiles, then 64 x 64 from row 1792
]


@pytest.mark.parametrize("case", MANY, ids=[f"s{c[0]}" for c in MANY])
@pytest.mark.parametrize("policy", ["exact", "padded"])
def test_many_runs(case, policy):
    seed, n, d_in, d_out, n_slots, p_base = case
    say("row tiles", case, policy)
    w = wl.make_random(seed, n, d_in, d_out, n_slots, 64, p_base=p_base)
    w.slot_rank[3] = 0
    r = run_hip(w, policy)
    check_metadata(w, r)
    say("errors", check_values(w, r))
    base_rows_bitwise(w, r)


# ---------------------------------------------------------------- around the switch
@pytest.mark.parametrize("shape", [(1024, 264, 128), (768, 11008, 192), (1024, 12288, 256)],
                         ids=["tile128", "tile192", "tile256"])
def test_run_counts_around_the_switch(shape):
    """Tiles with 1, 2, ..., 8 runs (128-row tiles) or 1, 2, 3, 4 runs (192-
    and 256-row tiles), then more runs in the last 256 rows, so tiles on both
    sides of the switch."""
    n, d_out, tile = shape
    rng = np.random.default_rng(704)
    row_slot = _runs_per_tile(tile, n // tile, 12, rng)
    if tile > 128:               # more runs in the last 256 rows
        row_slot[n - 256:] = _runs_per_tile(32, 8, 12, rng, base_run=False)
    ranks = [8, 16, 32, 64, 0, 16, 64, 8, 32, 64, 16, 8]
    w = _mapped(704, row_slot, 96, d_out, ranks)
    say("switch", shape)
    r = run_hip(w)
    check_metadata(w, r)
    say("errors", check_values(w, r))
    base_rows_bitwise(w, r)


def test_prefill_and_decode_rows_in_one_tile():
    """One long request, a base-only run and decode rows of random slots,
    sharing tiles."""
    rng = np.random.default_rng(705)
    row_slot = np.concatenate([np.full(300, 5), np.full(40, -1), rng.integers(0, 30, 90),
                               np.full(200, 7), rng.integers(-1, 30, 70)]).astype(np.int32)
    ranks = rng.choice([8, 16, 32, 64], size=30)
    for d_out in (520, 11008):
        w = _mapped(705, row_slot, 200, d_out, ranks)
        r = run_hip(w)
        check_metadata(w, r)
        say("mixed", d_out, check_values(w, r))
        base_rows_bitwise(w, r)


@pytest.mark.parametrize("n,d_out", [(1024, 1032), (1100, 8200)])
def test_b_layouts_give_identical_bits(n, d_out):
    w = wl.make_random(706, n, 200, d_out, 30, 64, p_base=0.1)
    d = wl.device_tensors(w, DEV)
    a = run_hip(w, d=d, separate=False, natural_b=True)
    b = run_hip(w, d=d, separate=False, natural_b=False)
    assert torch.equal(a.Yf, b.Yf)


# ---------------------------------------------------------------- DoRA and FP8 weights
@pytest.mark.parametrize("n,d_out", [(1024, 264), (600, 11008)])
def test_dora_many_runs(n, d_out):
    w = wl.make_random(707, n, 128, d_out, 20, 64, p_base=0.15)
    w.slot_rank[2] = 0
    mag = wl.make_magnitude(707, w.n_slots, w.d_out, 0.02 * math.sqrt(w.d_in), p_plain=0.25)
    d = wl.device_tensors(w, DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, "exact", dora=True)
    for a in range(w.n_slots):
        if mag[a] is not None:
            pool.dora_prepare(a, d["W"], torch.from_numpy(mag[a]).to(DEV))
    seg = srg.Segments(w.n, w.n_slots, DEV)
    H = torch.full((w.n, w.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_build_shrink(d["row_slot"], d["X"], pool, seg, H)
    Yf = torch.empty((w.n, w.d_out), dtype=torch.bfloat16, device=DEV)
    srg.lora_linear_fused(d["X"], d["W"], H, seg, pool, Yf)
    Yb = torch.empty_like(Yf)
    srg.lora_base_gemm(d["X"], d["W"], Yb)
    torch.cuda.synchronize()
    ref = oracle.dora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha, mag,
                              w.r_max, w.dtype)
    e = normwise(to_f64(Yf), ref)
    say("dora row tiles", n, d_out, e)
    assert e <= TOL["bf16"]
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    base = [i for i in range(w.n) if keys[i] < 0 or int(w.slot_rank[keys[i]]) == 0]
    tb = torch.as_tensor(base, device=DEV)
    assert torch.equal(Yf[tb], Yb[tb])


@pytest.mark.parametrize("n,d_out", [(1024, 264), (600, 11008)])
def test_fp8_weight_many_runs(n, d_out):
    w = wl.make_random(708, n, 144, d_out, 25, 64, p_base=0.1)
    codes, scale = wl.make_fp8_weight(708, d_out, w.d_in)
    d = wl.device_tensors(w, DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, "exact")
    seg = srg.Segments(w.n, w.n_slots, DEV)
    H = torch.full((w.n, w.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_build_shrink(d["row_slot"], d["X"], pool, seg, H)
    Wq = torch.from_numpy(codes).to(DEV)
    ws = torch.from_numpy(scale).to(DEV)
    Yf = torch.empty((w.n, w.d_out), dtype=torch.bfloat16, device=DEV)
    srg.lora_linear_fused_fp8w(d["X"], Wq, ws, H, seg, pool, Yf)
    Yb = torch.empty_like(Yf)
    srg.lora_base_gemm_fp8w(d["X"], Wq, ws, Yb)
    torch.cuda.synchronize()
    Y, dY, _ = oracle.lora_forward_fp8w(w.X, codes, scale, w.A, w.B, w.row_slot, w.slot_rank,
                                        w.slot_alpha, w.r_max, w.dtype)
    e = {"fused": normwise(to_f64(Yf), Y), "base": normwise(to_f64(Yb), Y - dY)}
    say("fp8 row tiles", n, d_out, e)
    assert max(e.values()) <= TOL["bf16"]
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    base = [i for i in range(w.n) if keys[i] < 0]
    tb = torch.as_tensor(base, device=DEV)
    assert torch.equal(Yf[tb], Yb[tb])


@pytest.mark.parametrize("where", ["first", "last", "both"])
def test_decode_rows_at_either_end_of_a_multi_wave_grid(where):
    """Decode rows (one random slot each) at the start, the end or both ends
    of a 1300-row batch with a prefill request in between, on a grid of more
    than one wave of 256 x 256 tiles, so the tile with more runs is ordered
    first (or, with both ends alike, neither is)."""
    rng = np.random.default_rng({"first": 711, "last": 712, "both": 713}[where])
    dec = lambda k: rng.integers(-1, 40, k)
    pre = np.full(1300 - 200 if where != "both" else 1300 - 400, 7)
    parts = {"first": [dec(200), pre], "last": [pre, dec(200)], "both": [dec(200), pre, dec(200)]}
    row_slot = np.concatenate(parts[where]).astype(np.int32)
    ranks = rng.choice([8, 16, 32, 64], size=40)
    w = _mapped(714, row_slot, 64, 12288, ranks)
    r = run_hip(w)
    check_metadata(w, r)
    say("either end", where, check_values(w, r))
    base_rows_bitwise(w, r)


@pytest.mark.parametrize("runs", [False, True], ids=["rows", "requests"])
@pytest.mark.parametrize("n,d_out", [(1024, 264), (600, 11008), (300, 264)])
def test_ranks_not_multiples_of_eight(n, d_out, runs):
    """Ranks 1, 5, 12, 24, 33, 47, 64 (a pool of r_max 64): each epilogue
    reads whole chunks of rank rows and must skip the rows at or past the
    rank, also when another item's rank runs further (the two-item step);
    random rows take the row epilogues, contiguous requests the staged MFMA
    term of the larger tiles."""
    ranks = [1, 5, 12, 24, 33, 47, 64, 12, 5]
    w = wl.make_random(715, n, 136, d_out, len(ranks), 64, ranks=ranks, p_base=0.1, runs=runs)
    r = run_hip(w)
    check_metadata(w, r)
    say("odd ranks", n, d_out, check_values(w, r))
    base_rows_bitwise(w, r)
