"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Metadata and token mapping must match bit for bit; values within the
normwise tolerance max|got - ref| / max|ref| <= 1e-2 for bf16 storage with
fp32 accumulation and <= 1e-5 for fp32, applied separately to H, Y (fused
and separate paths) and Delta Y.
"""
import copy

import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_segment_amd as srg
import workloads as wl
from gpu_harness import (DEV, TOL, base_rows_bitwise, check_metadata, check_values, normwise,
                         run_hip, sample_rows, say, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    srg.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- the configurations
def test_tiny_f32():
    w = wl.make_workload("tiny_f32")
    say("tiny f32", w.n, w.d_in, w.d_out)
    r = run_hip(w)
    ref = check_metadata(w, r)
    assert ref["segment_offsets"].tolist() == [0, 8, 12, 28, 32]
    e = check_values(w, r)
    base_rows_bitwise(w, r)
    say("tiny f32 errors", e)


def test_decode_bf16():
    w = wl.make_workload("decode")
    say("decode", w.n, w.d_in, w.d_out)
    r = run_hip(w)
    check_metadata(w, r)
    e = check_values(w, r)
    assert base_rows_bitwise(w, r) > 0
    say("decode errors", e)


_CACHE = {}


def _skewed():
    if "skewed" not in _CACHE:
        _CACHE["skewed"] = wl.make_workload("skewed_decode")
    return _CACHE["skewed"]


@pytest.mark.parametrize("policy", ["exact", "two_buckets", "padded"])
def test_skewed_decode_bf16(policy):
    w = _skewed()
    say("skewed decode", policy, w.n, w.d_in, w.d_out, w.n_slots)
    r = run_hip(w, policy)
    check_metadata(w, r)
    e = check_values(w, r)
    say("skewed decode errors", policy, e)


def test_prefill_structure_small():
    """The prefill workload's structure (d 4096 -> 14336, ranks 8..64, request 7
    base-only) with short, ragged requests so the oracle runs every row."""
    w = wl.prefill(lengths_override=[300, 17, 150, 1, 64, 200, 33, 90])
    say("prefill small", w.n, w.d_in, w.d_out)
    r = run_hip(w)
    check_metadata(w, r)
    e = check_values(w, r)
    assert base_rows_bitwise(w, r) == 90
    say("prefill small errors", e)


def test_prefill_full_sampled():
    w = wl.make_workload("prefill")
    say("prefill full", w.n, w.d_in, w.d_out, w.meta)
    r = run_hip(w, separate=False)
    ref = check_metadata(w, r)
    rows = sample_rows(w, ref, 512)
    e = check_values(w, r, rows=rows)
    assert torch.isfinite(r.Yf.float()).all()
    say("prefill full errors (sampled rows)", len(rows), e)


@pytest.mark.parametrize("proj", [p[0] for p in wl.LAYER70B_PROJECTIONS])
def test_layer70b_projection_sampled(proj):
    w = wl.layer70b_projection(proj)
    say("layer70b", proj, w.n, w.d_in, w.d_out)
    r = run_hip(w, separate=False)
    ref = check_metadata(w, r)
    rows = sample_rows(w, ref, 512, extra=range(2048, 2304))
    e = check_values(w, r, rows=rows)
    assert torch.isfinite(r.Yf.float()).all()
    say("layer70b errors", proj, len(rows), e)


# ---------------------------------------------------------------- structure and edge cases
CASES = [
    # seed, n, d_in, d_out, n_slots, r_max, p_base, dtype, runs
    (101, 1, 64, 72, 3, 8, 0.0, "bf16", False),
    (102, 7, 136, 200, 5, 16, 0.3, "bf16", False),
    (103, 300, 520, 264, 40, 64, 0.1, "bf16", False),
    (104, 333, 256, 384, 6, 32, 0.2, "bf16", True),
    (105, 1500, 128, 136, 9, 64, 0.05, "bf16", True),
    (106, 257, 96, 88, 300, 16, 0.5, "bf16", False),
    (107, 70, 64, 64, 4, 64, 0.1, "f32", True),
    (108, 513, 200, 120, 17, 32, 0.1, "f32", False),
    # long segments (tiled shrink) with a ragged K tail, large-tile GEMM K tail
    (109, 700, 200, 136, 7, 64, 0.1, "bf16", True),
    (110, 2100, 328, 264, 5, 32, 0.2, "bf16", True),
    # 128 x 128 tiles (few 256 x 256 tiles) and 256 x 256 tiles with a K tail
    (111, 1024, 256, 1024, 12, 64, 0.1, "bf16", False),
    (112, 1100, 200, 8200, 7, 64, 0.1, "bf16", True),
    # long segments at a long, ragged d_in (MFMA shrink K tail)
    (113, 2100, 8200, 136, 6, 64, 0.1, "bf16", True),
    # small batches with more 64 x 64 tiles than CUs (two-stage small tiles),
    # ragged N and K tails
    (114, 333, 200, 4168, 40, 32, 0.1, "bf16", False),
    (115, 500, 1032, 2056, 9, 64, 0.1, "bf16", True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
@pytest.mark.parametrize("policy", ["exact", "padded"])
def test_random_cases(case, policy):
    seed, n, d_in, d_out, n_slots, r_max, p_base, dtype, runs = case
    say("random", case, policy)
    w = wl.make_random(seed, n, d_in, d_out, n_slots, r_max, p_base=p_base, dtype=dtype, runs=runs)
    r = run_hip(w, policy)
    check_metadata(w, r)
    check_values(w, r)
    base_rows_bitwise(w, r)


@pytest.mark.parametrize("shape", [(400, 136, 4104), (512, 256, 4096), (320, 200, 4168),
                                   (256, 136, 4096)])
def test_short_k_fresh_operands_repeated(shape):
    """Small batches with one or two K stages on freshly copied operands,
    three times each: the GEMM prologue must wait for every stage it
    issued (a one-stage allowance let stage 0 be read before it had fully
    landed on cold operands).  Both paths against the oracle each time."""
    n, d_in, d_out = shape
    w = wl.make_random(400 + n, n, d_in, d_out, 9, 32, p_base=0.1, dtype="bf16", runs=True)
    for rep in range(3):
        say("short K", shape, rep)
        r = run_hip(w)
        check_values(w, r)
        base_rows_bitwise(w, r)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_target", [600, 2300])
def test_segment_lengths_around_row_blocks(n_target, dtype):
    """Segments of 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129 rows
    and longer, in shuffled order, so segments start on and off multiples of
    the shrink / expand row block (16 rows below 2048 rows, 64 from there on)
    and long segments span several blocks; batches on both sides of 2048."""
    rng = np.random.default_rng(n_target)
    lens = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 3, 2]
    while sum(lens) < n_target:
        lens.append(int(rng.integers(1, 90)))
    rng.shuffle(lens)
    n_slots = len(lens) + 2
    slots = rng.permutation(n_slots)[:len(lens)]
    slots[3] = -1                                   # one base-only run
    row_slot = np.concatenate([np.full(L, s) for L, s in zip(lens, slots)]).astype(np.int32)
    ranks = rng.choice([8, 16, 32, 64], size=n_slots).astype(np.int32)
    ranks[slots[5]] = 0                             # one rank-0 run
    w = wl.build_workload("lengths", dtype, np.random.SeedSequence(n_target), len(row_slot), 136,
                          264, row_slot, ranks, 64, 1.0, 0.02, 0.02)
    say("segment lengths", n_target, dtype, len(row_slot))
    r = run_hip(w)
    check_metadata(w, r)
    say("errors", check_values(w, r))
    base_rows_bitwise(w, r)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fingerprint_mapping_exact(dtype):
    """Fingerprint adapters: the increment of a row on slot a is exactly
    s_a (a + 1) x[a mod d_in] (exact in fp32 here), so the expand into zeros
    must equal its rounding bit for bit in every column."""
    w = wl.make_fingerprint(7, n=400, d_in=256, d_out=128, n_slots=60, r_max=32, dtype=dtype)
    r = run_hip(w)
    check_metadata(w, r)
    check_values(w, r)
    X = oracle.decode(w.X, dtype)
    exp = np.zeros((w.n,), dtype=np.float64)
    for i in range(w.n):
        a = int(w.row_slot[i])
        if a >= 0:
            exp[i] = 16.0 / int(w.slot_rank[a]) * (a + 1) * X[i, a % w.d_in]
    exp32 = exp.astype(np.float32)
    assert np.array_equal(exp32.astype(np.float64), exp)
    want = wl.bf16_bits_rne(exp32) if dtype == "bf16" else exp32.view(np.uint32)
    if dtype == "bf16":
        got = r.dY.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        got = r.dY.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, np.repeat(want[:, None], w.d_out, axis=1))


def test_invalid_rows_are_base_and_counted():
    w = wl.make_random(21, n=200, d_in=64, d_out=64, n_slots=10, r_max=16, dtype="bf16")
    w.slot_rank[3] = 40            # > r_max: every row on slot 3 is demoted
    w.row_slot[5] = 10             # >= n_slots
    w.row_slot[6] = -2
    w.row_slot[7] = 1 << 20
    r = run_hip(w)
    ref = check_metadata(w, r)
    assert ref["status"] >= 3 and r.meta["status"] == ref["status"]
    check_values(w, r)
    base_rows_bitwise(w, r)


def test_empty_batch():
    w = wl.make_random(22, n=0, d_in=64, d_out=64, n_slots=3, r_max=8, dtype="bf16")
    r = run_hip(w)
    assert r.meta["num_segments"] == 0 and r.meta["status"] == 0
    assert r.seg.segment_offsets[0].item() == 0


def test_all_rows_one_adapter_and_all_base():
    w = wl.make_random(23, n=130, d_in=128, d_out=96, n_slots=5, r_max=64, dtype="bf16")
    w.row_slot[:] = 2
    r = run_hip(w)
    m = check_metadata(w, r)
    assert int(m["num_segments"]) == 1
    check_values(w, r)
    w.row_slot[:] = -1
    r = run_hip(w)
    check_metadata(w, r)
    check_values(w, r)
    assert torch.equal(r.Yf, r.Yb)


def test_max_slots_pool():
    n_slots = srg.MAX_SLOTS
    w = wl.make_random(24, n=2000, d_in=64, d_out=64, n_slots=n_slots, r_max=8, dtype="bf16",
                       p_base=0.05)
    r = run_hip(w)
    check_metadata(w, r)
    check_values(w, r)


def test_policies_give_identical_bits():
    w = wl.make_random(25, n=600, d_in=256, d_out=192, n_slots=30, r_max=64, dtype="bf16")
    outs = [run_hip(w, p) for p in ("exact", "two_buckets", "padded")]
    for o in outs[1:]:
        assert torch.equal(o.H.nan_to_num(0), outs[0].H.nan_to_num(0))
        assert torch.equal(o.Yf, outs[0].Yf)
        assert torch.equal(o.Ys, outs[0].Ys)


@pytest.mark.parametrize("case", [
    # seed, n, d_in, d_out, n_slots, r_max  (small tiles / large tiles; r_max 8 edge)
    (40, 300, 256, 200, 9, 64),
    (41, 130, 128, 96, 5, 8),
    (42, 900, 192, 264, 6, 32),
    (43, 700, 136, 72, 4, 8),
])
def test_fused_b_layouts_give_identical_bits(case):
    """The fused product reads B from its d_out-major copy when the pool has
    one and gathers it from Bt otherwise: same staged values, same bits."""
    seed, n, d_in, d_out, n_slots, r_max = case
    say("b layouts", case)
    w = wl.make_random(seed, n, d_in, d_out, n_slots, r_max, p_base=0.1, dtype="bf16", runs=True)
    a = run_hip(w, separate=False, natural_b=True)
    b = run_hip(w, separate=False, natural_b=False)
    assert a.pool.B is not None and b.pool.B is None
    assert torch.equal(a.Yf, b.Yf)
    check_values(w, a)


def test_slot_relocation_and_determinism():
    w = wl.make_random(26, n=500, d_in=192, d_out=128, n_slots=12, r_max=32, dtype="bf16")
    a = run_hip(w)
    b = run_hip(w)
    assert torch.equal(a.Yf, b.Yf) and torch.equal(a.Ys, b.Ys)
    perm = np.random.default_rng(3).permutation(w.n_slots)
    c = wl.Workload(**{**w.__dict__})
    c.A = np.empty_like(w.A)
    c.Bt = np.empty_like(w.Bt)
    c.slot_rank = np.empty_like(w.slot_rank)
    for s in range(w.n_slots):
        c.A[perm[s]] = w.A[s]
        c.Bt[perm[s]] = w.Bt[s]
        c.slot_rank[perm[s]] = w.slot_rank[s]
    c.row_slot = np.where(w.row_slot < 0, -1, perm[np.maximum(w.row_slot, 0)]).astype(np.int32)
    rc = run_hip(c)
    assert torch.equal(rc.Yf, a.Yf) and torch.equal(rc.Ys, a.Ys)


def test_row_permutation_permutes_output():
    w = wl.make_random(27, n=300, d_in=128, d_out=128, n_slots=20, r_max=16, dtype="bf16")
    a = run_hip(w)
    perm = np.random.default_rng(4).permutation(w.n)
    c = wl.Workload(**{**w.__dict__})
    c.X = w.X[perm]
    c.row_slot = w.row_slot[perm]
    rc = run_hip(c)
    tp = torch.as_tensor(perm, device=DEV)
    assert torch.equal(rc.Yf, a.Yf[tp]) and torch.equal(rc.Ys, a.Ys[tp])


def test_graph_replay_matches_eager():
    """The whole step captured in a HIP graph: every replay (with eager work
    and synchronisation between replays) equals the eager result bit for bit."""
    w = wl.make_random(28, n=260, d_in=256, d_out=192, n_slots=40, r_max=16, dtype="bf16")
    eager = run_hip(w, separate=False)
    d = eager.d
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha)
    seg = srg.Segments(w.n, w.n_slots, DEV)
    H = torch.zeros((w.n, w.r_max), dtype=torch.float32, device=DEV)
    Y = torch.zeros((w.n, w.d_out), dtype=torch.bfloat16, device=DEV)
    srg.lora_build_segments(d["row_slot"], pool, seg)     # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        srg.lora_build_segments(d["row_slot"], pool, seg)
        srg.lora_shrink(d["X"], seg, pool, H)
        srg.lora_linear_fused(d["X"], d["W"], H, seg, pool, Y)
    for rep in range(4):
        Y.fill_(0)
        H.fill_(0)
        seg.token_indices.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager.Yf), rep
        assert torch.equal(seg.token_indices[:w.n].cpu(),
                           torch.as_tensor(eager.meta["token_indices"])), rep
        _ = (Y.float() * 2).sum().item()                   # eager work between replays


def test_two_stream_step_in_graph_matches_eager():
    """Base GEMM on a second stream beside build + shrink, joined before the
    expand, captured in one HIP graph: every replay equals the eager
    separate path bit for bit."""
    w = wl.make_random(29, n=256, d_in=512, d_out=384, n_slots=50, r_max=16, dtype="bf16")
    eager = run_hip(w, fused=False)
    d = eager.d
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha)
    seg = srg.Segments(w.n, w.n_slots, DEV)
    H = torch.zeros((w.n, w.r_max), dtype=torch.float32, device=DEV)
    Y = torch.zeros((w.n, w.d_out), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    def step():
        main = torch.cuda.current_stream()
        fork.record(main)
        side.wait_event(fork)
        with torch.cuda.stream(side):
            srg.lora_base_gemm(d["X"], d["W"], Y)
        join.record(side)
        srg.lora_build_segments(d["row_slot"], pool, seg)
        srg.lora_shrink(d["X"], seg, pool, H)
        main.wait_event(join)
        srg.lora_expand(H, seg, pool, Y)

    step()
    torch.cuda.synchronize()
    assert torch.equal(Y, eager.Ys)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        Y.fill_(0)
        H.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, eager.Ys), rep
        _ = (Y.float() + 1).sum().item()


# ---------------------------------------------------------------- adapter packing
def _run_with_pool(w, pool):
    """Every entry point on workload w's X, W and mapping, with a given pool."""
    d = wl.device_tensors(w, DEV)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    seg = srg.Segments(w.n, w.n_slots, DEV)
    srg.lora_build_segments(d["row_slot"], pool, seg)
    H = torch.full((w.n, w.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_shrink(d["X"], seg, pool, H)
    Yf = torch.empty((w.n, w.d_out), dtype=dt, device=DEV)
    srg.lora_linear_fused(d["X"], d["W"], H, seg, pool, Yf)
    Ys = torch.empty((w.n, w.d_out), dtype=dt, device=DEV)
    srg.lora_base_gemm(d["X"], d["W"], Ys)
    srg.lora_expand(H, seg, pool, Ys)
    torch.cuda.synchronize()
    return Yf, Ys


def _adapter(w, a):
    """Slot a's adapter in its own layouts: A [r, d_in], B [d_out, r] (bit patterns)."""
    r = int(w.slot_rank[a])
    return w.A[a, :r].copy(), w.B[a, :, :r].copy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_slots_layout_and_parity(dtype):
    """Adapters packed one by one into an empty pool give exactly the pool
    layout (zeros past the rank) and the oracle's outputs; repacking a slot
    switches the adapter; rank 0 empties it."""
    ranks = [8, 32, 5, 16, 1, 24]
    w = wl.make_random(60, n=200, d_in=136, d_out=72, n_slots=6, r_max=32, ranks=ranks,
                       p_base=0.1, dtype=dtype, pad="zero")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pool = srg.Pool.empty(6, 32, 136, 72, dtype=tdt, device=DEV)
    for a in range(6):
        Ah, Bh = _adapter(w, a)
        At = wl.to_torch(Ah, dtype, "cpu" if a % 2 else DEV)   # host and device sources
        Bt_ = wl.to_torch(Bh, dtype, "cpu" if a % 2 else DEV)
        assert pool.pack(a, At, Bt_, float(w.slot_alpha[a])) == 1
    torch.cuda.synchronize()
    ref = wl.device_tensors(w, DEV)
    assert torch.equal(pool.A, ref["A"])
    assert torch.equal(pool.Bt, ref["Bt"])
    assert torch.equal(pool.B, ref["Bt"].transpose(1, 2).contiguous())
    assert torch.equal(pool.slot_rank.cpu(), torch.tensor(ranks, dtype=torch.int32))
    exp_scale = torch.tensor([float(w.slot_alpha[a]) / r for a, r in enumerate(ranks)],
                             dtype=torch.float64).to(torch.float32)
    assert torch.equal(pool.slot_scale.cpu(), exp_scale)
    tol = TOL[dtype]
    Yr, _, _ = oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                   w.r_max, w.dtype)
    Yf, Ys = _run_with_pool(w, pool)
    assert normwise(to_f64(Yf), Yr) <= tol and normwise(to_f64(Ys), Yr) <= tol

    # repack slot 1 with slot 3's adapter (rank 16) and empty slot 2
    A3, B3 = _adapter(w, 3)
    assert pool.pack(1, wl.to_torch(A3, dtype, DEV), wl.to_torch(B3, dtype, DEV),
                     float(w.slot_alpha[3])) == 2
    empty_A = torch.zeros((0, 136), dtype=tdt)
    empty_B = torch.zeros((72, 0), dtype=tdt)
    assert pool.pack(2, empty_A, empty_B, 16.0) == 2
    torch.cuda.synchronize()
    w2 = copy.deepcopy(w)
    w2.A[1] = w.A[3]
    w2.Bt[1] = w.Bt[3]
    w2.slot_rank[1] = 16
    w2.A[2] = 0
    w2.Bt[2] = 0
    w2.slot_rank[2] = 0
    ref2 = wl.device_tensors(w2, DEV)
    assert torch.equal(pool.A, ref2["A"]) and torch.equal(pool.Bt, ref2["Bt"])
    assert int(pool.slot_rank[2]) == 0 and float(pool.slot_scale[2]) == 0.0
    Yr2, _, _ = oracle.lora_forward(w2.X, w2.W, w2.A, w2.B, w2.row_slot, w2.slot_rank,
                                    w2.slot_alpha, w2.r_max, w2.dtype)
    Yf2, Ys2 = _run_with_pool(w2, pool)
    assert normwise(to_f64(Yf2), Yr2) <= tol and normwise(to_f64(Ys2), Yr2) <= tol
    # rows of the emptied slot now equal the plain product
    rows = torch.as_tensor(np.nonzero(w.row_slot == 2)[0], device=DEV)
    Yb = torch.empty_like(Ys2)
    srg.lora_base_gemm(wl.to_torch(w.X, dtype, DEV), wl.to_torch(w.W, dtype, DEV), Yb)
    torch.cuda.synchronize()
    assert torch.equal(Ys2[rows], Yb[rows]) and torch.equal(Yf2[rows], Yb[rows])
