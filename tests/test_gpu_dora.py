"""GPU parity of the DoRA epilogue (ybb.press multi-LoRA serving article,
section 9.2): the column factors from lora_pool_dora_prepare against the
oracle's g_a = m_a / ||W0 + s_a B_a A_a||_c, and the fused and separate
forward paths against the oracle's DoRA layer, with the same normwise
tolerances as the plain layer (1e-2 bf16 storage, 1e-5 fp32).  Factors are
fp32 sums of squares, compared elementwise within 2e-5 relative.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_segment_amd as srg
import workloads as wl
from gpu_harness import DEV, TOL, normwise, sample_rows, say, to_f64

pytestmark = pytest.mark.gpu

G_RTOL = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    srg.lib()
    yield
    torch.cuda.synchronize()


def _magnitudes(w, seed, p_plain=0.25, plain_slots=None):
    return wl.make_magnitude(seed, w.n_slots, w.d_out, 0.02 * math.sqrt(w.d_in), p_plain=p_plain,
                             plain_slots=plain_slots)


def _dora_pool(w, d, mag, policy="exact", natural_b=True):
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, policy, natural_b=natural_b,
                    dora=True)
    for a in range(w.n_slots):
        if mag[a] is not None:
            pool.dora_prepare(a, d["W"], torch.from_numpy(mag[a]).to(DEV))
    return pool


def _forward(w, d, pool, fused=True, separate=True):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    seg = srg.Segments(w.n, w.n_slots, DEV)
    srg.lora_build_segments(d["row_slot"], pool, seg)
    H = torch.full((w.n, w.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_shrink(d["X"], seg, pool, H)
    out = {}
    if fused:
        Yf = torch.empty((w.n, w.d_out), dtype=dt, device=DEV)
        srg.lora_linear_fused(d["X"], d["W"], H, seg, pool, Yf)
        out["fused"] = Yf
    if separate:
        Ys = torch.empty((w.n, w.d_out), dtype=dt, device=DEV)
        srg.lora_base_gemm(d["X"], d["W"], Ys)
        out["base"] = Ys.clone()
        srg.lora_expand(H, seg, pool, Ys)
        out["separate"] = Ys
    torch.cuda.synchronize()
    return out


def _check(w, out, mag, rows=None, tol=None):
    tol = TOL[w.dtype] if tol is None else tol
    if rows is None:
        ref = oracle.dora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha, mag,
                                  w.r_max, w.dtype)
        idx = np.arange(w.n)
    else:
        ref = oracle.dora_factored_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank,
                                           w.slot_alpha, mag, w.r_max, w.dtype, rows=rows)
        idx = np.asarray(rows)
    ti = torch.as_tensor(idx, device=DEV, dtype=torch.long)
    errs = {}
    for k in ("fused", "separate"):
        if k in out:
            errs[k] = normwise(to_f64(out[k][ti]), ref)
            assert errs[k] <= tol, (k, errs[k], tol)
    return errs


def _unscaled_rows(w):
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    return np.array([k < 0 or int(w.slot_rank[k]) == 0 for k in keys], dtype=bool)


def _base_rows_untouched(w, out):
    rows = np.nonzero(_unscaled_rows(w))[0]
    if len(rows) == 0 or "base" not in out:
        return 0
    ti = torch.as_tensor(rows, device=DEV)
    assert torch.equal(out["separate"][ti], out["base"][ti])
    if "fused" in out:
        assert torch.equal(out["fused"][ti], out["base"][ti])
    return len(rows)


# ---------------------------------------------------------------- the column factors
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prepare_matches_oracle(dtype):
    """g for every slot (ranks 0..64, one slot without a magnitude), with a
    ragged input width and an output feature whose direction row is zero."""
    ranks = [8, 64, 0, 16, 32, 5, 64]
    w = wl.make_random(301, n=16, d_in=520, d_out=264, n_slots=7, r_max=64, ranks=ranks,
                       p_base=0.1, dtype=dtype)
    w.W[5, :] = 0                       # with B_a row 5 zero: V_a row 5 = 0, so g = 0
    w.Bt[:, :, 5] = 0
    mag = _magnitudes(w, 301, p_plain=0.0, plain_slots=[3])
    d = wl.device_tensors(w, DEV)
    pool = _dora_pool(w, d, mag)
    torch.cuda.synchronize()
    g = pool.dora_scale.cpu().numpy().astype(np.float64)
    for a in range(w.n_slots):
        ref = oracle.dora_column_scale(w.W, w.A, w.B, w.slot_rank, w.slot_alpha, mag, w.dtype, a)
        if mag[a] is None:
            assert np.array_equal(g[a], np.ones(w.d_out)), a
            continue
        assert g[a][5] == 0.0 and ref[5] == 0.0
        np.testing.assert_allclose(g[a], ref, rtol=G_RTOL, atol=0, err_msg=f"slot {a}")


# ---------------------------------------------------------------- forward parity
DCASES = [
    # seed, n, d_in, d_out, n_slots, r_max, p_base, dtype, runs
    (311, 1, 64, 72, 3, 8, 0.0, "bf16", False),
    (312, 300, 520, 264, 40, 64, 0.1, "bf16", False),
    (313, 333, 256, 384, 6, 32, 0.2, "bf16", True),
    (314, 700, 200, 136, 7, 64, 0.1, "bf16", True),      # large tiles, K tail
    (315, 2100, 328, 264, 5, 32, 0.2, "bf16", True),
    (316, 70, 64, 64, 4, 64, 0.1, "f32", True),
    (317, 513, 200, 120, 17, 32, 0.1, "f32", False),
    (318, 400, 136, 4104, 9, 32, 0.1, "bf16", True),     # two-stage small tiles
]


@pytest.mark.parametrize("case", DCASES, ids=[f"s{c[0]}" for c in DCASES])
@pytest.mark.parametrize("policy", ["exact", "padded"])
def test_dora_forward_cases(case, policy):
    seed, n, d_in, d_out, n_slots, r_max, p_base, dtype, runs = case
    say("dora", case, policy)
    w = wl.make_random(seed, n, d_in, d_out, n_slots, r_max, p_base=p_base, dtype=dtype, runs=runs)
    if n_slots > 2:
        w.slot_rank[1] = 0              # a rank-0 slot: its rows are never rescaled
    mag = _magnitudes(w, seed)
    d = wl.device_tensors(w, DEV)
    out = _forward(w, d, _dora_pool(w, d, mag, policy))
    e = _check(w, out, mag)
    _base_rows_untouched(w, out)
    say("dora errors", e)


@pytest.mark.parametrize("natural_b", [True, False])
def test_dora_both_b_layouts(natural_b):
    w = wl.make_random(320, 600, 264, 520, 9, 32, p_base=0.1, dtype="bf16", runs=True)
    mag = _magnitudes(w, 320)
    d = wl.device_tensors(w, DEV)
    out = _forward(w, d, _dora_pool(w, d, mag, natural_b=natural_b), separate=False)
    _check(w, out, mag)


def test_unit_factors_give_plain_lora_bits():
    """A DoRA pool whose factors are all ones (fresh, or prepared without a
    magnitude) returns exactly the plain pool's bits."""
    w = wl.make_random(321, 700, 200, 136, 7, 64, p_base=0.1, dtype="bf16", runs=True)
    d = wl.device_tensors(w, DEV)
    plain = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha)
    fresh = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, dora=True)
    prepared = _dora_pool(w, d, [None] * w.n_slots)
    for a in range(w.n_slots):
        prepared.dora_prepare(a, d["W"], None)
    ref = _forward(w, d, plain)
    for pool in (fresh, prepared):
        out = _forward(w, d, pool)
        assert torch.equal(out["fused"], ref["fused"])
        assert torch.equal(out["separate"], ref["separate"])


def test_pack_resets_factors_to_plain():
    """Packing into a DoRA pool writes ones into the slot's factors before
    publishing it; prepare then turns it into a DoRA adapter."""
    ranks = [16, 8, 32]
    w = wl.make_random(322, n=150, d_in=136, d_out=72, n_slots=3, r_max=32, ranks=ranks,
                       p_base=0.1, dtype="bf16", pad="zero")
    pool = srg.Pool.empty(3, 32, 136, 72, dtype=torch.bfloat16, device=DEV, dora=True)
    d = wl.device_tensors(w, DEV)
    for a in range(3):
        r = ranks[a]
        pool.pack(a, wl.to_torch(w.A[a, :r].copy(), "bf16", DEV),
                  wl.to_torch(w.B[a, :, :r].copy(), "bf16", DEV), float(w.slot_alpha[a]))
    mag = _magnitudes(w, 322, p_plain=0.0)
    for a in range(3):
        pool.dora_prepare(a, d["W"], torch.from_numpy(mag[a]).to(DEV))
    torch.cuda.synchronize()
    assert not torch.equal(pool.dora_scale[1], torch.ones(72, device=DEV))
    _check(w, _forward(w, d, pool), mag)
    # repack slot 1 with the same adapter: plain LoRA again until prepared
    pool.pack(1, wl.to_torch(w.A[1, :8].copy(), "bf16", DEV),
              wl.to_torch(w.B[1, :, :8].copy(), "bf16", DEV), float(w.slot_alpha[1]))
    torch.cuda.synchronize()
    assert torch.equal(pool.dora_scale[1], torch.ones(72, device=DEV))
    mag2 = list(mag)
    mag2[1] = None
    _check(w, _forward(w, d, pool), mag2)


def test_empty_batch_with_dora_pool():
    w = wl.make_random(323, 0, 64, 72, 3, 8, dtype="bf16")
    d = wl.device_tensors(w, DEV)
    pool = _dora_pool(w, d, _magnitudes(w, 323))
    seg = srg.Segments(0, 3, DEV)
    srg.lora_build_segments(d["row_slot"], pool, seg)
    H = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    Y = torch.empty((0, 72), dtype=torch.bfloat16, device=DEV)
    srg.lora_expand(H, seg, pool, Y)
    srg.lora_linear_fused(d["X"], d["W"], H, seg, pool, Y)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- full-size workloads
def test_dora_decode_full():
    """Decode workload (d 4096, 256 rows, 128 rank-16 slots), every row."""
    w = wl.make_workload("decode")
    mag = _magnitudes(w, 2)
    d = wl.device_tensors(w, DEV)
    out = _forward(w, d, _dora_pool(w, d, mag))
    rows = list(range(w.n))
    e = _check(w, out, mag, rows=rows)
    assert _base_rows_untouched(w, out) > 0
    say("dora decode errors", e)


def test_dora_prefill_sampled():
    """Prefill workload (d 4096 -> 14336, eight requests, ranks 8..64, one
    base-only request) on the large-tile fused kernel, sampled rows."""
    w = wl.make_workload("prefill")
    mag = _magnitudes(w, 3, p_plain=0.0)
    d = wl.device_tensors(w, DEV)
    out = _forward(w, d, _dora_pool(w, d, mag), separate=False)
    ref_meta = oracle.segment_metadata(w.row_slot, w.slot_rank, w.slot_alpha, w.r_max)
    rows = sample_rows(w, ref_meta, 256)
    e = _check(w, out, mag, rows=rows)
    assert torch.isfinite(out["fused"].float()).all()
    say("dora prefill errors", len(rows), e)
