"""Pins of the CPU oracle against what the pages and the mathematics fix.

No GPU and no HIP library here.  Each test names the fact it checks; chosen
so that a plausible oracle mistake (dropped term, wrong sign, wrong scale,
wrong or transposed operand, wrong row mapping, unstable grouping) fails at
least one of them.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _fwd(w, **kw):
    return oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                               w.r_max, w.dtype, **kw)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- metadata
def test_printed_metadata_example():
    """The page's printed segment_offsets / adapter_slots / ranks / scales."""
    g = _load("metadata_printed_example.json")
    m = oracle.segment_metadata(g["row_slot"], g["slot_rank"], g["slot_alpha"], g["r_max"])
    e = g["expected"]
    assert m["num_segments"] == e["num_segments"]
    for k in ("segment_offsets", "segment_slots", "segment_ranks", "token_indices"):
        assert m[k].tolist() == e[k], k
    assert m["segment_scales"].tolist() == e["segment_scales"]
    assert m["status"] == 0


def test_tiny_f32_offsets():
    """The tiny fp32 case's offsets [0, 8, 12, 28, 32] -> {A r8, base, B r16, C r8}."""
    w = wl.make_workload("tiny_f32")
    m = oracle.segment_metadata(w.row_slot, w.slot_rank, w.slot_alpha, w.r_max)
    assert m["segment_offsets"].tolist() == [0, 8, 12, 28, 32]
    assert m["segment_slots"].tolist() == [0, -1, 1, 2]
    assert m["segment_ranks"].tolist() == [8, 0, 16, 8]
    assert m["segment_scales"].tolist() == [2.0, 0.0, 1.0, 2.0]
    assert m["token_indices"].tolist() == list(range(32))


def _brute_force_metadata(row_slot, slot_rank, r_max):
    """Stable sort by (first-appearance index of the key, row) using sorted()."""
    keys, bad = oracle.validate_rows(row_slot, slot_rank, r_max)
    first = {}
    for i, k in enumerate(keys):
        first.setdefault(k, i)
    perm = sorted(range(len(keys)), key=lambda i: (first[keys[i]], i))
    return keys, perm, bad


@pytest.mark.parametrize("seed", range(12))
def test_metadata_fuzz_against_sort(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 300))
    n_slots = int(rng.integers(1, 40))
    r_max = 64
    slot_rank = rng.choice([0, 8, 16, 32, 64, 65, -1], size=n_slots,
                           p=[0.05, 0.3, 0.3, 0.15, 0.1, 0.05, 0.05])
    row_slot = rng.integers(-2, n_slots + 2, size=n)
    if seed % 3 == 0:                      # long runs, prefill-like
        row_slot = np.repeat(rng.integers(-1, n_slots, size=max(1, n // 50 + 1)), 50)[:n]
    m = oracle.segment_metadata(row_slot, slot_rank, np.full(n_slots, 16.0), r_max)
    keys, perm, bad = _brute_force_metadata(row_slot, slot_rank, r_max)
    ti = m["token_indices"]
    assert ti.tolist() == perm
    assert sorted(ti.tolist()) == list(range(n))            # permutation
    off = m["segment_offsets"]
    S = int(m["num_segments"])
    assert S == len(set(keys))
    assert off[0] == 0 and off[-1] == n and np.all(np.diff(off) > 0)
    for s in range(S):
        ks = {keys[i] for i in ti[off[s]:off[s + 1]]}
        assert ks == {int(m["segment_slots"][s])}
        assert all(m["row_segment"][i] == s for i in ti[off[s]:off[s + 1]])
    assert m["status"] == bad


def test_invalid_rows_become_base_and_are_counted():
    slot_rank = [8, 80, 16]                 # slot 1 rank exceeds r_max 64
    row_slot = [0, 5, 1, -1, -7, 2, 0]
    m = oracle.segment_metadata(row_slot, slot_rank, [16.0] * 3, 64)
    assert m["status"] == 3                 # rows 1, 2, 4
    assert m["segment_slots"].tolist() == [0, -1, 2]
    assert m["token_indices"].tolist() == [0, 6, 1, 2, 3, 4, 5]
    assert m["segment_offsets"].tolist() == [0, 2, 6, 7]


# ---------------------------------------------------------------- layer values
def test_hand_worked_example():
    g = _load("hand_worked_3x2.json")
    r_max = g["r_max"]
    A = np.array(g["A"], dtype=np.float32)
    B = np.array(g["B"], dtype=np.float32)
    Y, dY, H = oracle.lora_forward(np.array(g["X"], np.float32), np.array(g["W"], np.float32), A, B,
                                   g["row_slot"], g["slot_rank"], g["slot_alpha"], r_max, "f32")
    e = g["expected"]
    assert Y.tolist() == e["Y"]
    assert dY.tolist() == e["dY"]
    assert H.tolist() == e["H"]
    m = oracle.segment_metadata(g["row_slot"], g["slot_rank"], g["slot_alpha"], r_max)
    for k in ("segment_offsets", "segment_slots", "segment_ranks"):
        assert m[k].tolist() == e[k]
    assert m["segment_scales"].tolist() == e["segment_scales"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_merged_closed_form(dtype):
    """X (W + s_a B_a A_a)^T equals the two-stage form (adapter-batching page,
    '为什么单 Adapter 可以 Merge').  The merged weight is formed here, in the
    test, independently of the oracle's row loop."""
    w = wl.make_random(7, n=40, d_in=96, d_out=72, n_slots=5, r_max=16, dtype=dtype, p_base=0.2,
                       w_std=0.3, ab_std=0.3)
    Y, dY, H = _fwd(w)
    X = oracle.decode(w.X, dtype)
    W = oracle.decode(w.W, dtype)
    ref = np.empty_like(Y)
    for i in range(w.n):
        a = int(w.row_slot[i])
        Wm = W.copy()
        if a >= 0 and w.slot_rank[a] > 0:
            r = int(w.slot_rank[a])
            Aa = oracle.decode(w.A[a, :r], dtype)
            Ba = oracle.decode(w.B[a, :, :r], dtype)
            Wm += (w.slot_alpha[a] / r) * np.einsum("jk,kc->jc", Ba, Aa)
        ref[i] = np.einsum("jc,c->j", Wm, X[i])
    assert _rel(Y, ref) < 1e-12
    Ym = oracle.merged_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                               w.r_max, dtype)
    assert _rel(Ym, ref) < 1e-12


def test_base_only_rows_equal_plain_linear():
    """All rows base-only: the layer is X W^T exactly (the page's metadata
    gives base rows rank 0 and scale 0)."""
    w = wl.make_random(3, n=20, d_in=64, d_out=48, n_slots=3, r_max=8, p_base=1.0, dtype="bf16")
    Y, dY, H = _fwd(w)
    X = oracle.decode(w.X, "bf16")
    W = oracle.decode(w.W, "bf16")
    assert np.array_equal(Y, X @ W.T)
    assert not dY.any() and not H.any()


def test_rank_zero_slot_is_plain_linear():
    w = wl.make_random(4, n=30, d_in=32, d_out=40, n_slots=3, r_max=16, ranks=[0, 8, 0],
                       p_base=0.0, dtype="f32")
    Y, dY, H = _fwd(w)
    X = oracle.decode(w.X, "f32")
    W = oracle.decode(w.W, "f32")
    base = X @ W.T
    for i in range(w.n):
        if w.row_slot[i] != 1:
            assert np.array_equal(Y[i], base[i])
            assert not dY[i].any()
        else:
            assert dY[i].any()


def test_integer_case_exact_fractions():
    """Small integers: every value of the method is exact, so the oracle must
    equal a brute-force rational evaluation of each output element."""
    ranks = [2, 1, 3]
    row_slot = [0, 2, -1, 1, 0, 2, 2]
    w = wl.make_integer_case(11, n=7, d_in=5, d_out=4, n_slots=3, r_max=4, ranks=ranks,
                             row_slot=row_slot)
    Y, dY, H = _fwd(w)
    X = w.X.astype(int).tolist()
    W = w.W.astype(int).tolist()
    for i in range(w.n):
        a = row_slot[i]
        for j in range(w.d_out):
            y = sum(Fraction(W[j][c]) * X[i][c] for c in range(w.d_in))
            if a >= 0:
                r = ranks[a]
                s = Fraction(int(w.slot_alpha[a])) / r
                for k in range(r):
                    hk = sum(Fraction(int(w.A[a, k, c])) * X[i][c] for c in range(w.d_in))
                    y += s * int(w.Bt[a, k, j]) * hk
            assert Fraction(Y[i, j]) == y


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fingerprint_adapters(dtype):
    """A_a = e_(a mod d_in) in row 0, B_a = a + 1 everywhere: the increment of
    a row on slot a is s_a (a + 1) x[a mod d_in] in every column."""
    w = wl.make_fingerprint(5, n=64, d_in=48, d_out=24, n_slots=20, r_max=32, dtype=dtype)
    Y, dY, H = _fwd(w)
    X = oracle.decode(w.X, dtype)
    for i in range(w.n):
        a = int(w.row_slot[i])
        if a < 0:
            assert not dY[i].any()
            continue
        s = 16.0 / int(w.slot_rank[a])
        exp = s * (a + 1) * X[i, a % w.d_in]
        assert np.all(dY[i] == exp), (i, a)


def test_cross_formulations_agree():
    w = wl.make_random(9, n=80, d_in=64, d_out=56, n_slots=9, r_max=32, p_base=0.15, dtype="bf16")
    Y, dY, H = _fwd(w)
    args = (w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha, w.r_max, w.dtype)
    Yg, dYg, Hg = oracle.gather_bmm_forward(*args)
    Yp, dYp = oracle.per_adapter_forward(*args)
    assert _rel(Yg, Y) < 1e-12 and _rel(dYg, dY) < 1e-12
    assert _rel(Hg, H) < 1e-12
    assert _rel(Yp, Y) < 1e-12 and _rel(dYp, dY) < 1e-12


# ---------------------------------------------------------------- invariants
def _subset(w, rows, row_slot=None):
    c = wl.Workload(**{**w.__dict__})
    c.X = w.X[rows]
    c.n = len(rows)
    c.row_slot = (w.row_slot if row_slot is None else row_slot)[rows]
    return c


def test_row_permutation_permutes_output():
    w = wl.make_random(12, n=50, d_in=40, d_out=32, n_slots=6, r_max=16, dtype="bf16")
    Y, dY, H = _fwd(w)
    perm = np.random.default_rng(0).permutation(w.n)
    Yp, dYp, Hp = _fwd(_subset(w, perm))
    assert _rel(Yp, Y[perm]) < 1e-13
    assert np.array_equal(dYp, dY[perm]) and np.array_equal(Hp, H[perm])


def test_batch_equals_rows_one_at_a_time():
    """A mixed batch gives each row what it gets alone (adapter-batching page,
    '正确性测试怎样做', items 4 and 5)."""
    w = wl.make_random(13, n=24, d_in=40, d_out=32, n_slots=4, r_max=16, dtype="bf16")
    Y, dY, H = _fwd(w)
    for i in range(w.n):
        Yi, dYi, Hi = _fwd(_subset(w, [i]))
        assert _rel(Yi[0], Y[i]) < 1e-13
        assert np.array_equal(dYi[0], dY[i]) and np.array_equal(Hi[0], H[i])


def test_slot_relocation_leaves_output_unchanged():
    """Moving adapters to other slots (eviction + reload elsewhere) and
    remapping rows gives the same layer output."""
    w = wl.make_random(14, n=60, d_in=32, d_out=24, n_slots=7, r_max=16, dtype="bf16")
    Y, dY, H = _fwd(w)
    perm = np.random.default_rng(1).permutation(w.n_slots)      # old slot a -> new slot perm[a]
    c = wl.Workload(**{**w.__dict__})
    c.A = np.empty_like(w.A)
    c.Bt = np.empty_like(w.Bt)
    c.slot_rank = np.empty_like(w.slot_rank)
    c.slot_alpha = np.empty_like(w.slot_alpha)
    for a in range(w.n_slots):
        c.A[perm[a]] = w.A[a]
        c.Bt[perm[a]] = w.Bt[a]
        c.slot_rank[perm[a]] = w.slot_rank[a]
        c.slot_alpha[perm[a]] = w.slot_alpha[a]
    c.row_slot = np.where(w.row_slot < 0, -1, perm[np.maximum(w.row_slot, 0)]).astype(np.int32)
    Yc, dYc, Hc = _fwd(c)
    assert np.array_equal(Yc, Y) and np.array_equal(dYc, dY) and np.array_equal(Hc, H)


def test_segment_order_does_not_change_rows():
    """Reordering which key appears first changes the segment order only;
    every row's output and its metadata row group are unchanged."""
    w = wl.make_random(15, n=40, d_in=24, d_out=16, n_slots=5, r_max=8, dtype="f32", runs=True)
    Y, _, _ = _fwd(w)
    m = oracle.segment_metadata(w.row_slot, w.slot_rank, w.slot_alpha, w.r_max)
    rev = np.arange(w.n)[::-1].copy()
    c = _subset(w, rev)
    Yc, _, _ = _fwd(c)
    mc = oracle.segment_metadata(c.row_slot, c.slot_rank, c.slot_alpha, c.r_max)
    assert np.array_equal(Yc, Y[rev]) or _rel(Yc, Y[rev]) < 1e-13
    groups = {int(m["segment_slots"][s]): sorted(m["token_indices"][m["segment_offsets"][s]:m["segment_offsets"][s + 1]].tolist())
              for s in range(int(m["num_segments"]))}
    groups_c = {int(mc["segment_slots"][s]): sorted(rev[mc["token_indices"][mc["segment_offsets"][s]:mc["segment_offsets"][s + 1]]].tolist())
                for s in range(int(mc["num_segments"]))}
    assert groups == groups_c


def test_padding_is_never_read():
    """Pool padding holds NaN; a finite result means it was not read."""
    w = wl.make_random(16, n=50, d_in=32, d_out=24, n_slots=6, r_max=64, dtype="bf16")
    assert np.isnan(oracle.decode(w.A, "bf16")).any()
    Y, dY, H = _fwd(w)
    assert np.isfinite(Y).all() and np.isfinite(H).all()


# ---------------------------------------------------------------- arithmetic on the pages
def test_parameter_arithmetic_printed():
    # S-LoRA 深度解析, 1.1: 4096 x 4096, r = 8 -> about 65.5 thousand params, 256x fewer
    assert oracle.lora_param_count(8, 4096, 4096) == 65536
    assert oracle.full_param_count(4096, 4096) // oracle.lora_param_count(8, 4096, 4096) == 256
    # S-LoRA 深度解析, 4.1: r = 16 on Q/K/V/O of width 4096 -> 524,288 params a layer,
    # 80 layers in 2-byte storage is about 80 MB (80 MiB exactly)
    per_layer = 4 * oracle.lora_param_count(16, 4096, 4096)
    assert per_layer == 524288
    assert 80 * per_layer * 2 == 80 * 2 ** 20


def test_workload_configs_shapes():
    w1 = wl.make_workload("tiny_f32")
    assert (w1.n, w1.d_in, w1.d_out, w1.dtype) == (32, 512, 512, "f32")
    w2 = wl.make_workload("decode")
    assert (w2.n, w2.d_in, w2.d_out, w2.n_slots, w2.r_max) == (256, 4096, 4096, 128, 16)
    frac_base = np.mean(w2.row_slot < 0)
    assert 0.03 < frac_base < 0.2
    row_slot, ranks, _ = wl.layer70b_mapping()
    assert len(row_slot) == 2304 and len(set(row_slot[:2048].tolist())) == 1
    assert ranks.tolist() == [16] * 32 + [64] * 32
