"""Pins of the DoRA part of the oracle (ybb.press multi-LoRA serving article,
section 9.2: W' = m (W0 + BA) / ||W0 + BA||_c).

Each pin is a fact fixed by the page, the mathematics or a library routine,
not the oracle's formula typed again: a hand-worked fixture, DoRA's own
initialisation property (m = ||W0||_c and B = 0 give the base layer), scale
invariance of the direction, homogeneity in m, reductions to the plain layer,
a brute-force loop on tiny integer inputs, and planted mistakes that must
fail the fixture.
"""
import inspect
import json
import math
import os
import textwrap

import numpy as np
import pytest

import oracle
import oracle.lora_oracle as lo
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _fixture(dtype):
    with open(os.path.join(GOLD, "dora_hand_worked.json")) as f:
        g = json.load(f)
    enc = (lambda a: wl.bf16_bits_rne(np.asarray(a, np.float32))) if dtype == "bf16" else \
        (lambda a: np.asarray(a, np.float32))
    mag = [None if m is None else np.asarray(m, np.float32) for m in g["magnitude"]]
    args = (enc(g["X"]), enc(g["W"]), enc(g["A"]), enc(g["B"]), g["row_slot"], g["slot_rank"],
            g["slot_alpha"], mag, g["r_max"], dtype)
    return g, args


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fwd", [oracle.dora_forward, oracle.dora_factored_forward])
def test_hand_worked_fixture(fwd, dtype):
    g, args = _fixture(dtype)
    assert fwd(*args).tolist() == g["expected"]["Y"]


def test_hand_worked_column_scales():
    g, args = _fixture("f32")
    X, W, A, B, row_slot, slot_rank, slot_alpha, mag, r_max, dtype = args
    for a, exp in enumerate(g["expected"]["g"]):
        if exp is None:
            continue
        got = oracle.dora_column_scale(W, A, B, slot_rank, slot_alpha, mag, dtype, a)
        assert got.tolist() == exp, a


def _random(seed, n=48, d_in=64, d_out=40, n_slots=6, r_max=16, dtype="bf16", p_plain=0.3):
    w = wl.make_random(seed, n, d_in, d_out, n_slots, r_max, p_base=0.15, dtype=dtype)
    mag = wl.make_magnitude(seed, n_slots, d_out, 0.02 * math.sqrt(d_in), p_plain=p_plain)
    return w, mag


def _dora(w, mag, fwd=oracle.dora_forward, rows=None):
    return fwd(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha, mag, w.r_max, w.dtype,
               rows=rows)


def test_initialisation_gives_the_base_layer():
    """DoRA starts from m = ||W0||_c with the LoRA up-projection B = 0, so the
    adapted layer equals the base layer; the norm here is numpy's."""
    w, _ = _random(1, dtype="f32")
    w.Bt[:] = 0.0
    W64 = oracle.decode(w.W, "f32")
    m0 = np.linalg.norm(W64, axis=1)
    mag = [m0 for _ in range(w.n_slots)]
    Y = _dora(w, mag)
    np.testing.assert_allclose(Y, oracle.decode(w.X, "f32") @ W64.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("c", [0.25, 4.0])   # exact in float32
def test_direction_is_scale_invariant(c):
    """W0 -> c W0 and B -> c B scale the direction by c > 0: DoRA rows do not
    change; base-only rows scale by c; plain LoRA rows scale by c."""
    w, mag = _random(2, dtype="f32")
    Y = _dora(w, mag)
    w2, _ = _random(2, dtype="f32")
    w2.W = (w2.W * np.float32(c)).astype(np.float32)
    w2.Bt = (w2.Bt * np.float32(c)).astype(np.float32)
    Y2 = _dora(w2, mag)
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    for i, a in enumerate(keys):
        dora_row = a >= 0 and int(w.slot_rank[a]) > 0 and mag[a] is not None
        exp = Y[i] if dora_row else c * Y[i]
        np.testing.assert_allclose(Y2[i], exp, rtol=1e-9, atol=1e-12)


def test_output_is_linear_in_the_magnitude():
    w, mag = _random(3, p_plain=0.0)
    Y = _dora(w, mag)
    scaled = [None if m is None else (2.0 * m).astype(np.float32) for m in mag]
    Y2 = _dora(w, scaled)
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    for i, a in enumerate(keys):
        f = 2.0 if a >= 0 and int(w.slot_rank[a]) > 0 else 1.0
        np.testing.assert_allclose(Y2[i], f * Y[i], rtol=1e-12, atol=1e-15)


def test_plain_slots_and_base_rows_match_the_plain_layer():
    w, _ = _random(4)
    none = [None] * w.n_slots
    Y = _dora(w, none)
    Yl, _, _ = oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                   w.r_max, w.dtype)
    np.testing.assert_allclose(Y, Yl, rtol=1e-12, atol=1e-12)
    # with magnitudes everywhere, base-only rows still equal X W^T exactly
    w, mag = _random(4, p_plain=0.0)
    Y = _dora(w, mag)
    base = np.asarray(w.row_slot) < 0
    ref = oracle.decode(w.X, w.dtype)[base] @ oracle.decode(w.W, w.dtype).T
    np.testing.assert_array_equal(Y[base], ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("seed", [5, 6])
def test_factored_form_equals_definition(seed, dtype):
    """The epilogue order (plain output, then a per-column factor) gives the
    definition's result for every row."""
    w, mag = _random(seed, n=64, d_in=96, d_out=72, n_slots=8, r_max=32, dtype=dtype)
    w.slot_rank[1] = 0
    np.testing.assert_allclose(_dora(w, mag, oracle.dora_factored_forward), _dora(w, mag),
                               rtol=1e-11, atol=1e-13)


def test_row_subset_and_permutation():
    w, mag = _random(7)
    Y = _dora(w, mag)
    rows = [5, 0, 17, 17, 3]
    # (a matrix product over fewer rows may sum in another order: 1e-13)
    np.testing.assert_allclose(_dora(w, mag, rows=rows), Y[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(_dora(w, mag, oracle.dora_factored_forward, rows=rows),
                               _dora(w, mag, oracle.dora_factored_forward)[rows],
                               rtol=1e-13, atol=1e-15)


def test_brute_force_tiny_integers():
    """Every step as a Python loop over scalars (math.sqrt), on small
    integer inputs."""
    rng = np.random.default_rng(11)
    n, d_in, d_out, n_slots, r_max = 7, 5, 4, 3, 8
    ranks = [2, 0, 3]
    X = rng.integers(-3, 4, size=(n, d_in)).astype(np.float32)
    W = rng.integers(-3, 4, size=(d_out, d_in)).astype(np.float32)
    A = rng.integers(-2, 3, size=(n_slots, r_max, d_in)).astype(np.float32)
    B = rng.integers(-2, 3, size=(n_slots, d_out, r_max)).astype(np.float32)
    alpha = [4.0, 1.0, 6.0]
    row_slot = [0, -1, 2, 1, 0, 2, -1]
    mag = [rng.integers(1, 5, size=d_out).astype(np.float32), None,
           rng.integers(1, 5, size=d_out).astype(np.float32)]
    Y = oracle.dora_forward(X, W, A, B, row_slot, ranks, alpha, mag, r_max, "f32")
    for i in range(n):
        a = row_slot[i]
        for j in range(d_out):
            if a < 0 or ranks[a] == 0:
                exp = sum(float(W[j][c]) * float(X[i][c]) for c in range(d_in))
            else:
                s = alpha[a] / ranks[a]
                v = [float(W[j][c]) + s * sum(float(B[a][j][k]) * float(A[a][k][c])
                                               for k in range(ranks[a])) for c in range(d_in)]
                nrm = math.sqrt(sum(t * t for t in v))
                f = float(mag[a][j]) / nrm if nrm > 0 else 0.0
                exp = sum(f * v[c] * float(X[i][c]) for c in range(d_in))
            assert abs(Y[i][j] - exp) <= 1e-12 * max(1.0, abs(exp)), (i, j)


# planted mistakes in the definition: each must fail the hand-worked fixture
MUTATIONS = {
    "norm_of_W0": ("nj = np.sqrt(np.dot(V[j], V[j]))", "nj = np.sqrt(np.dot(W64[j], W64[j]))"),
    "squared_norm": ("nj = np.sqrt(np.dot(V[j], V[j]))", "nj = np.dot(V[j], V[j])"),
    "column_norm": ("nj = np.sqrt(np.dot(V[j], V[j]))",
                    "nj = np.sqrt(np.dot(V[:, j % V.shape[1]], V[:, j % V.shape[1]]))"),
    "no_normalisation": ("Wp[j] = m[j] * V[j] / nj", "Wp[j] = m[j] * V[j]"),
    "magnitude_reversed": ("Wp[j] = m[j] * V[j] / nj", "Wp[j] = m[::-1][j] * V[j] / nj"),
    "unscaled_delta": ("V = _direction(W64, A, B, slot_rank, slot_alpha, dtype, a)",
                       "V = _direction(W64, A, B, slot_rank, np.asarray(slot_rank, float), dtype, a)"),
    "rank0_rescaled": ("if a == -1 or int(slot_rank[a]) == 0:", "if a == -1:"),
    "plain_slot_normalised": ("if magnitude[a] is None:\n                Wp = V",
                              "if magnitude[a] is None:\n                Wp = V / np.linalg.norm(V, axis=1, keepdims=True)"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(lo.dora_forward))
    assert old in src, name
    ns = dict(vars(lo))
    exec(src.replace(old, new), ns)
    return ns["dora_forward"]


def _fixture_passes(fwd):
    g, args = _fixture("f32")
    try:
        with np.errstate(all="ignore"):
            return fwd(*args).tolist() == g["expected"]["Y"]
    except Exception:
        return False


def test_unmutated_definition_passes():
    assert _fixture_passes(lo.dora_forward)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_fails_the_fixture(name):
    assert not _fixture_passes(_mutant(name))
