"""Planted mistakes: each mutant of the oracle's row loop must fail a pin.

The mutant is built on the CPU from the oracle's own source with one textual
change, and run through the same checks the pins use (hand-worked example,
fingerprint adapters, base-only rows, exact integer case).  This shows that
the pins can see a dropped term, a wrong sign, a wrong scale, a wrong row
or a wrong operand.
"""
import inspect
import json
import os
import textwrap

import numpy as np
import pytest

import oracle
import oracle.lora_oracle as lo
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")

MUTATIONS = {
    "dropped_base": ("return Ybase + dY, dY, H", "return dY, dY, H"),
    "dropped_lora": ("dY[t] = s * (Ba @ h)", "dY[t] = 0.0 * (Ba @ h)"),
    "wrong_sign": ("dY[t] = s * (Ba @ h)", "dY[t] = -s * (Ba @ h)"),
    "scale_r_over_alpha": ("_scale(slot_alpha[a], r))", "(r / float(slot_alpha[a])))"),
    "scale_missing": ("_scale(slot_alpha[a], r))", "1.0)"),
    "wrong_row": ("x = X64[i]", "x = X64[(i + 1) % n]"),
    "transposed_A_index": ("np.dot(Aa[k], x)", "np.dot(Aa[r - 1 - k], x)"),
    "B_column_reversed": ("dY[t] = s * (Ba @ h)", "dY[t] = s * (Ba[::-1] @ h)"),
    "rank_off_by_one": ("r = int(slot_rank[a])\n        if r == 0:", "r = int(slot_rank[a]) - 1\n        if r <= 0:"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(lo.lora_forward))
    assert old in src, name
    ns = dict(vars(lo))
    exec(src.replace(old, new), ns)
    return ns["lora_forward"]


def _pins_pass(fwd):
    with open(os.path.join(GOLD, "hand_worked_3x2.json")) as f:
        g = json.load(f)
    Y, dY, H = fwd(np.array(g["X"], np.float32), np.array(g["W"], np.float32),
                   np.array(g["A"], np.float32), np.array(g["B"], np.float32),
                   g["row_slot"], g["slot_rank"], g["slot_alpha"], g["r_max"], "f32")
    if Y.tolist() != g["expected"]["Y"] or H.tolist() != g["expected"]["H"]:
        return False
    w = wl.make_fingerprint(5, n=64, d_in=48, d_out=24, n_slots=20, r_max=32, dtype="bf16")
    Y, dY, H = fwd(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha, w.r_max, w.dtype)
    X = oracle.decode(w.X, "bf16")
    for i in range(w.n):
        a = int(w.row_slot[i])
        exp = 0.0 if a < 0 else 16.0 / int(w.slot_rank[a]) * (a + 1) * X[i, a % w.d_in]
        if not np.all(dY[i] == exp):
            return False
    w = wl.make_random(3, n=20, d_in=64, d_out=48, n_slots=3, r_max=8, p_base=1.0, dtype="bf16")
    Y, dY, H = fwd(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha, w.r_max, w.dtype)
    if not np.array_equal(Y, oracle.decode(w.X, "bf16") @ oracle.decode(w.W, "bf16").T):
        return False
    return True


def test_unmutated_oracle_passes_pins():
    assert _pins_pass(lo.lora_forward)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_fails_a_pin(name):
    assert not _pins_pass(_mutant(name))
