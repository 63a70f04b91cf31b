"""Pins of the stacked-projection oracle (adapter-batching page, "Adapter 不是
一块连续 Weight": each target module keeps its own A and B; a fused QKV or
stacked gate/up weight runs them together and concatenates the outputs).

Checked against the merged closed form per projection (an independent
formulation), against block independence (changing one projection's adapter
or weight changes only that projection's columns) and against projection
order (a wrong order gives stable wrong outputs, as the page warns)."""
import numpy as np
import pytest

import oracle
import workloads as wl


def _projections(seed, n=30, d_in=48, outs=(24, 8, 16), n_slots=4, r_max=16, dtype="bf16"):
    base = wl.make_random(seed, n, d_in, outs[0], n_slots, r_max, p_base=0.2, dtype=dtype)
    ws = [base]
    for p, d_out in enumerate(outs[1:], 1):
        w = wl.make_random(seed * 10 + p, n, d_in, d_out, n_slots, r_max, dtype=dtype,
                           ranks=list(base.slot_rank))
        w.X, w.row_slot = base.X, base.row_slot
        ws.append(w)
    return ws


def _stacked(ws, rows=None):
    b = ws[0]
    return oracle.stacked_forward(b.X, [w.W for w in ws], [w.A for w in ws], [w.B for w in ws],
                                  b.row_slot, b.slot_rank, b.slot_alpha, b.r_max, b.dtype, rows=rows)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_equals_merged_form_per_projection(dtype):
    ws = _projections(1, dtype=dtype)
    Y, dY, H = _stacked(ws)
    b = ws[0]
    col = 0
    for w in ws:
        Ym = oracle.merged_forward(b.X, w.W, w.A, w.B, b.row_slot, b.slot_rank, b.slot_alpha,
                                   b.r_max, dtype)
        np.testing.assert_allclose(Y[:, col:col + w.d_out], Ym, rtol=1e-10, atol=1e-12)
        col += w.d_out
    assert col == Y.shape[1] and H.shape == (b.n, len(ws) * b.r_max)


def test_block_independence_and_rank_columns():
    ws = _projections(2)
    Y, _, H = _stacked(ws)
    ws2 = _projections(2)
    ws2[1].A[:] = ws2[2].A                    # change projection 1's adapters only
    ws2[1].W[:] = ws2[1].W[::-1]              # and its base weight
    Y2, _, H2 = _stacked(ws2)
    c0, c1 = ws[0].d_out, ws[0].d_out + ws[1].d_out
    np.testing.assert_array_equal(Y2[:, :c0], Y[:, :c0])
    np.testing.assert_array_equal(Y2[:, c1:], Y[:, c1:])
    assert not np.allclose(Y2[:, c0:c1], Y[:, c0:c1])
    r = ws[0].r_max
    np.testing.assert_array_equal(H2[:, :r], H[:, :r])
    np.testing.assert_array_equal(H2[:, 2 * r:], H[:, 2 * r:])


def test_projection_order_matters():
    ws = _projections(3, outs=(16, 16, 16))
    Y, _, _ = _stacked(ws)
    Ys, _, _ = _stacked([ws[1], ws[0], ws[2]])
    np.testing.assert_array_equal(Ys[:, :16], Y[:, 16:32])
    np.testing.assert_array_equal(Ys[:, 16:32], Y[:, :16])
    assert not np.allclose(Ys, Y)


def test_single_projection_and_rows():
    ws = _projections(4)
    b = ws[0]
    Y, dY, H = _stacked(ws[:1])
    Yr, dYr, Hr = oracle.lora_forward(b.X, b.W, b.A, b.B, b.row_slot, b.slot_rank, b.slot_alpha,
                                      b.r_max, b.dtype)
    np.testing.assert_array_equal(Y, Yr)
    np.testing.assert_array_equal(H, Hr)
    rows = [3, 0, 17]
    Ys, _, _ = _stacked(ws, rows=rows)
    np.testing.assert_allclose(Ys, _stacked(ws)[0][rows], rtol=1e-13, atol=1e-15)
