"""GPU: lora_build_shrink (metadata build and shrink in one call) gives the
same metadata and the same H bits as lora_build_segments followed by
lora_shrink, in its one-launch range (up to 512 rows) and past it, and H
matches the oracle."""
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


def _both(w, policy="exact"):
    d = wl.device_tensors(w, DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, policy)
    out = []
    for one_call in (False, True):
        seg = srg.Segments(w.n, w.n_slots, DEV)
        H = torch.full((w.n, w.r_max), float("nan"), dtype=torch.float32, device=DEV)
        if one_call:
            srg.lora_build_shrink(d["row_slot"], d["X"], pool, seg, H)
        else:
            srg.lora_build_segments(d["row_slot"], pool, seg)
            srg.lora_shrink(d["X"], seg, pool, H)
        torch.cuda.synchronize()
        out.append((seg.to_host(), H))
    return out


def _same(w, policy="exact"):
    (m0, H0), (m1, H1) = _both(w, policy)
    for k in ("segment_offsets", "segment_slots", "segment_ranks", "token_indices", "row_segment"):
        assert np.array_equal(m0[k], m1[k]), k
    assert np.array_equal(m0["segment_scales"].view(np.uint32), m1["segment_scales"].view(np.uint32))
    assert m0["num_segments"] == m1["num_segments"] and m0["status"] == m1["status"]
    # bit patterns, so untouched NaN entries compare equal too
    assert torch.equal(H0.view(torch.int32), H1.view(torch.int32))
    return m1, H1


def _oracle_H(w, H):
    _, _, Hr = oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                   w.r_max, w.dtype)
    Hg = to_f64(H)
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    mask = np.zeros_like(Hg, dtype=bool)
    for i, a in enumerate(keys):
        if a >= 0:
            mask[i, :int(w.slot_rank[a])] = True
    assert np.all(np.isnan(Hg[~mask])) and np.all(np.isfinite(Hg[mask]))
    e = normwise(np.where(mask, Hg, 0.0), Hr)
    assert e <= TOL[w.dtype], e
    return e


CASES = [
    # seed, n, d_in, d_out, n_slots, r_max, p_base, dtype, runs
    (401, 1, 64, 72, 3, 8, 0.0, "bf16", False),
    (402, 7, 136, 200, 5, 16, 0.3, "bf16", False),
    (403, 300, 520, 264, 40, 64, 0.1, "bf16", False),
    (404, 333, 256, 384, 6, 32, 0.2, "bf16", True),      # long runs: several row blocks per slot
    (405, 257, 96, 88, 300, 16, 0.5, "bf16", False),
    (406, 512, 200, 136, 7, 64, 0.1, "bf16", True),      # the largest one-launch batch
    (407, 513, 200, 136, 7, 64, 0.1, "bf16", True),      # just past it: two launches
    (408, 70, 64, 64, 4, 64, 0.1, "f32", True),
    (409, 100, 200, 120, 17, 32, 0.1, "f32", False),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
@pytest.mark.parametrize("policy", ["exact", "padded"])
def test_one_call_equals_two_calls(case, policy):
    seed, n, d_in, d_out, n_slots, r_max, p_base, dtype, runs = case
    say("build_shrink", case, policy)
    w = wl.make_random(seed, n, d_in, d_out, n_slots, r_max, p_base=p_base, dtype=dtype, runs=runs)
    if n_slots > 2:
        w.slot_rank[1] = 0
    _, H = _same(w, policy)
    _oracle_H(w, H)


def test_decode_workload():
    w = wl.make_workload("decode")
    _, H = _same(w)
    say("decode H error", _oracle_H(w, H))


def test_invalid_rows():
    w = wl.make_random(410, 200, 64, 72, 6, 16, p_base=0.2, dtype="bf16")
    w.slot_rank[2] = 99                    # outside [0, r_max]: its rows are base-only
    w.row_slot[5] = 6                      # slot outside the pool
    w.row_slot[9] = -7
    m, H = _same(w)
    assert m["status"] == 2 + int(np.sum(w.row_slot == 2))
    rows = [i for i in range(w.n) if w.row_slot[i] in (2, 6, -7)]
    assert torch.isnan(H[rows]).all()


def test_empty_batch():
    w = wl.make_random(411, 0, 64, 72, 3, 8, dtype="bf16")
    d = wl.device_tensors(w, DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha)
    seg = srg.Segments(0, 3, DEV)
    H = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    srg.lora_build_shrink(d["row_slot"], d["X"], pool, seg, H)
    torch.cuda.synchronize()
    m = seg.to_host()
    assert m["num_segments"] == 0 and m["status"] == 0
