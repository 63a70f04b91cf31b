"""GPU parity of the segment build (adapter-batching page, section "Segmented
Kernel 需要哪些 Metadata": one segment per distinct adapter in order of first
appearance, rows ascending inside each, with offsets, slots, ranks, scales
and the token permutation) on the shapes that take each of its paths:
segments numbered from the row bitmap (up to 65,536 rows) or chunk by
chunk (more rows), rows placed through the per-wave segment table (up to
256 segments) or by the serial walk over the waves' group leaders (more),
and row keys kept in registers (up to 24 chunks of 1024 rows) or read back
from memory.  Every field must equal the oracle's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_segment_amd as srg
from gpu_harness import DEV, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    srg.lib()
    yield
    torch.cuda.synchronize()


def mapping(seed, n, n_slots, kind, p_base=0.1, p_bad=0.0):
    rng = np.random.default_rng(seed)
    if kind == "runs":
        out = []
        while len(out) < n:
            L = int(rng.integers(1, max(2, n // 8) + 1))
            s = -1 if rng.random() < p_base else int(rng.integers(0, n_slots))
            out.extend([s] * L)
        rs = np.array(out[:n], dtype=np.int32)
    elif kind == "zipf":
        rs = (rng.zipf(1.2, size=n) - 1) % n_slots
        rs = np.where(rng.random(n) < p_base, -1, rs).astype(np.int32)
    else:
        rs = np.where(rng.random(n) < p_base, -1, rng.integers(0, n_slots, size=n)).astype(np.int32)
    if p_bad:
        bad = rng.random(n) < p_bad
        rs = np.where(bad, rng.choice([-5, n_slots, n_slots + 7], size=n), rs).astype(np.int32)
    return rs


def build(seed, n, n_slots, kind, r_max=16, **kw):
    rng = np.random.default_rng(seed + 1)
    rank = rng.choice([0, 8, 16, r_max], size=n_slots).astype(np.int32)
    rank[rng.random(n_slots) < 0.05] = r_max + 8        # out of range: rows demoted
    alpha = rng.uniform(4.0, 32.0, size=n_slots)
    rs = mapping(seed, n, n_slots, kind, **kw)
    A = torch.zeros((n_slots, r_max, 8), dtype=torch.bfloat16, device=DEV)
    Bt = torch.zeros((n_slots, r_max, 8), dtype=torch.bfloat16, device=DEV)
    pool = srg.Pool(A, Bt, torch.from_numpy(rank).to(DEV), alpha)
    seg = srg.Segments(n, n_slots, DEV)
    srg.lora_build_segments(torch.from_numpy(rs).to(DEV), pool, seg)
    torch.cuda.synchronize()
    return rs, rank, alpha, seg.to_host()


def check(rs, rank, alpha, r_max, m):
    ref = oracle.segment_metadata(rs, rank, alpha, r_max)
    assert m["num_segments"] == int(ref["num_segments"])
    for k in ("segment_offsets", "segment_slots", "segment_ranks", "token_indices", "row_segment"):
        assert np.array_equal(m[k], ref[k]), k
    assert np.array_equal(m["segment_scales"].view(np.uint32),
                          ref["segment_scales"].astype(np.float32).view(np.uint32))
    assert m["status"] == int(ref["status"])
    return int(ref["num_segments"])


CASES = [
    # seed, rows, slots, mapping, extra
    (901, 16943, 7, "runs", {}),                   # prefill-like: bitmap, table, keys in registers
    (902, 30000, 200, "uniform", {}),              # keys past the register chunks, table
    (903, 5000, 1000, "uniform", {}),              # > 256 segments: the serial walk
    (904, 40000, 4095, "zipf", {"p_bad": 0.01}),   # largest pool, walk, keys read back
    (905, 65536, 50, "runs", {}),                  # last bitmap size
    (906, 65537, 50, "runs", {}),                  # chunk-by-chunk numbering
    (907, 100000, 300, "zipf", {"p_bad": 0.02}),   # chunk numbering and the walk
    (908, 24576, 255, "uniform", {"p_base": 0.0}),  # 255 slots (+ base rows demoted): <= 256 segments
    (909, 24577, 300, "uniform", {"p_base": 0.3}),  # one row past the register chunks
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_build_paths(case):
    seed, n, n_slots, kind, kw = case
    say("build", case)
    rs, rank, alpha, m = build(seed, n, n_slots, kind, **kw)
    S = check(rs, rank, alpha, 16, m)
    say("segments", S)


def test_segment_count_around_the_table_size():
    """Exactly 256 and 257 segments (one row per key plus a base-only run)."""
    for S in (256, 257):
        n_slots = S - 1
        rng = np.random.default_rng(S)
        rs = np.concatenate([rng.permutation(n_slots), np.full(3000, -1),
                             rng.integers(0, n_slots, 2000)]).astype(np.int32)
        rank = np.full(n_slots, 8, dtype=np.int32)
        alpha = np.full(n_slots, 16.0)
        A = torch.zeros((n_slots, 8, 8), dtype=torch.bfloat16, device=DEV)
        pool = srg.Pool(A, A.clone(), torch.from_numpy(rank).to(DEV), alpha)
        seg = srg.Segments(len(rs), n_slots, DEV)
        srg.lora_build_segments(torch.from_numpy(rs).to(DEV), pool, seg)
        torch.cuda.synchronize()
        assert check(rs, rank, alpha, 8, seg.to_host()) == S
