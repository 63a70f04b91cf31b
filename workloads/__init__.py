"""Seeded synthetic inputs for the multi-LoRA linear layer.

This module only draws numbers and lays them out. It holds none of the
method's arithmetic (no products, no scales, no grouping): both the CPU
oracle (``oracle/``) and the HIP path (``segmented_rank_gemm_segment_amd``)
take their inputs from here, and neither imports the other.

Layouts (row-major, element units):

* ``X``  [n, d_in]                 token rows
* ``W``  [d_out, d_in]             base weight, ``nn.Linear`` layout
* ``A``  [n_slots, r_max, d_in]    adapter down-projections, rank-major
* ``Bt`` [n_slots, r_max, d_out]   adapter up-projections stored transposed
  (row k of slot a is column k of B_a); ``Workload.B`` is the [n_slots,
  d_out, r_max] view the pages' notation uses (B_a in R^{d_out x r}).
* rows ``k >= slot_rank[a]`` of a slot are pool padding.  By default they
  hold NaN so that any consumer that reads padding into a result is caught.

bf16 tensors are ``numpy.uint16`` bit patterns, rounded from float32 draws
with round-to-nearest-even.  fp32 tensors are ``numpy.float32``.

Shapes, distributions and mappings follow the five workloads the pages'
prefill / decode discussion implies (see the docstrings of ``tiny_f32``,
``decode``, ``prefill``, ``skewed_decode`` and ``layer70b_projection``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

ALPHA = 16.0          # LoRA alpha used by every workload
RANK_SET = (8, 16, 32, 64)

BF16_NAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# number formats (input encoding only)
# --------------------------------------------------------------------------
def bf16_bits_rne(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even (IEEE-754).

    Only finite inputs are expected (the generators draw normals)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_bits_rne expects finite input")
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    dtype: str                 # "bf16" or "f32"
    n: int
    d_in: int
    d_out: int
    n_slots: int
    r_max: int
    row_slot: np.ndarray       # int32 [n], -1 = base-only row
    slot_rank: np.ndarray      # int32 [n_slots]
    slot_alpha: np.ndarray     # float64 [n_slots]
    X: np.ndarray              # [n, d_in]
    W: np.ndarray              # [d_out, d_in]
    A: np.ndarray              # [n_slots, r_max, d_in]
    Bt: np.ndarray             # [n_slots, r_max, d_out]
    meta: Dict = field(default_factory=dict)

    @property
    def B(self) -> np.ndarray:
        """[n_slots, d_out, r_max] view: B[a] is the pages' B_a."""
        return self.Bt.transpose(0, 2, 1)

    def as_f32(self, name: str) -> np.ndarray:
        """Widen one tensor to float32 (bf16 decode is exact)."""
        t = getattr(self, name)
        return bf16_bits_to_f32(t) if self.dtype == "bf16" else t


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def _encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_rne(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _normal(rng, shape, std, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _encode(x, dtype)


def _pool(rng, slot_rank, r_max, d, std, dtype, pad):
    """[n_slots, r_max, d] with N(0, std) in rows < rank and `pad` elsewhere."""
    n_slots = len(slot_rank)
    et = np.uint16 if dtype == "bf16" else np.float32
    if pad == "nan":
        fill = BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    elif pad == "zero":
        fill = 0
    else:
        raise ValueError(pad)
    P = np.full((n_slots, r_max, d), fill, dtype=et)
    total = int(np.sum(slot_rank))
    if total:
        draws = _normal(rng, (total, d), std, dtype)
        o = 0
        for a in range(n_slots):
            r = int(slot_rank[a])
            P[a, :r] = draws[o:o + r]
            o += r
    return P


def build_workload(name, dtype, seed_seq, n, d_in, d_out, row_slot, slot_rank, r_max,
                   x_std, w_std, ab_std, pad="nan", meta=None) -> Workload:
    """Draw X, W, A, B for a given mapping. Sub-streams: X, W, A, B."""
    sx, sw, sa, sb = seed_seq.spawn(4)
    slot_rank = np.asarray(slot_rank, dtype=np.int32)
    X = _normal(_rng(sx), (n, d_in), x_std, dtype)
    W = _normal(_rng(sw), (d_out, d_in), w_std, dtype)
    A = _pool(_rng(sa), slot_rank, r_max, d_in, ab_std, dtype, pad)
    Bt = _pool(_rng(sb), slot_rank, r_max, d_out, ab_std, dtype, pad)
    return Workload(name=name, dtype=dtype, n=n, d_in=d_in, d_out=d_out,
                    n_slots=len(slot_rank), r_max=r_max,
                    row_slot=np.asarray(row_slot, dtype=np.int32), slot_rank=slot_rank,
                    slot_alpha=np.full(len(slot_rank), ALPHA, dtype=np.float64),
                    X=X, W=W, A=A, Bt=Bt, meta=dict(meta or {}))


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
def tiny_f32(pad="nan") -> Workload:
    """Tiny fp32 check: d_in = d_out = 512, 32 rows in four runs
    [0,8) -> adapter A (r=8), [8,12) -> base only, [12,28) -> adapter B (r=16),
    [28,32) -> adapter C (r=8); alpha 16; W, A, B, X ~ N(0, 0.02)."""
    ss = np.random.SeedSequence(1)
    s_map, s_data = ss.spawn(2)
    row_slot = np.array([0] * 8 + [-1] * 4 + [1] * 16 + [2] * 4, dtype=np.int32)
    return build_workload("tiny_f32", "f32", s_data, 32, 512, 512, row_slot,
                          [8, 16, 8], 16, 0.02, 0.02, 0.02, pad,
                          meta={"offsets_printed": [0, 8, 12, 28, 32]})


def decode(pad="nan") -> Workload:
    """Decode GEMV, bf16: d_in = d_out = 4096 (an 8B-class q_proj), 256 rows of
    one token each, 128 slots all rank 16, each row base-only with p = 0.1 else
    a uniform slot; W, A, B ~ N(0, 0.02), X ~ N(0, 1)."""
    ss = np.random.SeedSequence(2)
    s_map, s_data = ss.spawn(2)
    rng = _rng(s_map)
    n = 256
    is_base = rng.random(n) < 0.1
    slots = rng.integers(0, 128, size=n)
    row_slot = np.where(is_base, -1, slots).astype(np.int32)
    return build_workload("decode_bf16", "bf16", s_data, n, 4096, 4096, row_slot,
                          [16] * 128, 16, 1.0, 0.02, 0.02, pad)


def prefill(pad="nan", lengths_override: Optional[List[int]] = None) -> Workload:
    """Prefill segmented GEMM, bf16: d_in 4096 -> d_out 14336 (MLP up-proj);
    8 requests with lengths uniform in [512, 4096]; slots 0..7 with ranks
    8,8,16,16,32,32,64,64; request k uses slot k for k < 7, request 7 is
    base-only (slot 7 stays resident, unused).  X ~ N(0,1), W/A/B ~ N(0,0.02).
    ``lengths_override`` keeps the structure at a smaller size (tests)."""
    ss = np.random.SeedSequence(3)
    s_map, s_data = ss.spawn(2)
    rng = _rng(s_map)
    lengths = rng.integers(512, 4097, size=8)
    if lengths_override is not None:
        lengths = np.asarray(lengths_override)
    row_slot = np.concatenate([np.full(int(L), k if k < 7 else -1, dtype=np.int32)
                               for k, L in enumerate(lengths)])
    return build_workload("prefill_bf16", "bf16", s_data, int(lengths.sum()), 4096, 14336,
                          row_slot, [8, 8, 16, 16, 32, 32, 64, 64], 64, 1.0, 0.02, 0.02, pad,
                          meta={"lengths": [int(v) for v in lengths]})


def skewed_decode(pad="nan") -> Workload:
    """Skewed large-pool decode, bf16: d_in = d_out = 4096, 1024 rows, 1000
    resident slots (r_max 64), ranks uniform over {8,16,32,64}, adapter ids
    Zipf(1.0) truncated to 1000 ids (P(k) proportional to 1/(k+1)); adapter k
    lives in slot k; no base-only rows."""
    ss = np.random.SeedSequence(4)
    s_map, s_data = ss.spawn(2)
    rng = _rng(s_map)
    n_slots, n = 1000, 1024
    ranks = rng.choice(np.array(RANK_SET), size=n_slots)
    p = 1.0 / np.arange(1, n_slots + 1, dtype=np.float64)
    p /= p.sum()
    row_slot = rng.choice(n_slots, size=n, p=p).astype(np.int32)
    return build_workload("skewed_decode_bf16", "bf16", s_data, n, 4096, 4096, row_slot,
                          ranks, 64, 1.0, 0.02, 0.02, pad)


# 70B-class layer: GQA attention projections plus a gated MLP.
LAYER70B_PROJECTIONS = (
    ("q_proj", 8192, 8192),
    ("k_proj", 8192, 1024),
    ("v_proj", 8192, 1024),
    ("o_proj", 8192, 8192),
    ("gate_proj", 8192, 28672),
    ("up_proj", 8192, 28672),
    ("down_proj", 28672, 8192),
)


def layer70b_mapping():
    """Rows [0, 2048) are one chunked-prefill request on one seeded slot; rows
    [2048, 2304) are decode rows, each on a uniform slot of 64.  Slots 0..31
    have rank 16, slots 32..63 rank 64.  No base-only rows."""
    ss = np.random.SeedSequence(5)
    s_map, s_data = ss.spawn(2)
    rng = _rng(s_map)
    prefill_slot = int(rng.integers(0, 64))
    dec = rng.integers(0, 64, size=256)
    row_slot = np.concatenate([np.full(2048, prefill_slot), dec]).astype(np.int32)
    ranks = np.array([16] * 32 + [64] * 32, dtype=np.int32)
    return row_slot, ranks, s_data


def layer70b_projection(name: str, pad="nan", n_rows: Optional[int] = None) -> Workload:
    """One projection of the 70B-shaped mixed layer (own seeded X, W, pool)."""
    names = [p[0] for p in LAYER70B_PROJECTIONS]
    i = names.index(name)
    _, d_in, d_out = LAYER70B_PROJECTIONS[i]
    row_slot, ranks, s_data = layer70b_mapping()
    s_proj = s_data.spawn(len(LAYER70B_PROJECTIONS))[i]
    if n_rows is not None:
        row_slot = row_slot[:n_rows]
    return build_workload("layer70b_" + name, "bf16", s_proj, len(row_slot), d_in, d_out, row_slot,
                          ranks, 64, 1.0, 0.02, 0.02, pad, meta={"projection": name})


# the single-projection workloads by name, and the seed each draws from (the
# 70B-shaped layer, seven projections, is ``layer70b_projection``; seed 5)
WORKLOADS = {"tiny_f32": tiny_f32, "decode": decode, "prefill": prefill,
             "skewed_decode": skewed_decode}
SEEDS = {"tiny_f32": 1, "decode": 2, "prefill": 3, "skewed_decode": 4, "layer70b": 5}


def make_workload(name: str, pad: str = "nan") -> Workload:
    """One of ``WORKLOADS`` by name."""
    return WORKLOADS[name](pad=pad)


# --------------------------------------------------------------------------
# generic and special-purpose generators for tests
# --------------------------------------------------------------------------
def make_random(seed: int, n: int, d_in: int, d_out: int, n_slots: int, r_max: int,
                ranks=None, p_base: float = 0.1, dtype: str = "bf16", pad: str = "nan",
                x_std: float = 1.0, w_std: float = 0.02, ab_std: float = 0.02,
                runs: bool = False) -> Workload:
    """Random mapping: each row base-only with probability p_base, else a
    uniform slot.  ``ranks`` is a list per slot, or None for uniform draws
    from the ranks <= r_max in {8,16,32,64}.  ``runs`` draws contiguous
    request runs of random length instead of independent rows."""
    ss = np.random.SeedSequence(seed)
    s_map, s_data = ss.spawn(2)
    rng = _rng(s_map)
    if ranks is None:
        choices = np.array([r for r in RANK_SET if r <= r_max])
        ranks = rng.choice(choices, size=n_slots)
    ranks = np.asarray(ranks, dtype=np.int32)
    if runs:
        row_slot = []
        while len(row_slot) < n:
            L = int(rng.integers(1, max(2, n // 4) + 1))
            s = -1 if rng.random() < p_base else int(rng.integers(0, n_slots))
            row_slot.extend([s] * L)
        row_slot = np.array(row_slot[:n], dtype=np.int32)
    else:
        is_base = rng.random(n) < p_base
        slots = rng.integers(0, n_slots, size=n)
        row_slot = np.where(is_base, -1, slots).astype(np.int32)
    return build_workload(f"random_s{seed}", dtype, s_data, n, d_in, d_out, row_slot, ranks,
                          r_max, x_std, w_std, ab_std, pad)


def make_integer_case(seed: int, n: int, d_in: int, d_out: int, n_slots: int, r_max: int,
                      ranks, row_slot, lo: int = -3, hi: int = 3, dtype: str = "f32",
                      pad: str = "nan") -> Workload:
    """Small-integer entries in [lo, hi]: every product and sum of the method
    is exact in fp32 at these sizes, so results can be pinned exactly."""
    ss = np.random.SeedSequence(seed)
    rng = _rng(ss)
    ranks = np.asarray(ranks, dtype=np.int32)

    def ints(shape):
        return _encode(rng.integers(lo, hi + 1, size=shape).astype(np.float32), dtype)

    X = ints((n, d_in))
    W = ints((d_out, d_in))
    et = np.uint16 if dtype == "bf16" else np.float32
    fill = (BF16_NAN if dtype == "bf16" else np.float32(np.nan)) if pad == "nan" else 0
    A = np.full((n_slots, r_max, d_in), fill, dtype=et)
    Bt = np.full((n_slots, r_max, d_out), fill, dtype=et)
    for a in range(n_slots):
        r = int(ranks[a])
        A[a, :r] = ints((r, d_in))
        Bt[a, :r] = ints((r, d_out))
    return Workload(name=f"int_s{seed}", dtype=dtype, n=n, d_in=d_in, d_out=d_out,
                    n_slots=n_slots, r_max=r_max,
                    row_slot=np.asarray(row_slot, dtype=np.int32), slot_rank=ranks,
                    slot_alpha=np.asarray(ranks, dtype=np.float64).copy(),  # alpha = r -> s = 1
                    X=X, W=W, A=A, Bt=Bt)


def make_fingerprint(seed: int, n: int, d_in: int, d_out: int, n_slots: int, r_max: int,
                     ranks=None, p_base: float = 0.1, dtype: str = "bf16", runs: bool = False,
                     row_slot=None) -> Workload:
    """Fingerprint adapters: slot a has A_a row 0 = unit vector at column
    (a mod d_in) and every other rank row zero, and B_a filled with the
    constant (a + 1) (exact in bf16 for a < 256).  The LoRA increment of a row
    on slot a is then s_a * (a + 1) * x[a mod d_in] in every output column, so
    a row that picks up another slot's weights is off by a visible amount.
    ``runs`` draws request runs as make_random does; ``row_slot`` (int32 [n])
    replaces the drawn mapping."""
    w = make_random(seed, n, d_in, d_out, n_slots, r_max, ranks=ranks, p_base=p_base,
                    dtype=dtype, pad="nan", runs=runs)
    if row_slot is not None:
        w.row_slot = np.asarray(row_slot, dtype=np.int32).copy()
        if len(w.row_slot) != n:
            raise ValueError("row_slot must have n entries")
    if dtype == "f32":
        # keep x on the bf16 grid so that s_a (a + 1) x is exact in fp32 too
        w.X = bf16_bits_to_f32(bf16_bits_rne(w.X))
    et = np.uint16 if dtype == "bf16" else np.float32
    for a in range(n_slots):
        r = int(w.slot_rank[a])
        rowsA = np.zeros((r, d_in), dtype=np.float32)
        if r > 0:
            rowsA[0, a % d_in] = 1.0
        rowsB = np.full((r, d_out), float(a + 1), dtype=np.float32)
        w.A[a, :r] = _encode(rowsA, dtype).astype(et)
        w.Bt[a, :r] = _encode(rowsB, dtype).astype(et)
    w.name = f"fingerprint_s{seed}"
    return w


def tile_runs_mapping(seed: int, n: int, tile_rows: int, runs, n_slots: int,
                      base_every: int = 3) -> np.ndarray:
    """A row -> slot mapping whose consecutive blocks of ``tile_rows`` rows
    hold runs[t % len(runs)] runs each (block t), every run on a slot other
    than its neighbours', and in every ``base_every``-th block one run
    base-only (-1).  The last block may be short.  Mapping only."""
    rng = _rng(np.random.SeedSequence([seed, 0x7E]))
    out = []
    t = 0
    while len(out) < n:
        rows = min(tile_rows, n - len(out))
        k = max(1, min(int(runs[t % len(runs)]), rows))
        cuts = np.sort(rng.choice(np.arange(1, rows), size=k - 1, replace=False)) if k > 1 else []
        lens = np.diff(np.concatenate([[0], cuts, [rows]])).astype(int)
        slots = rng.choice(n_slots, size=k, replace=k > n_slots)
        for j in range(1, k):
            if slots[j] == slots[j - 1]:
                slots[j] = (slots[j] + 1) % n_slots
        if base_every and t % base_every == base_every - 1:
            slots[k // 2] = -1
        for L, sl in zip(lens, slots):
            out.extend([int(sl)] * int(L))
        t += 1
    return np.array(out[:n], dtype=np.int32)


def fp8_e4m3_bits_rne(x32) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 bit patterns (uint8), round to nearest even,
    saturating at +-448 (input encoding only; torch's conversion)."""
    import torch
    t = torch.from_numpy(np.clip(np.asarray(x32, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def make_fp8_weight(seed: int, d_out: int, d_in: int, w_std: float = 0.02):
    """A quantized base weight: E4M3 codes of N(0, 1) draws [d_out, d_in]
    (uint8) and one float32 scale per output row, uniform in
    [0.5 w_std, 1.5 w_std], so the weight the codes stand for has about the
    spread of the bf16 workloads' W."""
    rng = _rng(np.random.SeedSequence([seed, 0xF8]))
    codes = fp8_e4m3_bits_rne(rng.standard_normal((d_out, d_in), dtype=np.float32))
    scale = ((rng.random(d_out, dtype=np.float32) + np.float32(0.5)) * np.float32(w_std))
    return codes, scale.astype(np.float32)


def make_magnitude(seed: int, n_slots: int, d_out: int, scale: float, p_plain: float = 0.25,
                   plain_slots=None):
    """DoRA magnitude vectors, one per slot: float32 [d_out] drawn uniform in
    [0.5 scale, 1.5 scale], or None (a plain LoRA slot) with probability
    ``p_plain`` or for the slots listed in ``plain_slots``.  ``scale`` is the
    caller's guess of a weight row's norm (e.g. w_std * sqrt(d_in)), so DoRA
    outputs keep the size of the base outputs."""
    rng = _rng(np.random.SeedSequence([seed, 0xD0]))
    plain = rng.random(n_slots) < p_plain
    if plain_slots is not None:
        plain[list(plain_slots)] = True
    out = []
    for a in range(n_slots):
        m = (rng.random(d_out, dtype=np.float32) + np.float32(0.5)) * np.float32(scale)
        out.append(None if plain[a] else m.astype(np.float32))
    return out


# --------------------------------------------------------------------------
# torch views (device placement only)
# --------------------------------------------------------------------------
def to_torch(arr: np.ndarray, dtype: str, device="cpu"):
    """numpy storage -> torch tensor of the same bits (bf16 from uint16)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def device_tensors(w: Workload, device) -> Dict:
    """X, W, A, Bt, row_slot, slot_rank of a workload on `device`."""
    import torch
    return {
        "X": to_torch(w.X, w.dtype, device),
        "W": to_torch(w.W, w.dtype, device),
        "A": to_torch(w.A, w.dtype, device),
        "Bt": to_torch(w.Bt, w.dtype, device),
        "row_slot": torch.from_numpy(np.ascontiguousarray(w.row_slot, dtype=np.int32)).to(device),
        "slot_rank": torch.from_numpy(np.ascontiguousarray(w.slot_rank, dtype=np.int32)).to(device),
    }
