"""Plain, slow, float64 CPU oracle of the multi-LoRA linear layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Notation follows the adapter-batching page ("Multi-LoRA Serving",
charlestar.github.io, section "LoRA 在一层 Linear 上增加了什么"):

    W in R^{d_out x d_in},  X in R^{n x d_in},  A in R^{r x d_in},
    B in R^{d_out x r},     s = alpha / r,
    Y = X W^T + s (X A^T) B^T.

For a mixed batch (same page, section "一个混合 Batch 的数学形式") every row
i carries its own slot a(i) (or none), and row i uses only A_{a(i)},
B_{a(i)}, s_{a(i)}; the base product is shared by all rows.  The page says
the batched kernels do not change this computation, so the oracle is that
definition written out row by row.

Inputs are taken exactly: bf16 bit patterns are widened by the oracle's own
shift (bf16 is the high half of an IEEE float32), then promoted to float64.
The pool argument ``B`` is the [n_slots, d_out, r_max] array whose slot a is
B_a as the pages write it; rows/columns at or beyond a slot's rank are pool
padding and are never read.

Readings of points the pages leave open:

* a row whose slot is outside [-1, n_slots) or whose slot rank is outside
  [0, r_max] is treated as base-only and counted in ``status``;
* a valid slot of rank 0 contributes nothing (scale 0) but keeps its own
  segment;
* segments come in first-appearance order of their key (the base-only key
  -1 is a key like any other) and rows inside a segment in ascending order;
  this reproduces the page's printed example.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np


# ---------------------------------------------------------------------------
# input decoding
# ---------------------------------------------------------------------------
def decode(t: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor.

    bf16 storage is the upper 16 bits of an IEEE-754 binary32, so shifting
    the pattern left by 16 gives the binary32 with the same value."""
    if dtype == "bf16":
        u = np.ascontiguousarray(t, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(t, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _scale(alpha: float, rank: int) -> float:
    """s = alpha / r (adapter-batching page, "LoRA 在一层 Linear 上增加了什么");
    zero for a rank-0 slot, which adds nothing."""
    return float(alpha) / float(rank) if rank > 0 else 0.0


# ---------------------------------------------------------------------------
# segment metadata
# ---------------------------------------------------------------------------
def validate_rows(row_slot, slot_rank, r_max: int):
    """Key of every row: its slot, or -1 (base-only) for a base row and for a
    row whose slot or slot rank is out of range.  Returns (keys, bad)."""
    n_slots = len(slot_rank)
    keys = []
    bad = 0
    for a in row_slot:
        a = int(a)
        ok = (a == -1) or (0 <= a < n_slots and 0 <= int(slot_rank[a]) <= r_max)
        if not ok:
            bad += 1
            a = -1
        keys.append(a)
    return keys, bad


def segment_metadata(row_slot, slot_rank, slot_alpha, r_max: int) -> Dict[str, np.ndarray]:
    """Group token rows by adapter slot (adapter-batching page, section
    "Segmented Kernel 需要哪些 Metadata"): one segment per distinct key,
    segments in order of first appearance, rows ascending inside a segment
    (plain Python lists; no sort routine).

    Returns the page's fields ``segment_offsets``, ``segment_slots``
    (``adapter_slots`` on the page, -1 for base), ``token_indices`` (gather
    form: sorted position -> original row), ``segment_ranks``,
    ``segment_scales`` (float64), plus ``num_segments``, ``row_segment``
    (original row -> segment id) and ``status`` (rows treated as base-only
    because their slot or rank was out of range)."""
    keys, bad = validate_rows(row_slot, slot_rank, r_max)
    order = []
    rows_of = {}
    for i, k in enumerate(keys):
        if k not in rows_of:
            rows_of[k] = []
            order.append(k)
        rows_of[k].append(i)
    token_indices = []
    offsets = [0]
    for k in order:
        token_indices.extend(rows_of[k])
        offsets.append(len(token_indices))
    seg_of_key = {k: s for s, k in enumerate(order)}
    ranks = [0 if k == -1 else int(slot_rank[k]) for k in order]
    scales = [0.0 if k == -1 else _scale(slot_alpha[k], r) for k, r in zip(order, ranks)]
    return {
        "num_segments": np.int32(len(order)),
        "segment_offsets": np.asarray(offsets, dtype=np.int32),
        "segment_slots": np.asarray(order, dtype=np.int32),
        "token_indices": np.asarray(token_indices, dtype=np.int32),
        "segment_ranks": np.asarray(ranks, dtype=np.int32),
        "segment_scales": np.asarray(scales, dtype=np.float64),
        "row_segment": np.asarray([seg_of_key[k] for k in keys], dtype=np.int32),
        "status": np.int32(bad),
    }


# ---------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------
def lora_forward(X, W, A, B, row_slot, slot_rank, slot_alpha, r_max: int, dtype: str,
                 rows: Optional[Iterable[int]] = None):
    """Y = X W^T + s_a (X_a A_a^T) B_a^T, one row at a time.

    For every requested row i (all rows by default):

    * base:    y_i[j] = sum_c W[j, c] x_i[c] for every output column j
      (adapter-batching page, "一个混合 Batch 的数学形式": the base product is
      shared by all rows; taken for the requested rows as one float64
      matrix product, which is that definition);
    * shrink:  h_i[k] = sum_c A_a[k, c] x_i[c] for k < r_a (same page,
      "Segmented Kernel 需要哪些 Metadata", H_a = X_a A_a^T);
    * expand:  dy_i[j] = s_a sum_k B_a[j, k] h_i[k] (same section,
      Delta Y_a = s_a H_a B_a^T), added back to row i.

    Returns float64 (Y, dY, H) for the requested rows, in request order;
    H is [len(rows), r_max] with zeros past each row's rank and for
    base-only rows."""
    X64 = decode(X, dtype)
    n = X64.shape[0]
    rows = list(range(n)) if rows is None else [int(i) for i in rows]
    keys, _ = validate_rows(row_slot, slot_rank, r_max)
    W64 = decode(W, dtype)
    Xr = X64[rows]
    Ybase = Xr @ W64.T
    d_out = W64.shape[0]
    dY = np.zeros((len(rows), d_out), dtype=np.float64)
    H = np.zeros((len(rows), r_max), dtype=np.float64)
    cache = {}
    for t, i in enumerate(rows):
        a = keys[i]
        if a == -1:
            continue
        r = int(slot_rank[a])
        if r == 0:
            continue
        if a not in cache:
            cache[a] = (decode(A[a, :r, :], dtype), decode(B[a, :, :r], dtype),
                        _scale(slot_alpha[a], r))
        Aa, Ba, s = cache[a]
        x = X64[i]
        h = np.array([np.dot(Aa[k], x) for k in range(r)])
        H[t, :r] = h
        dY[t] = s * (Ba @ h)
    return Ybase + dY, dY, H


# ---------------------------------------------------------------------------
# independent formulations used to cross-check the row loop
# ---------------------------------------------------------------------------
def _adapters_zero_padded(A, B, slot_rank, r_max, dtype):
    """float64 copies of A, B with every padding row/column set to 0 and one
    extra all-zero adapter appended at index n_slots for base-only rows."""
    n_slots = len(slot_rank)
    d_in = A.shape[2]
    d_out = B.shape[1]
    A64 = np.zeros((n_slots + 1, r_max, d_in))
    B64 = np.zeros((n_slots + 1, d_out, r_max))
    for a in range(n_slots):
        r = int(slot_rank[a])
        if 0 < r <= r_max:
            A64[a, :r] = decode(A[a, :r, :], dtype)
            B64[a, :, :r] = decode(B[a, :, :r], dtype)
    return A64, B64


def gather_bmm_forward(X, W, A, B, row_slot, slot_rank, slot_alpha, r_max, dtype):
    """Per-row gather of (A, B) followed by two batched products, as in the
    gather-scatter formulation (S-LoRA 深度解析, section 3.2 "收集-分发"):
    selected_A = A[idx], tmp = selected_A x, selected_B = B[idx],
    delta = selected_B tmp, Y = base + delta; the scale s_a is applied to
    delta per row.  Padding is zeroed first so r_max-wide products are valid."""
    keys, _ = validate_rows(row_slot, slot_rank, r_max)
    n_slots = len(slot_rank)
    X64 = decode(X, dtype)
    W64 = decode(W, dtype)
    A64, B64 = _adapters_zero_padded(A, B, slot_rank, r_max, dtype)
    idx = np.array([n_slots if k == -1 else k for k in keys], dtype=np.int64)
    s = np.array([0.0 if k == -1 else _scale(slot_alpha[k], int(slot_rank[k])) for k in keys])
    tmp = np.matmul(A64[idx], X64[:, :, None])[:, :, 0]          # [n, r_max]
    delta = np.matmul(B64[idx], tmp[:, :, None])[:, :, 0]        # [n, d_out]
    dY = s[:, None] * delta
    return X64 @ W64.T + dY, dY, tmp


def per_adapter_forward(X, W, A, B, row_slot, slot_rank, slot_alpha, r_max, dtype):
    """One base product for every row, then a masked low-rank product per
    distinct adapter (ybb.press multi-LoRA serving article, section 5.3
    "异质 LoRA 单 Batch 内核"), with the shapes in the adapter-batching
    page's convention: ax = X_a A_a^T, bax = ax B_a^T, out[mask] += s_a bax."""
    keys, _ = validate_rows(row_slot, slot_rank, r_max)
    X64 = decode(X, dtype)
    W64 = decode(W, dtype)
    base = X64 @ W64.T
    dY = np.zeros_like(base)
    karr = np.array(keys)
    for a in sorted(set(keys)):
        if a == -1:
            continue
        r = int(slot_rank[a])
        if r == 0:
            continue
        mask = karr == a
        Aa = decode(A[a, :r, :], dtype)
        Ba = decode(B[a, :, :r], dtype)
        ax = X64[mask] @ Aa.T
        dY[mask] += _scale(slot_alpha[a], r) * (ax @ Ba.T)
    return base + dY, dY


def merged_forward(X, W, A, B, row_slot, slot_rank, slot_alpha, r_max, dtype):
    """Merged form W'_a = W + s_a B_a A_a applied as a plain linear layer to
    the rows of adapter a (adapter-batching page, section "为什么单 Adapter
    可以 Merge"); base-only rows use W."""
    keys, _ = validate_rows(row_slot, slot_rank, r_max)
    X64 = decode(X, dtype)
    W64 = decode(W, dtype)
    Y = np.zeros((X64.shape[0], W64.shape[0]))
    karr = np.array(keys)
    for a in set(keys):
        mask = karr == a
        Wm = W64
        if a != -1 and int(slot_rank[a]) > 0:
            r = int(slot_rank[a])
            Wm = W64 + _scale(slot_alpha[a], r) * (decode(B[a, :, :r], dtype) @ decode(A[a, :r, :], dtype))
        Y[mask] = X64[mask] @ Wm.T
    return Y


# ---------------------------------------------------------------------------
# stacked projections (fused QKV, stacked gate/up)
# ---------------------------------------------------------------------------
def stacked_forward(X, Ws, As, Bs, row_slot, slot_rank, slot_alpha, r_max: int, dtype: str,
                    rows: Optional[Iterable[int]] = None):
    """Several target projections of one input (adapter-batching page,
    section "Adapter 不是一块连续 Weight": every target module has its own A
    and B, and a model with fused QKV or stacked gate/up runs them as one
    weight whose output concatenates the projections' outputs).  Projection
    p has base weight Ws[p] [d_out_p, d_in] and adapter pools As[p]
    [n_slots, r_max, d_in], Bs[p] [n_slots, d_out_p, r_max]; a slot's rank
    and scale are shared by its projections.  Returns (Y, dY, H) with Y and
    dY [rows, sum d_out_p] in projection order and H [rows, P * r_max]
    (projection p's ranks at columns [p r_max, (p + 1) r_max))."""
    outs = [lora_forward(X, W, A, B, row_slot, slot_rank, slot_alpha, r_max, dtype, rows=rows)
            for W, A, B in zip(Ws, As, Bs)]
    return (np.concatenate([o[0] for o in outs], axis=1),
            np.concatenate([o[1] for o in outs], axis=1),
            np.concatenate([o[2] for o in outs], axis=1))


# ---------------------------------------------------------------------------
# quantized base weight (FP8 E4M3 codes, one scale per output row)
# ---------------------------------------------------------------------------
# The adapter-batching page (section "Quantized Base Model 与 LoRA 的 Dtype
# 边界") lets the base weight be INT4/INT8/FP8 while A and B stay 16-bit, and
# asks where the two paths add; the multi-tenant serving article (section 1.2)
# dequantizes the base weight inside the kernel and keeps the alpha/r scaling
# there too.  Readings: the base weight is W[j, c] = w_scale[j] * e4m3(Wq[j,
# c]) with E4M3 as the OCP 8-bit floating point specification defines it;
# the LoRA branch takes the same (unquantized) activations X; the two paths
# add in full precision before the output is rounded once.
def decode_fp8_e4m3(codes) -> np.ndarray:
    """Exact float64 value of OCP FP8 E4M3 codes: 1 sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6;
    S.1111.111 is NaN; there are no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (m / 8.0) * np.exp2(-6.0)
    v = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)


def lora_forward_fp8w(X, Wq, w_scale, A, B, row_slot, slot_rank, slot_alpha, r_max: int,
                      dtype: str, rows: Optional[Iterable[int]] = None):
    """Y = X W^T + s_a (X_a A_a^T) B_a^T with the base weight given as E4M3
    codes and per-row scales: W = w_scale[:, None] * e4m3(Wq), in float64.
    The LoRA branch is ``lora_forward``'s (evaluated with a zero base weight,
    so it does not depend on W).  Returns (Y, dY, H) like ``lora_forward``."""
    d_out, d_in = np.shape(Wq)
    zero_w = np.zeros((d_out, d_in), dtype=np.uint16 if dtype == "bf16" else np.float32)
    _, dY, H = lora_forward(X, zero_w, A, B, row_slot, slot_rank, slot_alpha, r_max, dtype,
                            rows=rows)
    W64 = decode_fp8_e4m3(Wq) * np.asarray(w_scale, dtype=np.float64)[:, None]
    X64 = decode(X, dtype)
    n = X64.shape[0]
    rows = list(range(n)) if rows is None else [int(i) for i in rows]
    Xr = X64[rows] if rows else np.zeros((0, d_in))
    return Xr @ W64.T + dY, dY, H


# ---------------------------------------------------------------------------
# DoRA: magnitude times normalised direction
# ---------------------------------------------------------------------------
# The ybb.press multi-LoRA serving article, section 9.2 (DoRA), writes the
# adapted weight as a magnitude m times the direction W0 + BA divided by its
# norm ||W0 + BA||_c, applied at inference by one extra vector normalisation
# in a custom epilogue.  Readings (the page leaves them open):
#
# * the direction is the weight the layer applies, W0 + s_a B_a A_a (the
#   merged form of the adapter-batching page, "为什么单 Adapter 可以 Merge");
# * ||.||_c is the 2-norm of each output feature's weight vector, i.e. of
#   each row of the nn.Linear weight [d_out, d_in], so m_a has d_out entries
#   and the normalisation is a per-output-column factor (the only kind an
#   epilogue can apply);
# * an output feature whose direction row is exactly zero gets a zero row;
# * a slot without a magnitude vector (None) is a plain LoRA adapter, and
#   base-only rows and rank-0 slots keep the base weight W0.
def _direction(W64, A, B, slot_rank, slot_alpha, dtype, a):
    """V_a = W0 + s_a B_a A_a in float64 (W0 for a rank-0 slot)."""
    r = int(slot_rank[a])
    if r == 0:
        return W64.copy()
    return W64 + _scale(slot_alpha[a], r) * (decode(B[a, :, :r], dtype) @ decode(A[a, :r, :], dtype))


def dora_column_scale(W, A, B, slot_rank, slot_alpha, magnitude, dtype, a):
    """g_a[j] = m_a[j] / ||V_a[j, :]||_2 for every output feature j of slot a
    (0 where the norm is 0; all ones when the slot has no magnitude).  The
    DoRA output of a row on slot a is g_a times its plain LoRA output."""
    W64 = decode(W, dtype)
    if magnitude[a] is None:
        return np.ones(W64.shape[0])
    V = _direction(W64, A, B, slot_rank, slot_alpha, dtype, a)
    norm = np.sqrt(np.sum(V * V, axis=1))
    m = np.asarray(magnitude[a], dtype=np.float64)
    return np.where(norm > 0.0, m / np.where(norm > 0.0, norm, 1.0), 0.0)


def dora_forward(X, W, A, B, row_slot, slot_rank, slot_alpha, magnitude, r_max, dtype,
                 rows: Optional[Iterable[int]] = None):
    """DoRA layer by its definition: for every adapter a among the requested
    rows, build W'_a = m_a * V_a / ||V_a||_c row by row, then y_i = W'_a x_i
    for the rows on a.  Base-only rows, rank-0 slots and slots without a
    magnitude use W0 and W0 + s_a B_a A_a as the plain layer does.
    ``magnitude`` is a list over slots of float arrays [d_out] or None.
    Returns float64 Y for the requested rows, in request order."""
    X64 = decode(X, dtype)
    n = X64.shape[0]
    rows = list(range(n)) if rows is None else [int(i) for i in rows]
    keys, _ = validate_rows(row_slot, slot_rank, r_max)
    W64 = decode(W, dtype)
    Y = np.zeros((len(rows), W64.shape[0]))
    req = np.array([keys[i] for i in rows], dtype=np.int64)
    Xr = X64[rows] if rows else np.zeros((0, X64.shape[1]))
    for a in sorted(set(req.tolist())):
        mask = req == a
        if a == -1 or int(slot_rank[a]) == 0:
            Wp = W64
        else:
            V = _direction(W64, A, B, slot_rank, slot_alpha, dtype, a)
            if magnitude[a] is None:
                Wp = V
            else:
                m = np.asarray(magnitude[a], dtype=np.float64)
                Wp = np.zeros_like(V)
                for j in range(V.shape[0]):
                    nj = np.sqrt(np.dot(V[j], V[j]))
                    if nj > 0.0:
                        Wp[j] = m[j] * V[j] / nj
        Y[mask] = Xr[mask] @ Wp.T
    return Y


def dora_factored_forward(X, W, A, B, row_slot, slot_rank, slot_alpha, magnitude, r_max, dtype,
                          rows: Optional[Iterable[int]] = None):
    """The same layer in the order an epilogue applies it: the plain LoRA
    output y_i = W0 x_i + s_a B_a A_a x_i, then each output column j times
    g_a[j] (``dora_column_scale``) on rows of a slot of rank > 0.  Equal to
    ``dora_forward`` because the normalisation is a per-row factor of W'_a."""
    Y, _, _ = lora_forward(X, W, A, B, row_slot, slot_rank, slot_alpha, r_max, dtype, rows=rows)
    n = len(row_slot)
    rows = list(range(n)) if rows is None else [int(i) for i in rows]
    keys, _ = validate_rows(row_slot, slot_rank, r_max)
    cache = {}
    for t, i in enumerate(rows):
        a = keys[i]
        if a == -1 or int(slot_rank[a]) == 0:
            continue
        if a not in cache:
            cache[a] = dora_column_scale(W, A, B, slot_rank, slot_alpha, magnitude, dtype, a)
        Y[t] = Y[t] * cache[a]
    return Y


# ---------------------------------------------------------------------------
# parameter arithmetic
# ---------------------------------------------------------------------------
def lora_param_count(r: int, d_in: int, d_out: int) -> int:
    """P_LoRA = r (d_in + d_out) (adapter-batching page, "LoRA 在一层 Linear
    上增加了什么")."""
    return r * (d_in + d_out)


def full_param_count(d_in: int, d_out: int) -> int:
    """P_W = d_in d_out (same section)."""
    return d_in * d_out
