"""Segmented multi-LoRA linear layer for MI355X (gfx950): Python binding.

Thin ctypes layer over ``liblora.so`` (C ABI in ``include/lora.h``).  It only
marshals arguments: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the current HIP stream.

Entry points carry the C names:

* ``lora_build_segments(row_slot, pool, seg)``
* ``lora_shrink(X, seg, pool, H)``
* ``lora_expand(H, seg, pool, Y)``            (Y += ...)
* ``lora_base_gemm(X, W, Y)``                 (Y = X W^T)
* ``lora_linear_fused(X, W, H, seg, pool, Y)``  (Y = X W^T + LoRA)

If the library is missing the import still succeeds, but every entry point
raises ``RuntimeError``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblora.so")

LORA_F32, LORA_BF16 = 0, 1
RANK_EXACT, RANK_TWO_BUCKETS, RANK_PADDED = 0, 1, 2
RANK_POLICIES = {"exact": RANK_EXACT, "two_buckets": RANK_TWO_BUCKETS, "padded": RANK_PADDED}
MAX_SLOTS = 4095
ABI_VERSION = 9
STATIC_MAX_ROWS = 32768
STATIC_MAX_H = 1 << 21
LAYER_ONE_LAUNCH_ROWS = 512
LAYER_SYNC_BYTES = 4096

_c_int32_p = ctypes.POINTER(ctypes.c_int32)


class LoraPoolC(ctypes.Structure):
    _fields_ = [
        ("n_slots", ctypes.c_int32),
        ("r_max", ctypes.c_int32),
        ("d_in", ctypes.c_int32),
        ("d_out", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rank_policy", ctypes.c_int32),
        ("A", ctypes.c_void_p),
        ("Bt", ctypes.c_void_p),
        ("slot_rank", ctypes.c_void_p),
        ("slot_scale", ctypes.c_void_p),
        ("B", ctypes.c_void_p),
        ("dora_scale", ctypes.c_void_p),
        ("n_proj", ctypes.c_int32),
        ("proj_cols", ctypes.c_void_p),      # host int32 [n_proj + 1]
    ]


class LoraSegmentsC(ctypes.Structure):
    _fields_ = [
        ("n_rows", ctypes.c_int32),
        ("max_segments", ctypes.c_int32),
        ("token_indices", ctypes.c_void_p),
        ("row_segment", ctypes.c_void_p),
        ("segment_offsets", ctypes.c_void_p),
        ("segment_slots", ctypes.c_void_p),
        ("segment_ranks", ctypes.c_void_p),
        ("segment_scales", ctypes.c_void_p),
        ("num_segments", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
    ]


class LoraError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"liblora status {code}: {msg}")
        self.code = code


_lib = None

EXPORTS = (
    "lora_abi_version",
    "lora_status_str",
    "lora_build_segments",
    "lora_shrink",
    "lora_build_shrink",
    "lora_expand",
    "lora_pool_pack_slot",
    "lora_pool_set_scales",
    "lora_pool_write_b",
    "lora_pool_dora_prepare",
    "lora_base_gemm",
    "lora_linear_fused",
    "lora_base_gemm_fp8w",
    "lora_linear_fused_fp8w",
    "lora_linear_fused_static",
    "lora_layer_fused",
    "lora_layer_fused_fp8w",
)


def lib() -> ctypes.CDLL:
    """Load liblora.so (built by ``python -m segmented_rank_gemm_segment_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m segmented_rank_gemm_segment_amd.build` (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    PP, SP = ctypes.POINTER(LoraPoolC), ctypes.POINTER(LoraSegmentsC)
    L.lora_abi_version.restype = i32
    L.lora_abi_version.argtypes = []
    L.lora_status_str.restype = ctypes.c_char_p
    L.lora_status_str.argtypes = [i32]
    L.lora_build_segments.restype = i32
    L.lora_build_segments.argtypes = [vp, PP, SP, vp]
    L.lora_shrink.restype = i32
    L.lora_shrink.argtypes = [vp, i64, SP, PP, vp, vp]
    L.lora_build_shrink.restype = i32
    L.lora_build_shrink.argtypes = [vp, vp, i64, PP, SP, vp, vp]
    L.lora_expand.restype = i32
    L.lora_expand.argtypes = [vp, SP, PP, vp, i64, vp]
    L.lora_pool_pack_slot.restype = i32
    L.lora_pool_pack_slot.argtypes = [PP, i32, i32, ctypes.c_double, vp, vp, vp, vp, i32, vp]
    L.lora_pool_set_scales.restype = i32
    L.lora_pool_set_scales.argtypes = [PP, vp, vp]
    L.lora_pool_write_b.restype = i32
    L.lora_pool_write_b.argtypes = [PP, vp]
    L.lora_pool_dora_prepare.restype = i32
    L.lora_pool_dora_prepare.argtypes = [PP, i32, vp, i64, vp, vp]
    L.lora_base_gemm.restype = i32
    L.lora_base_gemm.argtypes = [vp, i64, vp, i64, vp, i64, i32, i32, i32, i32, vp]
    L.lora_linear_fused.restype = i32
    L.lora_linear_fused.argtypes = [vp, i64, vp, i64, vp, SP, PP, vp, i64, vp]
    L.lora_base_gemm_fp8w.restype = i32
    L.lora_base_gemm_fp8w.argtypes = [vp, i64, vp, i64, vp, vp, i64, i32, i32, i32, vp]
    L.lora_linear_fused_fp8w.restype = i32
    L.lora_linear_fused_fp8w.argtypes = [vp, i64, vp, i64, vp, vp, SP, PP, vp, i64, vp]
    L.lora_linear_fused_static.restype = i32
    L.lora_linear_fused_static.argtypes = [vp, vp, i64, vp, i64, PP, i32, vp, i64, vp]
    L.lora_layer_fused.restype = i32
    L.lora_layer_fused.argtypes = [vp, vp, i64, vp, i64, PP, SP, vp, vp, i64, vp, vp]
    L.lora_layer_fused_fp8w.restype = i32
    L.lora_layer_fused_fp8w.argtypes = [vp, vp, i64, vp, i64, vp, PP, SP, vp, vp, i64, vp, vp]
    if L.lora_abi_version() != ABI_VERSION:
        raise RuntimeError("liblora ABI version mismatch")
    _lib = L
    return L


def _check(code: int) -> None:
    if code != 0:
        raise LoraError(code, lib().lora_status_str(code).decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return LORA_BF16
    if t == torch.float32:
        return LORA_F32
    raise ValueError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ld(t: torch.Tensor) -> int:
    if t.dim() == 2 and t.numel() == 0:
        return max(int(t.shape[1]), 8)
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a row-major 2-D tensor")
    return t.stride(0)


# ---------------------------------------------------------------------------
# pool and metadata holders
# ---------------------------------------------------------------------------
class Pool:
    """Fixed-slot adapter pool resident on the device.

    ``A``  [n_slots, r_max, d_in]  and  ``Bt`` [n_slots, rs, d_out]
    (rank-major; row k of Bt[a] is column k of B_a; rs = r_max for one
    projection), ``slot_rank`` int32 [n_slots] and ``slot_scale`` float32
    [n_slots], which the library writes from the slots' alphas
    (lora_pool_set_scales, lora_pool_pack_slot).  With ``natural_b``
    (default) the pool also keeps B in its d_out-major layout, ``B``
    [n_slots, d_out, rs], for the fused GEMM (written by the library:
    lora_pool_write_b, lora_pool_pack_slot).  With ``dora`` it
    keeps DoRA column factors ``dora_scale`` float32 [n_slots, d_out], all
    ones (plain LoRA) until ``dora_prepare`` sets a slot's.  A pool of
    stacked projections (``empty(..., proj_outs=...)``, ``stacked``) serves
    several projections of one input; its ``proj_cols`` are the host column
    offsets, A holds the P projections' rank rows (r_max = P rs) and Bt each
    column's own projection in rs rank rows.  torch only allocates here:
    every value is written by liblora.
    """

    def __init__(self, A: torch.Tensor, Bt: torch.Tensor, slot_rank: torch.Tensor,
                 slot_alpha, rank_policy: str = "exact", natural_b: bool = True,
                 dora: bool = False, proj_outs=None, stream=None):
        P = len(proj_outs) if proj_outs is not None and len(proj_outs) >= 2 else 1
        if A.dim() != 3 or Bt.dim() != 3 or A.shape[0] != Bt.shape[0] \
                or A.shape[1] != P * Bt.shape[1]:
            raise ValueError("A [n_slots, P rs, d_in] and Bt [n_slots, rs, d_out] expected")
        if A.dtype != Bt.dtype or not A.is_contiguous() or not Bt.is_contiguous():
            raise ValueError("A and Bt: same dtype, contiguous")
        dev = A.device
        self.A, self.Bt = A, Bt
        self.n_slots, self.r_max, self.d_in = A.shape
        self.d_out = Bt.shape[2]
        self.dtype = A.dtype
        self.B = (torch.empty((self.n_slots, self.d_out, Bt.shape[1]), dtype=A.dtype, device=dev)
                  if natural_b else None)
        self.dora_scale = (torch.ones((self.n_slots, self.d_out), dtype=torch.float32, device=dev)
                           if dora else None)
        self.proj_cols = None             # stacked projections: host int32 column offsets
        if proj_outs is not None and len(proj_outs) >= 2:
            cols = [0]
            for c in proj_outs:
                cols.append(cols[-1] + int(c))
            if cols[-1] != self.d_out:
                raise ValueError("projection widths must add up to d_out")
            self.proj_cols = (ctypes.c_int32 * len(cols))(*cols)
        self.slot_rank = slot_rank.to(device=dev, dtype=torch.int32).contiguous()
        self.slot_scale = torch.empty(self.n_slots, dtype=torch.float32, device=dev)
        alpha = torch.as_tensor(slot_alpha, dtype=torch.float64).reshape(-1)
        if alpha.numel() == 1:
            alpha = alpha.expand(self.n_slots)
        if alpha.numel() != self.n_slots:
            raise ValueError("slot_alpha: one value or one per slot")
        self.slot_alpha = alpha.clone()   # host copy of each slot's alpha (bookkeeping)
        self.generation = [0] * self.n_slots
        self.set_policy(rank_policy)
        st = torch.cuda.current_stream(dev) if stream is None else stream
        alpha_d = alpha.contiguous().to(dev)
        with torch.cuda.stream(st):
            _check(lib().lora_pool_set_scales(self.c, _ptr(alpha_d), _stream(st)))
            if self.B is not None:
                _check(lib().lora_pool_write_b(self.c, _stream(st)))
        alpha_d.record_stream(st)         # alive until the queued kernel has read it

    @classmethod
    def empty(cls, n_slots: int, r_max: int, d_in: int, d_out: int, dtype=torch.bfloat16,
              device="cuda", rank_policy: str = "exact", natural_b: bool = True,
              dora: bool = False, proj_outs=None) -> "Pool":
        """A pool of empty slots (rank 0, zero weights), filled by ``pack``.
        ``proj_outs``: output widths of stacked projections (r_max is then
        the per-projection rank bound, the pool's being len(proj_outs)
        times it)."""
        P = len(proj_outs) if proj_outs is not None and len(proj_outs) >= 2 else 1
        if P > 1:
            d_out = sum(int(c) for c in proj_outs)
        A = torch.zeros((n_slots, P * r_max, d_in), dtype=dtype, device=device)
        Bt = torch.zeros((n_slots, r_max, d_out), dtype=dtype, device=device)
        rank = torch.zeros(n_slots, dtype=torch.int32, device=device)
        return cls(A, Bt, rank, 0.0, rank_policy, natural_b, dora,
                   proj_outs=proj_outs if P > 1 else None)

    @property
    def n_proj(self) -> int:
        return 1 if self.proj_cols is None else len(self.proj_cols) - 1

    def _on_device(self, t: torch.Tensor) -> torch.Tensor:
        dev = self.A.device
        t = t.to(dtype=self.dtype)
        if t.device != dev:
            t = t.contiguous()
            if t.device.type == "cpu":
                t = t.pin_memory()
            t = t.to(dev, non_blocking=True)
        return t.contiguous()

    def pack(self, slot: int, A, B, alpha: float, stream=None, b_layout: str = "rows") -> int:
        """Load one adapter into ``slot`` through lora_pool_pack_slot: A and B
        are one tensor each (A [r, d_in], B [d_out, r], the layouts of the
        adapter's own weights) or, for a stacked pool, lists with one per
        projection; ``b_layout="rank_rows"`` takes B transposed ([r,
        d_out_q]).  The library stores scale alpha / r.  Host tensors are
        copied over first (from pinned memory, asynchronously).  Returns the
        slot's new generation.  r = 0 (A [0, d_in]) empties the slot."""
        As = list(A) if isinstance(A, (list, tuple)) else [A]
        Bs = list(B) if isinstance(B, (list, tuple)) else [B]
        P = self.n_proj
        if len(As) != P or len(Bs) != P:
            raise ValueError(f"{P} projection(s): one A and one B each")
        r = int(As[0].shape[0])
        cols = [self.d_out] if P == 1 else [self.proj_cols[q + 1] - self.proj_cols[q]
                                             for q in range(P)]
        rank_rows = b_layout == "rank_rows"
        for q in range(P):
            want_b = (r, cols[q]) if rank_rows else (cols[q], r)
            if As[q].dim() != 2 or tuple(As[q].shape) != (r, self.d_in) \
                    or tuple(Bs[q].shape) != want_b:
                raise ValueError("A [r, d_in] and B [d_out_q, r] (or [r, d_out_q]) per projection")
        st = torch.cuda.current_stream(self.A.device) if stream is None else stream
        keep = []
        if r > 0:
            Ad = [self._on_device(t) for t in As]
            Bd = [self._on_device(t) for t in Bs]
            keep = Ad + Bd
            a_ptrs = (ctypes.c_void_p * P)(*[t.data_ptr() for t in Ad])
            b_ptrs = (ctypes.c_void_p * P)(*[t.data_ptr() for t in Bd])
            ldas = (ctypes.c_int64 * P)(*[_ld(t) for t in Ad])
            ldbs = (ctypes.c_int64 * P)(*[_ld(t) for t in Bd])
        else:
            a_ptrs = b_ptrs = ldas = ldbs = None
        with torch.cuda.stream(st):
            _check(lib().lora_pool_pack_slot(self.c, int(slot), r, float(alpha), a_ptrs, ldas,
                                             b_ptrs, ldbs, 1 if rank_rows else 0, _stream(st)))
        for t in keep:                    # the copies stay alive until the kernels read them
            t.record_stream(st)
        self.slot_alpha[slot] = float(alpha)
        self.generation[slot] += 1
        return self.generation[slot]

    def dora_prepare(self, slot: int, W: torch.Tensor, magnitude: Optional[torch.Tensor] = None,
                     stream=None) -> None:
        """DoRA column factors of ``slot`` from its current weights and the
        base weight W [d_out, d_in] (lora_pool_dora_prepare):
        g[j] = magnitude[j] / ||W[j] + s (B A)[j]||, or all ones for
        magnitude None.  Queue it after ``pack`` on the same stream."""
        if self.dora_scale is None:
            raise ValueError("pool was created without dora=True")
        dev = self.A.device
        st = torch.cuda.current_stream(dev) if stream is None else stream
        m = None
        if magnitude is not None:
            if tuple(magnitude.shape) != (self.d_out,):
                raise ValueError("magnitude [d_out] expected")
            m = magnitude.to(device=dev, dtype=torch.float32).contiguous()
        with torch.cuda.stream(st):
            _check(lib().lora_pool_dora_prepare(self.c, int(slot), _ptr(W), _ld(W), _ptr(m),
                                                _stream(st)))
        if m is not None and m is not magnitude:
            m.record_stream(st)           # a copy made here: alive until read

    @classmethod
    def stacked(cls, pools, rank_policy: str = "exact", natural_b: bool = True,
                dora: bool = False, slot_alpha=None) -> "Pool":
        """One pool serving several projections of the same input (fused QKV,
        stacked gate/up), packed slot by slot by lora_pool_pack_slot from the
        projections' pools (which must agree on slots, r_max, d_in, dtype and
        slot ranks; a slot's alpha is pools[0]'s unless ``slot_alpha`` is
        given).  The output columns are the projections' in order."""
        p0 = pools[0]
        P = len(pools)
        if not 2 <= P <= 8:
            raise ValueError("2..8 projections")
        for p in pools:
            if (p.n_slots, p.r_max, p.d_in, p.dtype) != (p0.n_slots, p0.r_max, p0.d_in, p0.dtype):
                raise ValueError("projections must share n_slots, r_max, d_in and dtype")
            if not torch.equal(p.slot_rank, p0.slot_rank):
                raise ValueError("projections must share slot ranks")
        alpha = p0.slot_alpha if slot_alpha is None else \
            torch.as_tensor(slot_alpha, dtype=torch.float64).reshape(-1).expand(p0.n_slots)
        obj = cls.empty(p0.n_slots, p0.r_max, p0.d_in, 0, dtype=p0.dtype, device=p0.A.device,
                        rank_policy=rank_policy, natural_b=natural_b, dora=dora,
                        proj_outs=[p.d_out for p in pools])
        ranks = p0.slot_rank.cpu().tolist()
        for a, r in enumerate(ranks):
            if 0 < r <= p0.r_max:
                obj.pack(a, [p.A[a, :r] for p in pools], [p.Bt[a, :r] for p in pools],
                         float(alpha[a]), b_layout="rank_rows")
            elif r != 0:
                raise ValueError(f"slot {a}: rank {r} outside [0, r_max]")
        return obj

    def set_policy(self, rank_policy: str):
        self.rank_policy = rank_policy
        P = 0 if self.proj_cols is None else len(self.proj_cols) - 1
        self._c = LoraPoolC(self.n_slots, self.r_max, self.d_in, self.d_out, _dtype_code(self.dtype),
                            RANK_POLICIES[rank_policy], self.A.data_ptr(), self.Bt.data_ptr(),
                            self.slot_rank.data_ptr(), self.slot_scale.data_ptr(),
                            self.B.data_ptr() if self.B is not None else None,
                            self.dora_scale.data_ptr() if self.dora_scale is not None else None,
                            P, ctypes.cast(self.proj_cols, ctypes.c_void_p) if P else None)
        return self

    @property
    def c(self):
        return ctypes.byref(self._c)


class Segments:
    """Device arrays of the segment metadata for a batch of n_rows rows."""

    def __init__(self, n_rows: int, n_slots: int, device, max_segments: Optional[int] = None):
        cap = min(n_rows, n_slots + 1) if max_segments is None else max_segments
        i32 = dict(dtype=torch.int32, device=device)
        self.n_rows = n_rows
        self.max_segments = cap
        self.token_indices = torch.empty(max(n_rows, 1), **i32)
        self.row_segment = torch.empty(max(n_rows, 1), **i32)
        self.segment_offsets = torch.empty(cap + 1, **i32)
        self.segment_slots = torch.empty(max(cap, 1), **i32)
        self.segment_ranks = torch.empty(max(cap, 1), **i32)
        self.segment_scales = torch.empty(max(cap, 1), dtype=torch.float32, device=device)
        self.num_segments = torch.empty(1, **i32)
        self.status = torch.empty(1, **i32)
        self._c = LoraSegmentsC(n_rows, cap, self.token_indices.data_ptr(),
                                self.row_segment.data_ptr(), self.segment_offsets.data_ptr(),
                                self.segment_slots.data_ptr(), self.segment_ranks.data_ptr(),
                                self.segment_scales.data_ptr(), self.num_segments.data_ptr(),
                                self.status.data_ptr())

    @property
    def c(self):
        return ctypes.byref(self._c)

    def to_host(self) -> dict:
        """Metadata as numpy arrays (synchronises)."""
        S = int(self.num_segments.item())
        return {
            "num_segments": S,
            "segment_offsets": self.segment_offsets[:S + 1].cpu().numpy(),
            "segment_slots": self.segment_slots[:S].cpu().numpy(),
            "segment_ranks": self.segment_ranks[:S].cpu().numpy(),
            "segment_scales": self.segment_scales[:S].cpu().numpy(),
            "token_indices": self.token_indices[:self.n_rows].cpu().numpy(),
            "row_segment": self.row_segment[:self.n_rows].cpu().numpy(),
            "status": int(self.status.item()),
        }


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def lora_build_segments(row_slot: torch.Tensor, pool: Pool, seg: Segments, stream=None) -> None:
    if row_slot.dtype != torch.int32 or (row_slot.numel() and not row_slot.is_contiguous()):
        raise ValueError("row_slot: contiguous int32")
    if row_slot.numel() != seg.n_rows:
        raise ValueError("row_slot length != seg.n_rows")
    _check(lib().lora_build_segments(_ptr(row_slot), pool.c, seg.c, _stream(stream)))


def lora_shrink(X: torch.Tensor, seg: Segments, pool: Pool, H: torch.Tensor, stream=None) -> None:
    if H.dtype != torch.float32 or tuple(H.shape) != (seg.n_rows, pool.r_max) or not H.is_contiguous():
        raise ValueError("H: contiguous float32 [n_rows, r_max]")
    if X.shape[0] != seg.n_rows or X.dtype != pool.dtype:
        raise ValueError("X: [n_rows, d_in] of the pool dtype")
    _check(lib().lora_shrink(_ptr(X), _ld(X), seg.c, pool.c, _ptr(H), _stream(stream)))


def lora_build_shrink(row_slot: torch.Tensor, X: torch.Tensor, pool: Pool, seg: Segments,
                      H: torch.Tensor, stream=None) -> None:
    """lora_build_segments followed by lora_shrink, in one launch for
    decode-sized batches."""
    if row_slot.dtype != torch.int32 or (row_slot.numel() and not row_slot.is_contiguous()):
        raise ValueError("row_slot: contiguous int32")
    if row_slot.numel() != seg.n_rows:
        raise ValueError("row_slot length != seg.n_rows")
    if H.dtype != torch.float32 or tuple(H.shape) != (seg.n_rows, pool.r_max) or not H.is_contiguous():
        raise ValueError("H: contiguous float32 [n_rows, r_max]")
    if X.shape[0] != seg.n_rows or X.dtype != pool.dtype:
        raise ValueError("X: [n_rows, d_in] of the pool dtype")
    _check(lib().lora_build_shrink(_ptr(row_slot), _ptr(X), _ld(X), pool.c, seg.c, _ptr(H),
                                   _stream(stream)))


def lora_expand(H: torch.Tensor, seg: Segments, pool: Pool, Y: torch.Tensor, stream=None) -> None:
    if H.dtype != torch.float32 or tuple(H.shape) != (seg.n_rows, pool.r_max) or not H.is_contiguous():
        raise ValueError("H: contiguous float32 [n_rows, r_max]")
    if Y.shape[0] != seg.n_rows or Y.dtype != pool.dtype:
        raise ValueError("Y: [n_rows, d_out] of the pool dtype")
    _check(lib().lora_expand(_ptr(H), seg.c, pool.c, _ptr(Y), _ld(Y), _stream(stream)))


def lora_base_gemm(X: torch.Tensor, W: torch.Tensor, Y: torch.Tensor, stream=None) -> None:
    if not (X.dtype == W.dtype == Y.dtype):
        raise ValueError("X, W, Y must share a dtype")
    n, d_in = X.shape
    d_out = W.shape[0]
    if W.shape[1] != d_in or tuple(Y.shape) != (n, d_out):
        raise ValueError("shapes: X [n, d_in], W [d_out, d_in], Y [n, d_out]")
    _check(lib().lora_base_gemm(_ptr(X), _ld(X), _ptr(W), _ld(W), _ptr(Y), _ld(Y), n, d_in, d_out,
                                _dtype_code(X.dtype), _stream(stream)))


def lora_linear_fused(X: torch.Tensor, W: torch.Tensor, H: torch.Tensor, seg: Segments, pool: Pool,
                      Y: torch.Tensor, stream=None) -> None:
    if not (X.dtype == W.dtype == Y.dtype == pool.dtype):
        raise ValueError("X, W, Y must share the pool dtype")
    if X.shape[0] != seg.n_rows or tuple(W.shape) != (pool.d_out, pool.d_in) \
            or tuple(Y.shape) != (seg.n_rows, pool.d_out):
        raise ValueError("shapes: X [n, d_in], W [d_out, d_in], Y [n, d_out]")
    if H.dtype != torch.float32 or tuple(H.shape) != (seg.n_rows, pool.r_max) or not H.is_contiguous():
        raise ValueError("H: contiguous float32 [n_rows, r_max]")
    _check(lib().lora_linear_fused(_ptr(X), _ld(X), _ptr(W), _ld(W), _ptr(H), seg.c, pool.c,
                                   _ptr(Y), _ld(Y), _stream(stream)))


def layer_sync(device) -> torch.Tensor:
    """A zero-filled sync buffer for lora_layer_fused (LAYER_SYNC_BYTES)."""
    return torch.zeros(LAYER_SYNC_BYTES // 4, dtype=torch.int32, device=device)


def lora_layer_fused(row_slot: torch.Tensor, X: torch.Tensor, W: torch.Tensor, pool: Pool,
                     seg: Segments, H: torch.Tensor, Y: torch.Tensor,
                     sync: Optional[torch.Tensor] = None, stream=None) -> None:
    """Segment build, shrink and fused product in one call (one launch for
    bf16 batches of up to LAYER_ONE_LAUNCH_ROWS rows).  sync: a buffer from
    layer_sync(), reused across calls ordered on one stream; None makes
    every tile compute its own rows' H."""
    if row_slot.dtype != torch.int32 or (row_slot.numel() and not row_slot.is_contiguous()):
        raise ValueError("row_slot: contiguous int32")
    if row_slot.numel() != seg.n_rows:
        raise ValueError("row_slot length != seg.n_rows")
    if not (X.dtype == W.dtype == Y.dtype == pool.dtype):
        raise ValueError("X, W, Y must share the pool dtype")
    if X.shape[0] != seg.n_rows or tuple(W.shape) != (pool.d_out, pool.d_in) \
            or tuple(Y.shape) != (seg.n_rows, pool.d_out):
        raise ValueError("shapes: X [n, d_in], W [d_out, d_in], Y [n, d_out]")
    if H.dtype != torch.float32 or tuple(H.shape) != (seg.n_rows, pool.r_max) or not H.is_contiguous():
        raise ValueError("H: contiguous float32 [n_rows, r_max]")
    if sync is not None and (sync.numel() * sync.element_size() < LAYER_SYNC_BYTES
                             or not sync.is_contiguous()):
        raise ValueError("sync: a contiguous buffer of LAYER_SYNC_BYTES bytes (layer_sync())")
    _check(lib().lora_layer_fused(_ptr(row_slot), _ptr(X), _ld(X), _ptr(W), _ld(W), pool.c, seg.c,
                                  _ptr(H), _ptr(Y), _ld(Y), _ptr(sync), _stream(stream)))


def lora_layer_fused_fp8w(row_slot: torch.Tensor, X: torch.Tensor, Wq: torch.Tensor,
                          w_scale: torch.Tensor, pool: Pool, seg: Segments, H: torch.Tensor,
                          Y: torch.Tensor, sync: Optional[torch.Tensor] = None,
                          stream=None) -> None:
    """lora_layer_fused with the FP8 E4M3 base weight (Wq uint8 codes
    [d_out, d_in], w_scale float32 [d_out])."""
    if row_slot.dtype != torch.int32 or (row_slot.numel() and not row_slot.is_contiguous()):
        raise ValueError("row_slot: contiguous int32")
    if row_slot.numel() != seg.n_rows:
        raise ValueError("row_slot length != seg.n_rows")
    if not (X.dtype == Y.dtype == pool.dtype == torch.bfloat16):
        raise ValueError("X and Y must be bf16, as the pool")
    if Wq.dtype != torch.uint8 or w_scale.dtype != torch.float32 or not w_scale.is_contiguous():
        raise ValueError("Wq uint8 E4M3 codes, w_scale contiguous float32")
    if X.shape[0] != seg.n_rows or tuple(Wq.shape) != (pool.d_out, pool.d_in) \
            or tuple(Y.shape) != (seg.n_rows, pool.d_out) or w_scale.numel() != pool.d_out:
        raise ValueError("shapes: X [n, d_in], Wq [d_out, d_in], w_scale [d_out], Y [n, d_out]")
    if H.dtype != torch.float32 or tuple(H.shape) != (seg.n_rows, pool.r_max) or not H.is_contiguous():
        raise ValueError("H: contiguous float32 [n_rows, r_max]")
    if sync is not None and (sync.numel() * sync.element_size() < LAYER_SYNC_BYTES
                             or not sync.is_contiguous()):
        raise ValueError("sync: a contiguous buffer of LAYER_SYNC_BYTES bytes (layer_sync())")
    _check(lib().lora_layer_fused_fp8w(_ptr(row_slot), _ptr(X), _ld(X), _ptr(Wq), _ld(Wq),
                                       _ptr(w_scale), pool.c, seg.c, _ptr(H), _ptr(Y), _ld(Y),
                                       _ptr(sync), _stream(stream)))


def lora_base_gemm_fp8w(X: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor, Y: torch.Tensor,
                        stream=None) -> None:
    """Y = X (w_scale * e4m3(Wq))^T with Wq uint8 E4M3 codes [d_out, d_in]
    and w_scale float32 [d_out]; X, Y bf16."""
    if X.dtype != torch.bfloat16 or Y.dtype != torch.bfloat16:
        raise ValueError("X and Y must be bf16")
    if Wq.dtype != torch.uint8 or w_scale.dtype != torch.float32 or not w_scale.is_contiguous():
        raise ValueError("Wq uint8 E4M3 codes, w_scale contiguous float32")
    n, d_in = X.shape
    d_out = Wq.shape[0]
    if Wq.shape[1] != d_in or tuple(Y.shape) != (n, d_out) or w_scale.numel() != d_out:
        raise ValueError("shapes: X [n, d_in], Wq [d_out, d_in], w_scale [d_out], Y [n, d_out]")
    _check(lib().lora_base_gemm_fp8w(_ptr(X), _ld(X), _ptr(Wq), _ld(Wq), _ptr(w_scale), _ptr(Y),
                                     _ld(Y), n, d_in, d_out, _stream(stream)))


def lora_linear_fused_fp8w(X: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor,
                           H: torch.Tensor, seg: Segments, pool: Pool, Y: torch.Tensor,
                           stream=None) -> None:
    """lora_linear_fused with the FP8 E4M3 base weight (Wq, w_scale)."""
    if Wq.dtype != torch.uint8 or w_scale.dtype != torch.float32 or not w_scale.is_contiguous():
        raise ValueError("Wq uint8 E4M3 codes, w_scale contiguous float32")
    if tuple(Wq.shape) != (pool.d_out, pool.d_in) or w_scale.numel() != pool.d_out:
        raise ValueError("Wq [d_out, d_in], w_scale [d_out]")
    if H.dtype != torch.float32 or tuple(H.shape) != (seg.n_rows, pool.r_max):
        raise ValueError("H: float32 [n_rows, r_max]")
    _check(lib().lora_linear_fused_fp8w(_ptr(X), _ld(X), _ptr(Wq), _ld(Wq), _ptr(w_scale), _ptr(H),
                                        seg.c, pool.c, _ptr(Y), _ld(Y), _stream(stream)))


def lora_linear_fused_static(row_slot: torch.Tensor, X: torch.Tensor, W: torch.Tensor, pool: Pool,
                             Y: torch.Tensor, stream=None) -> None:
    """The whole layer, Y = X W^T + LoRA, with the segment metadata and H in
    the library's static device scratch (no workspace, nothing allocated);
    the same bits as lora_build_shrink followed by lora_linear_fused.  Calls
    that overlap on one GPU race on that scratch."""
    if row_slot.dtype != torch.int32 or (row_slot.numel() and not row_slot.is_contiguous()):
        raise ValueError("row_slot: contiguous int32")
    n = row_slot.numel()
    if not (X.dtype == W.dtype == Y.dtype == pool.dtype):
        raise ValueError("X, W, Y must share the pool dtype")
    if X.shape[0] != n or tuple(W.shape) != (pool.d_out, pool.d_in) \
            or tuple(Y.shape) != (n, pool.d_out):
        raise ValueError("shapes: row_slot [n], X [n, d_in], W [d_out, d_in], Y [n, d_out]")
    _check(lib().lora_linear_fused_static(_ptr(row_slot), _ptr(X), _ld(X), _ptr(W), _ld(W), pool.c,
                                          n, _ptr(Y), _ld(Y), _stream(stream)))
