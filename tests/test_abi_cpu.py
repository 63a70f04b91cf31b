"""C ABI checks that need no GPU: the library loads, exports every function
that include/lora.h declares, and rejects bad arguments on the host before
any HIP call (so nothing here launches a kernel)."""
import ctypes
import os
import re
import subprocess

import pytest

import segmented_rank_gemm_segment_amd as srg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")

OK, ENULL, ESHAPE, ERANK, EALIGN, EDTYPE, ECAP, EHIP, EPOLICY, ESCRATCH = (0, -1, -2, -3, -4, -5,
                                                                   -6, -7, -8, -9)


@pytest.fixture(scope="session")
def L():
    if not os.path.exists(srg.LIB_PATH):
        from segmented_rank_gemm_segment_amd import build
        build.build()
    return srg.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(lora_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("lora_build_segments", "lora_shrink", "lora_expand", "lora_linear_fused",
              "lora_base_gemm", "lora_pool_pack_slot", "lora_pool_dora_prepare", "lora_build_shrink",
              "lora_base_gemm_fp8w", "lora_linear_fused_fp8w", "lora_status_str",
              "lora_abi_version", "lora_linear_fused_static", "lora_pool_set_scales",
              "lora_pool_write_b", "lora_layer_fused", "lora_layer_fused_fp8w"):
        assert n in names
    assert set(names) == set(srg.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", srg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(L, n)


def test_abi_version_and_status_strings(L):
    assert L.lora_abi_version() == srg.ABI_VERSION == 9
    for code in (OK, ENULL, ESHAPE, ERANK, EALIGN, EDTYPE, ECAP, EHIP, EPOLICY, ESCRATCH):
        s = L.lora_status_str(code).decode()
        assert s and s != "unknown status"
    assert L.lora_status_str(12345).decode() == "unknown status"


# fake, 16-byte aligned addresses: validation never dereferences them
P = 0x10000


def pool(**kw):
    d = dict(n_slots=4, r_max=16, d_in=64, d_out=32, dtype=1, rank_policy=0,
             A=P, Bt=P + 0x1000, slot_rank=P + 0x2000, slot_scale=P + 0x3000)
    d.update(kw)
    return srg.LoraPoolC(**d)


def segs(**kw):
    d = dict(n_rows=10, max_segments=5, token_indices=P + 0x4000, row_segment=P + 0x5000,
             segment_offsets=P + 0x6000, segment_slots=P + 0x7000, segment_ranks=P + 0x8000,
             segment_scales=P + 0x9000, num_segments=P + 0xA000, status=P + 0xB000)
    d.update(kw)
    return srg.LoraSegmentsC(**d)


def shrink(L, p, s, X=P + 0xC000, ldx=64, H=P + 0xD000):
    return L.lora_shrink(X, ldx, ctypes.byref(s), ctypes.byref(p), H, None)


@pytest.mark.parametrize("kw,code", [
    (dict(r_max=12), ERANK),
    (dict(r_max=128), ERANK),
    (dict(dtype=7), EDTYPE),
    (dict(rank_policy=3), EPOLICY),
    (dict(n_slots=0), ESHAPE),
    (dict(n_slots=4096), ESHAPE),
    (dict(d_in=0), ESHAPE),
    (dict(d_in=60), EALIGN),
    (dict(d_out=36), EALIGN),
    (dict(A=0), ENULL),
    (dict(slot_scale=0), ENULL),
    (dict(Bt=P + 8), EALIGN),
    (dict(dora_scale=P + 4), EALIGN),
])
def test_pool_validation(L, kw, code):
    assert shrink(L, pool(**kw), segs()) == code
    assert L.lora_build_segments(P, ctypes.byref(pool(**kw)), ctypes.byref(segs()), None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(n_rows=-1), ESHAPE),
    (dict(max_segments=4), ECAP),           # worst case min(10, 4 + 1) = 5
    (dict(token_indices=0), ENULL),
    (dict(num_segments=0), ENULL),
    (dict(status=0), ENULL),
])
def test_segment_validation(L, kw, code):
    assert shrink(L, pool(), segs(**kw)) == code


def test_capacity_bound_uses_rows_when_fewer():
    # 3 rows can make at most 3 segments even with 4 slots + base
    assert srg.lib().lora_shrink(P + 0xC000, 64, ctypes.byref(segs(n_rows=3, max_segments=2)),
                                 ctypes.byref(pool()), P, None) == ECAP


@pytest.mark.parametrize("kw,code", [
    (dict(X=0), ENULL),
    (dict(X=P + 4), EALIGN),
    (dict(ldx=60), ESHAPE),
    (dict(ldx=68), EALIGN),
    (dict(H=0), ENULL),
    (dict(H=P + 8), EALIGN),
])
def test_shrink_matrix_validation(L, kw, code):
    assert shrink(L, pool(), segs(), **kw) == code


def test_empty_batch_is_a_noop_without_launch(L):
    s = segs(n_rows=0, max_segments=0, token_indices=0, row_segment=0)
    assert shrink(L, pool(), s, X=0, H=0) == OK
    assert L.lora_expand(0, ctypes.byref(s), ctypes.byref(pool()), 0, 32, None) == OK
    assert L.lora_linear_fused(0, 64, P, 64, 0, ctypes.byref(s), ctypes.byref(pool()), 0, 32,
                               None) == OK
    assert L.lora_base_gemm(0, 64, P, 64, 0, 32, 0, 64, 32, 1, None) == OK


def _arr(kind, *vals):
    return (kind * len(vals))(*vals)


def test_pack_slot_validation(L):
    """Every bad argument is rejected on the host (nothing is launched)."""
    p = ctypes.byref(pool())                        # 4 slots, r_max 16, d_in 64, d_out 32
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    A, B = _arr(vp, P + 0xC000), _arr(vp, P + 0xD000)
    la, lb = _arr(i64, 64), _arr(i64, 8)
    pack = L.lora_pool_pack_slot
    assert pack(None, 0, 8, 16.0, A, la, B, lb, 0, None) == ENULL
    assert pack(p, -1, 8, 16.0, A, la, B, lb, 0, None) == ESHAPE
    assert pack(p, 4, 8, 16.0, A, la, B, lb, 0, None) == ESHAPE
    assert pack(p, 0, 17, 16.0, A, la, B, _arr(i64, 17), 0, None) == ESHAPE
    assert pack(p, 0, -1, 16.0, A, la, B, lb, 0, None) == ESHAPE
    assert pack(p, 0, 8, 16.0, A, la, B, lb, 2, None) == ESHAPE        # unknown B layout
    assert pack(p, 0, 8, 16.0, None, la, B, lb, 0, None) == ENULL
    assert pack(p, 0, 8, 16.0, A, None, B, lb, 0, None) == ENULL
    assert pack(p, 0, 8, 16.0, _arr(vp, 0), la, B, lb, 0, None) == ENULL
    assert pack(p, 0, 8, 16.0, A, la, None, lb, 0, None) == ENULL
    assert pack(p, 0, 8, 16.0, A, la, _arr(vp, 0), lb, 0, None) == ENULL
    assert pack(p, 0, 8, 16.0, A, _arr(i64, 56), B, lb, 0, None) == ESHAPE   # lda < d_in
    assert pack(p, 0, 8, 16.0, A, _arr(i64, 68), B, lb, 0, None) == EALIGN   # lda % 8
    assert pack(p, 0, 8, 16.0, _arr(vp, P + 0xC004), la, B, lb, 0, None) == EALIGN
    assert pack(p, 0, 8, 16.0, A, la, B, _arr(i64, 7), 0, None) == ESHAPE    # ldb < rank
    assert pack(p, 0, 8, 16.0, A, la, B, _arr(i64, 31), 1, None) == ESHAPE   # ldb < d_out (B^T)
    assert pack(ctypes.byref(pool(A=0)), 0, 8, 16.0, A, la, B, lb, 0, None) == ENULL


def test_set_scales_and_write_b_validation(L):
    p = ctypes.byref(pool())
    assert L.lora_pool_set_scales(None, P, None) == ENULL
    assert L.lora_pool_set_scales(p, None, None) == ENULL
    assert L.lora_pool_set_scales(p, P + 4, None) == EALIGN              # double array
    assert L.lora_pool_set_scales(ctypes.byref(pool(dtype=7)), P, None) == EDTYPE
    assert L.lora_pool_write_b(p, None) == ENULL                         # pool without B
    assert L.lora_pool_write_b(ctypes.byref(pool(B=P + 0x4008)), None) == EALIGN


def test_dora_prepare_validation(L):
    """Every bad argument is rejected on the host (nothing is launched)."""
    W = P + 0xC000
    p = ctypes.byref(pool(dora_scale=P + 0xE000))      # 4 slots, d_in 64, d_out 32
    prep = L.lora_pool_dora_prepare
    assert prep(None, 0, W, 64, P, None) == ENULL
    assert prep(ctypes.byref(pool()), 0, W, 64, P, None) == ENULL      # pool without factors
    assert prep(p, -1, W, 64, P, None) == ESHAPE
    assert prep(p, 4, W, 64, P, None) == ESHAPE
    assert prep(p, 0, None, 64, P, None) == ENULL
    assert prep(p, 0, W, 56, P, None) == ESHAPE                        # ldw < d_in
    assert prep(p, 0, W, 68, P, None) == EALIGN                        # ldw % 8
    assert prep(p, 0, W + 8, 64, P, None) == EALIGN
    assert prep(p, 0, W, 64, P + 2, None) == EALIGN                    # magnitude
    assert prep(ctypes.byref(pool(dora_scale=P + 4)), 0, W, 64, P, None) == EALIGN
    assert prep(ctypes.byref(pool(r_max=12, dora_scale=P)), 0, W, 64, P, None) == ERANK


def test_build_shrink_validation(L):
    """The one-call build + shrink rejects what either call rejects."""
    bs = L.lora_build_shrink
    X, H = P + 0xC000, P + 0xD000
    assert bs(P, X, 64, ctypes.byref(pool(r_max=12)), ctypes.byref(segs()), H, None) == ERANK
    assert bs(P, X, 64, ctypes.byref(pool()), ctypes.byref(segs(max_segments=4)), H, None) == ECAP
    assert bs(None, X, 64, ctypes.byref(pool()), ctypes.byref(segs()), H, None) == ENULL
    assert bs(P, None, 64, ctypes.byref(pool()), ctypes.byref(segs()), H, None) == ENULL
    assert bs(P, X, 60, ctypes.byref(pool()), ctypes.byref(segs()), H, None) == ESHAPE
    assert bs(P, X + 4, 64, ctypes.byref(pool()), ctypes.byref(segs()), H, None) == EALIGN
    assert bs(P, X, 64, ctypes.byref(pool()), ctypes.byref(segs()), None, None) == ENULL
    assert bs(P, X, 64, ctypes.byref(pool()), ctypes.byref(segs()), H + 8, None) == EALIGN


def test_fp8_weight_validation(L):
    """FP8-weight calls: bf16 only, d_in % 16, 16-byte aligned codes, rows
    and scales; checked on the host before any launch."""
    W, S, X, Y, H = P + 0xC000, P + 0xC800, P + 0xD000, P + 0xE000, P + 0xF000
    g = L.lora_base_gemm_fp8w
    assert g(X, 64, W, 64, S, Y, 32, -1, 64, 32, None) == ESHAPE
    assert g(X, 48, W, 48, S, Y, 32, 10, 40, 32, None) == EALIGN        # d_in % 16
    assert g(X, 64, None, 64, S, Y, 32, 10, 64, 32, None) == ENULL
    assert g(X, 64, W, 64, None, Y, 32, 10, 64, 32, None) == ENULL
    assert g(X, 64, W, 56, S, Y, 32, 10, 64, 32, None) == ESHAPE        # ldw < d_in
    assert g(X, 64, W, 72, S, Y, 32, 10, 64, 32, None) == EALIGN        # ldw % 16
    assert g(X, 64, W + 8, 64, S, Y, 32, 10, 64, 32, None) == EALIGN
    assert g(X, 64, W, 64, S + 4, Y, 32, 10, 64, 32, None) == EALIGN
    assert g(X, 64, W, 64, S, Y + 2, 32, 10, 64, 32, None) == EALIGN
    assert g(X, 64, W, 64, S, Y, 32, 0, 64, 32, None) == OK             # empty batch
    f = L.lora_linear_fused_fp8w
    p, sg = ctypes.byref(pool()), ctypes.byref(segs())
    assert f(X, 64, W, 64, S, H, sg, ctypes.byref(pool(dtype=0)), Y, 32, None) == EDTYPE
    assert f(X, 64, None, 64, S, H, sg, p, Y, 32, None) == ENULL
    assert f(X, 64, W, 64, S, None, sg, p, Y, 32, None) == ENULL
    assert f(X, 64, W, 72, S, H, sg, p, Y, 32, None) == EALIGN
    assert f(X, 64, W, 64, S, H, sg, ctypes.byref(pool(d_in=40)), Y, 32, None) == EALIGN


def _cols(*v):
    arr = (ctypes.c_int32 * len(v))(*v)
    _cols.keep.append(arr)               # the pool struct points at it (host memory)
    return ctypes.cast(arr, ctypes.c_void_p).value


_cols.keep = []


@pytest.mark.parametrize("kw,code", [
    (dict(n_proj=3, r_max=48, d_out=48), None),              # valid: rs 16, columns below
    (dict(n_proj=2, r_max=48, d_out=48), ERANK),             # rs = 24
    (dict(n_proj=3, r_max=48, d_out=48, proj_cols=0), ENULL),
    (dict(n_proj=9, r_max=72, d_out=48), ESHAPE),
    (dict(n_proj=-1), ESHAPE),
])
def test_stacked_pool_validation(L, kw, code):
    d = dict(kw)
    if "proj_cols" not in d:
        d["proj_cols"] = _cols(0, 16, 24, 48)
    p = pool(**d)
    # an empty batch: a valid pool returns OK without launching anything
    empty = segs(n_rows=0, max_segments=0, token_indices=0, row_segment=0)
    assert shrink(L, p, empty, X=0, H=0) == (OK if code is None else code)


@pytest.mark.parametrize("cols", [(0, 16, 20, 48), (0, 24, 16, 48), (0, 16, 24, 40), (8, 16, 24, 48)])
def test_stacked_pool_column_offsets(L, cols):
    p = pool(n_proj=3, r_max=48, d_out=48, proj_cols=_cols(*cols))
    assert shrink(L, p, segs()) == ESHAPE


def test_stacked_pool_pack_validation(L):
    """A stacked pool takes one A and one B source per projection, each B
    checked against its own projection's width; ranks are bounded by the
    per-projection rank stride."""
    p = ctypes.byref(pool(n_proj=3, r_max=48, d_out=48, proj_cols=_cols(0, 16, 24, 48)))
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    A = _arr(vp, P + 0xC000, P + 0xC400, P + 0xC800)
    B = _arr(vp, P + 0xD000, P + 0xD400, P + 0xD800)
    la = _arr(i64, 64, 64, 64)
    pack = L.lora_pool_pack_slot
    assert pack(p, 0, 17, 16.0, A, la, B, _arr(i64, 17, 17, 17), 0, None) == ESHAPE  # rs 16
    assert pack(p, 0, 8, 16.0, _arr(vp, P + 0xC000, 0, P + 0xC800), la, B,
                _arr(i64, 8, 8, 8), 0, None) == ENULL
    # B^T sources: ldb >= 16, 8 and 24 columns
    assert pack(p, 0, 8, 16.0, A, la, B, _arr(i64, 16, 8, 23), 1, None) == ESHAPE
    assert pack(p, 0, 8, 16.0, A, _arr(i64, 64, 64, 60), B, _arr(i64, 16, 8, 24), 1,
                None) == ESHAPE


def test_expand_and_fused_validation(L):
    p, s = pool(), segs()
    assert L.lora_expand(P, ctypes.byref(s), ctypes.byref(p), P, 24, None) == ESHAPE   # ldy < d_out
    assert L.lora_expand(P, ctypes.byref(s), ctypes.byref(p), 0, 32, None) == ENULL
    assert L.lora_linear_fused(P, 64, 0, 64, P, ctypes.byref(s), ctypes.byref(p), P, 32,
                               None) == ENULL       # W
    assert L.lora_linear_fused(P, 64, P, 56, P, ctypes.byref(s), ctypes.byref(p), P, 32,
                               None) == ESHAPE      # ldw < d_in
    assert L.lora_linear_fused(P, 64, P, 64, 0, ctypes.byref(s), ctypes.byref(p), P, 32,
                               None) == ENULL       # H


def test_base_gemm_validation(L):
    assert L.lora_base_gemm(P, 64, P, 64, P, 32, 10, 64, 32, 5, None) == EDTYPE
    assert L.lora_base_gemm(P, 64, P, 64, P, 32, -1, 64, 32, 1, None) == ESHAPE
    assert L.lora_base_gemm(P, 64, P, 64, P, 32, 10, 60, 32, 1, None) == EALIGN
    assert L.lora_base_gemm(P, 64, 0, 64, P, 32, 10, 64, 32, 1, None) == ENULL
    assert L.lora_base_gemm(P, 64, P, 64, P + 2, 32, 10, 64, 32, 1, None) == EALIGN


def test_binding_raises_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(srg, "_lib", None)
    monkeypatch.setattr(srg, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        srg.lib()


def test_static_call_validation(L):
    """The allocation-free call rejects batches beyond its scratch, and bad
    arguments, on the host (nothing is launched: these addresses are fake)."""
    f = L.lora_linear_fused_static
    p = pool()                                              # r_max 16
    rs, X, W, Y = P + 0x4000, P + 0xC000, P + 0xD000, P + 0xE000
    pp = ctypes.byref(p)
    assert f(rs, X, 64, W, 64, None, 10, Y, 32, None) == ENULL
    assert f(rs, X, 64, W, 64, pp, srg.STATIC_MAX_ROWS + 1, Y, 32, None) == ESCRATCH
    big = ctypes.byref(pool(r_max=64))                      # 32768 rows x 64 > 2^21
    assert f(rs, X, 64, W, 64, big, srg.STATIC_MAX_H // 64 + 1, Y, 32, None) == ESCRATCH
    assert f(rs, X, 64, W, 64, pp, -1, Y, 32, None) == ESHAPE
    assert f(None, X, 64, W, 64, pp, 10, Y, 32, None) == ENULL
    assert f(rs, None, 64, W, 64, pp, 10, Y, 32, None) == ENULL
    assert f(rs, X, 60, W, 64, pp, 10, Y, 32, None) == ESHAPE        # ldx < d_in
    assert f(rs, X, 64, W, 64, pp, 10, Y + 8, 32, None) == EALIGN    # Y not 16-byte aligned
    assert f(rs, X, 64, W, 64, pp, 0, Y, 32, None) == OK             # empty batch: no-op


def test_leading_dimension_limit(L):
    """Leading dimensions above LORA_MAX_LD (2^22 elements) are rejected on
    the host: the GEMM addresses a tile's rows with 32-bit byte offsets."""
    big = (1 << 22) + 8
    assert L.lora_base_gemm(P, big, P, 64, P, 32, 10, 64, 32, 1, None) == ESHAPE
    assert L.lora_base_gemm(P, 64, P, big, P, 32, 10, 64, 32, 1, None) == ESHAPE
    assert L.lora_base_gemm(P, 64, P, 64, P, big, 10, 64, 32, 1, None) == ESHAPE
    assert L.lora_base_gemm_fp8w(P, 64, P, big, P, P, 32, 10, 64, 32, None) == ESHAPE


def test_layer_call_validation(L):
    """The one-call layer checks the arguments of the three calls it stands
    for, and its sync buffer's alignment, on the host (fake addresses: nothing
    is launched)."""
    f = L.lora_layer_fused
    rs, X, W, H, Y, SY = P + 0xC000, P + 0xD000, P + 0xE000, P + 0xF000, P + 0x10000, P + 0x11000
    p, sg = ctypes.byref(pool()), ctypes.byref(segs())
    assert f(rs, X, 64, W, 64, None, sg, H, Y, 32, SY, None) == ENULL
    assert f(rs, X, 64, W, 64, p, None, H, Y, 32, SY, None) == ENULL
    assert f(None, X, 64, W, 64, p, sg, H, Y, 32, SY, None) == ENULL
    assert f(rs, None, 64, W, 64, p, sg, H, Y, 32, SY, None) == ENULL
    assert f(rs, X, 64, None, 64, p, sg, H, Y, 32, SY, None) == ENULL
    assert f(rs, X, 64, W, 64, p, sg, None, Y, 32, SY, None) == ENULL
    assert f(rs, X, 64, W, 64, p, sg, H, None, 32, SY, None) == ENULL
    assert f(rs, X, 60, W, 64, p, sg, H, Y, 32, SY, None) == ESHAPE       # ldx < d_in
    assert f(rs, X, 64, W, 64, p, sg, H + 8, Y, 32, SY, None) == EALIGN
    assert f(rs, X, 64, W, 64, p, sg, H, Y, 32, SY + 4, None) == EALIGN   # sync alignment
    assert f(rs, X, 64, W, 64, ctypes.byref(pool(rank_policy=5)), sg, H, Y, 32, SY, None) == EPOLICY
    assert f(rs, X, 64, W, 64, p, ctypes.byref(segs(max_segments=4)), H, Y, 32, SY, None) == ECAP
    assert srg.LAYER_SYNC_BYTES == 4096 and srg.LAYER_ONE_LAUNCH_ROWS == 512



def test_fp8_layer_call_validation(L):
    """The FP8-weight layer call checks the same arguments, the weight's
    scales and code layout, and bf16 pools only, before any launch."""
    f = L.lora_layer_fused_fp8w
    rs, X, Wq, WS, H, Y, SY = (P + 0xC000, P + 0xD000, P + 0xE000, P + 0x12000, P + 0xF000,
                               P + 0x10000, P + 0x11000)
    p, sg = ctypes.byref(pool()), ctypes.byref(segs())
    assert f(rs, X, 64, Wq, 64, None, p, sg, H, Y, 32, SY, None) == ENULL     # no scales
    assert f(rs, X, 64, None, 64, WS, p, sg, H, Y, 32, SY, None) == ENULL
    assert f(None, X, 64, Wq, 64, WS, p, sg, H, Y, 32, SY, None) == ENULL
    assert f(rs, X, 64, Wq, 64, WS, p, sg, None, Y, 32, SY, None) == ENULL
    assert f(rs, X, 64, Wq, 60, WS, p, sg, H, Y, 32, SY, None) != 0          # ldw < d_in
    assert f(rs, X, 64, Wq, 64, WS, p, sg, H, Y, 32, SY + 4, None) == EALIGN
    assert f(rs, X, 64, Wq, 64, WS, ctypes.byref(pool(dtype=0)), sg, H, Y, 32, SY, None) == EDTYPE
