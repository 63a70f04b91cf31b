"""GPU parity of the LoRA term of the fused product on its own.

lora_linear_fused adds s_a H[i][0:r] B_a^T into the base accumulator and
rounds once (the epilogue fusion of the ybb.press multi-LoRA serving article,
section 5.3; the term itself is Delta Y_a = s_a H_a B_a^T of the
adapter-batching page, "Segmented Kernel 需要哪些 Metadata").  Checked through
Y alone, a wrong term hides under the base output (Delta Y is about a tenth
of Y in these workloads).  Here the base weight is zero, so the fp32
accumulator holds exactly the LoRA term and the output is its one rounding:

* random adapters: the fused output against the oracle's Delta Y, normwise
  at the layer's tolerance (1e-2 bf16, 1e-5 fp32) and element by element
  within one rounding of each value (half an ulp: 2^-8 of |Delta Y| for bf16)
  plus 2^-12 of max |Delta Y| for the fp32 sums and the bf16 high/low split
  of s H in the staged MFMA term;
* fingerprint adapters (Delta Y_i = s_a (a + 1) x_i[a mod d_in] in every
  column, exact in fp32): bit for bit.

Every tile family of the fused GEMM is covered, by the shapes that select it:
64 x 64 two-group tiles with the four- and two-stage rings (batches of at
most 512 rows), 128 x 128 and 256 x 256 tiles with at most four LoRA runs
per tile (the staged MFMA term) and with more (the row epilogue), both B
layouts, both rank policies, the DoRA and FP8-weight variants, stacked
projections and fp32.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_segment_amd as srg
import workloads as wl
from gpu_harness import DEV, TOL, normwise, say, to_f64

pytestmark = pytest.mark.gpu

# element-wise bound |got - ref| <= REL |ref| + ABS max|ref|
TERM_BOUND = {"bf16": (2.0 ** -8, 2.0 ** -12), "f32": (1e-6, 1e-6)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    srg.lib()
    yield
    torch.cuda.synchronize()


def _zero_base(w):
    w.W = np.zeros_like(w.W)
    return w


def check_term(got: np.ndarray, ref: np.ndarray, dtype: str) -> dict:
    """Normwise and element-wise comparison of a fused output (zero base)
    with the oracle's Delta Y."""
    e = normwise(got, ref)
    assert e <= TOL[dtype], ("normwise", e)
    rel, absf = TERM_BOUND[dtype]
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    excess = np.abs(got - ref) - (rel * np.abs(ref) + absf * m)
    worst = float(np.max(excess)) if ref.size else 0.0
    if worst > 0:
        i, j = np.unravel_index(int(np.argmax(excess)), excess.shape)
        raise AssertionError(f"element ({i}, {j}): got {got[i, j]!r}, oracle {ref[i, j]!r}, "
                             f"bound {rel} |ref| + {absf} max|ref| (max|ref| {m})")
    return {"normwise": e, "n": int(ref.size)}


def fingerprint_bits(w) -> np.ndarray:
    """Expected output bits of the fused product with a zero base on a
    fingerprint workload: rows on slot a hold s_a (a + 1) x[a mod d_in] in
    every column (exact in fp32, then one rounding), other rows zero."""
    X = oracle.decode(w.X, w.dtype)
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    exp = np.zeros((w.n,), dtype=np.float64)
    for i in range(w.n):
        a = keys[i]
        if a >= 0 and int(w.slot_rank[a]) > 0:
            exp[i] = float(w.slot_alpha[a]) / int(w.slot_rank[a]) * (a + 1) * X[i, a % w.d_in]
    exp32 = exp.astype(np.float32)
    assert np.array_equal(exp32.astype(np.float64), exp), "fingerprint not exact in fp32"
    bits = wl.bf16_bits_rne(exp32) if w.dtype == "bf16" else exp32.view(np.uint32)
    return np.repeat(bits[:, None], w.d_out, axis=1)


def _bits(Y: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return Y.view(torch.int16).cpu().numpy().view(np.uint16)
    return Y.cpu().numpy().view(np.uint32)


def _fused(w, pool, d, fp8=None):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    seg = srg.Segments(w.n, w.n_slots, DEV)
    H = torch.full((w.n, pool.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_build_shrink(d["row_slot"], d["X"], pool, seg, H)
    Y = torch.full((w.n, pool.d_out), float("nan"), dtype=dt, device=DEV)
    if fp8 is None:
        srg.lora_linear_fused(d["X"], d["W"], H, seg, pool, Y)
    else:
        srg.lora_linear_fused_fp8w(d["X"], fp8[0], fp8[1], H, seg, pool, Y)
    torch.cuda.synchronize()
    return Y


def _pool(w, d, policy="exact", natural_b=True, dora=False):
    return srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, policy, natural_b=natural_b,
                    dora=dora)


# Tile families, each selected by its shape: (id, n, d_in, d_out, tile rows,
# LoRA runs per tile or None for independent random rows).
FAMILIES = [
    ("t64_4stage", 400, 256, 264, 64, None),          # 7 x 5 tiles
    ("t64_2stage", 500, 136, 4168, 64, None),         # 8 x 66 tiles: more than the CUs
    ("t128_staged", 1100, 200, 1032, 128, [1, 2, 3, 4]),
    ("t128_rows", 1100, 200, 1032, 128, [5, 9, 30, 128]),
    ("t128_mixed", 1100, 200, 1032, 128, [1, 7, 4, 64, 2]),
    ("t192_staged", 1100, 136, 8200, 192, [1, 2, 3, 4]),   # 6 x 33 tiles of 192 x 256
    ("t192_rows", 1100, 136, 8200, 192, [5, 40, 192]),
    ("t192_mixed", 1100, 136, 8200, 192, [4, 192, 1, 6]),
    # rows [0, 1792) on 7 x 33 tiles of 256 x 256, rows [1792, 2100) on 64 x 64 tiles
    ("split_staged", 2100, 136, 8200, 256, [1, 2, 3, 4]),
    ("split_rows", 2100, 136, 8200, 256, [5, 40, 256]),
    ("t256_staged", 2040, 136, 7944, 256, [1, 2, 3, 4]),   # 8 x 32 tiles of 256 x 256
    ("t256_rows", 2040, 136, 7944, 256, [5, 40, 256]),
    ("t256_mixed", 2040, 136, 7944, 256, [4, 256, 1, 6]),
]


def _mapping(fam, seed, n_slots):
    _, n, _, _, tile, runs = fam
    if runs is None:
        rng = np.random.default_rng(seed)
        return np.where(rng.random(n) < 0.1, -1, rng.integers(0, n_slots, size=n)).astype(np.int32)
    return wl.tile_runs_mapping(seed, n, tile, runs, n_slots)


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
@pytest.mark.parametrize("natural_b", [True, False], ids=["Bn", "Bt"])
def test_term_random(fam, natural_b):
    name, n, d_in, d_out, _, _ = fam
    seed = 800 + FAMILIES.index(fam)
    say("term random", name, natural_b)
    w = _zero_base(wl.make_random(seed, n, d_in, d_out, 40, 64, p_base=0.0))
    w.row_slot = _mapping(fam, seed, w.n_slots)
    w.slot_rank[5] = 0
    d = wl.device_tensors(w, DEV)
    Y = _fused(w, _pool(w, d, natural_b=natural_b), d)
    _, dY, _ = oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                   w.r_max, w.dtype)
    say("term", name, check_term(to_f64(Y), dY, w.dtype))


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
@pytest.mark.parametrize("policy", ["exact", "padded"])
def test_term_fingerprint_exact(fam, policy):
    name, n, d_in, d_out, _, _ = fam
    seed = 850 + FAMILIES.index(fam)
    say("term fingerprint", name, policy)
    w = _zero_base(wl.make_fingerprint(seed, n, d_in, d_out, 200, 64,
                                       row_slot=_mapping(fam, seed, 200)))
    d = wl.device_tensors(w, DEV)
    Y = _fused(w, _pool(w, d, policy=policy), d)
    got, want = _bits(Y, w.dtype), fingerprint_bits(w)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{len(bad)} elements differ; first (row, col) {bad[:4].tolist()}, "
                           f"slots {[int(w.row_slot[i]) for i, _ in bad[:4]]}")


@pytest.mark.parametrize("fam", [FAMILIES[0], FAMILIES[2], FAMILIES[6]],
                         ids=[FAMILIES[i][0] for i in (0, 2, 6)])
def test_term_fp8_weight(fam):
    """FP8 weight of zero codes (row scales still applied to the zero base)."""
    name, n, d_in, d_out, _, _ = fam
    d_in = (d_in + 15) // 16 * 16          # FP8 rows: d_in a multiple of 16
    seed = 870 + FAMILIES.index(fam)
    say("term fp8", name)
    w = wl.make_random(seed, n, d_in, d_out, 40, 64, p_base=0.0)
    w.row_slot = _mapping(fam, seed, w.n_slots)
    codes = np.zeros((d_out, d_in), dtype=np.uint8)
    scale = wl.make_fp8_weight(seed, d_out, d_in)[1]
    d = wl.device_tensors(w, DEV)
    fp8 = (torch.from_numpy(codes).to(DEV), torch.from_numpy(scale).to(DEV))
    Y = _fused(w, _pool(w, d), d, fp8=fp8)
    _, dY, _ = oracle.lora_forward_fp8w(w.X, codes, scale, w.A, w.B, w.row_slot, w.slot_rank,
                                        w.slot_alpha, w.r_max, w.dtype)
    say("term fp8", name, check_term(to_f64(Y), dY, "bf16"))
    # fingerprints through the FP8 path: bit for bit
    wf = wl.make_fingerprint(seed, n, d_in, d_out, 200, 64, row_slot=_mapping(fam, seed, 200))
    df = wl.device_tensors(wf, DEV)
    Yf = _fused(wf, _pool(wf, df), df, fp8=fp8)
    assert np.array_equal(_bits(Yf, "bf16"), fingerprint_bits(wf))


@pytest.mark.parametrize("fam", [FAMILIES[0], FAMILIES[4], FAMILIES[7]],
                         ids=[FAMILIES[i][0] for i in (0, 4, 7)])
def test_term_dora(fam):
    """DoRA factors prepared against the zero base: rows of rank > 0 are
    g_a * Delta Y with g_a = m_a / ||s_a B_a A_a||_c (oracle.dora_forward with
    W = 0)."""
    name, n, d_in, d_out, _, _ = fam
    seed = 880 + FAMILIES.index(fam)
    say("term dora", name)
    w = _zero_base(wl.make_random(seed, n, d_in, d_out, 40, 64, p_base=0.0))
    w.row_slot = _mapping(fam, seed, w.n_slots)
    mag = wl.make_magnitude(seed, w.n_slots, d_out, 0.02 * math.sqrt(d_in), p_plain=0.25)
    d = wl.device_tensors(w, DEV)
    pool = _pool(w, d, dora=True)
    for a in range(w.n_slots):
        if mag[a] is not None:
            pool.dora_prepare(a, d["W"], torch.from_numpy(mag[a]).to(DEV))
    Y = _fused(w, pool, d)
    ref = oracle.dora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha, mag,
                              w.r_max, w.dtype)
    say("term dora", name, check_term(to_f64(Y), ref, "bf16"))


@pytest.mark.parametrize("n", [300, 1100, 2100])
def test_term_stacked(n):
    """q|k|v-like stacked projections with a zero base: every projection's
    block equals its own Delta Y (tiles straddle the projection bounds)."""
    seed = 890 + n
    say("term stacked", n)
    outs = (520, 136, 264)
    mapping = wl.tile_runs_mapping(seed, n, 128, [1, 3, 6, 2], 12)
    ws = []
    for p, d_out in enumerate(outs):
        w = wl.make_random(seed * 10 + p, n, 192, d_out, 12, 32, p_base=0.0,
                           ranks=None if p == 0 else list(ws[0].slot_rank))
        if p:
            w.X = ws[0].X
        w.row_slot = mapping
        ws.append(_zero_base(w))
    pools = []
    for w in ws:
        dw = wl.device_tensors(w, DEV)
        pools.append(srg.Pool(dw["A"], dw["Bt"], dw["slot_rank"], w.slot_alpha, natural_b=False))
    pool = srg.Pool.stacked(pools)
    b = ws[0]
    d = wl.device_tensors(b, DEV)
    d["W"] = torch.zeros((sum(outs), b.d_in), dtype=torch.bfloat16, device=DEV)
    Y = _fused(b, pool, d)
    _, dY, _ = oracle.stacked_forward(b.X, [w.W for w in ws], [w.A for w in ws],
                                      [w.B for w in ws], b.row_slot, b.slot_rank, b.slot_alpha,
                                      b.r_max, "bf16")
    say("term stacked", n, check_term(to_f64(Y), dY, "bf16"))


@pytest.mark.parametrize("n", [32, 300])
def test_term_f32(n):
    """The fp32 product's LoRA term (the tiny fp32 case's layout at n = 32)."""
    w = _zero_base(wl.make_workload("tiny_f32") if n == 32 else
                   wl.make_random(895, n, 136, 200, 9, 32, p_base=0.1, dtype="f32",
                                  x_std=0.02, runs=True))
    d = wl.device_tensors(w, DEV)
    Y = _fused(w, _pool(w, d), d)
    _, dY, _ = oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                   w.r_max, w.dtype)
    say("term f32", n, check_term(to_f64(Y), dY, "f32"))
    wf = _zero_base(wl.make_fingerprint(896, 300, 136, 200, 60, 32, dtype="f32", runs=True))
    df = wl.device_tensors(wf, DEV)
    Yf = _fused(wf, _pool(wf, df), df)
    assert np.array_equal(_bits(Yf, "f32"), fingerprint_bits(wf))
