"""GPU parity of the FP8-E4M3 base weight (W = w_scale * e4m3(Wq); adapter-
batching page, "Quantized Base Model 与 LoRA 的 Dtype 边界"): the base GEMM
and the fused layer against the oracle's lora_forward_fp8w, with the bf16
normwise tolerance (1e-2), on both tile configurations, ragged shapes and
K tails; exact results on small-integer inputs; base-only rows of the fused
call equal the base call bit for bit; both B layouts give the same bits."""
import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_segment_amd as srg
import workloads as wl
from gpu_harness import DEV, TOL, normwise, sample_rows, say, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    srg.lib()
    yield
    torch.cuda.synchronize()


def _run(w, codes, scale, natural_b=True, policy="exact"):
    d = wl.device_tensors(w, DEV)
    Wq = torch.from_numpy(codes).to(DEV)
    ws = torch.from_numpy(scale).to(DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha, policy, natural_b=natural_b)
    seg = srg.Segments(w.n, w.n_slots, DEV)
    H = torch.full((w.n, w.r_max), float("nan"), dtype=torch.float32, device=DEV)
    srg.lora_build_shrink(d["row_slot"], d["X"], pool, seg, H)
    Yf = torch.empty((w.n, w.d_out), dtype=torch.bfloat16, device=DEV)
    srg.lora_linear_fused_fp8w(d["X"], Wq, ws, H, seg, pool, Yf)
    Yb = torch.empty_like(Yf)
    srg.lora_base_gemm_fp8w(d["X"], Wq, ws, Yb)
    torch.cuda.synchronize()
    return Yf, Yb


def _check(w, codes, scale, Yf, Yb, rows=None):
    Y, dY, _ = oracle.lora_forward_fp8w(w.X, codes, scale, w.A, w.B, w.row_slot, w.slot_rank,
                                        w.slot_alpha, w.r_max, w.dtype, rows=rows)
    idx = np.arange(w.n) if rows is None else np.asarray(rows)
    ti = torch.as_tensor(idx, device=DEV, dtype=torch.long)
    e = {"fused": normwise(to_f64(Yf[ti]), Y), "base": normwise(to_f64(Yb[ti]), Y - dY)}
    for k, v in e.items():
        assert v <= TOL["bf16"], (k, v)
    # base-only and rank-0 rows: the fused output is the base output
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    base = [i for i in idx if keys[i] < 0 or int(w.slot_rank[keys[i]]) == 0]
    if base:
        tb = torch.as_tensor(base, device=DEV)
        assert torch.equal(Yf[tb], Yb[tb])
    return e


CASES = [
    # seed, n, d_in, d_out, n_slots, r_max, p_base, runs
    (501, 1, 64, 72, 3, 8, 0.0, False),
    (502, 7, 144, 200, 5, 16, 0.3, False),
    (503, 300, 528, 264, 40, 64, 0.1, False),    # K tail on the small tiles (528 % 128)
    (504, 512, 256, 384, 6, 32, 0.2, True),
    (505, 700, 208, 136, 7, 64, 0.1, True),      # large tiles, K tail (208 % 64), ragged N
    (506, 2100, 336, 264, 5, 32, 0.2, True),
    (507, 1100, 208, 8200, 7, 64, 0.1, True),    # 192 x 256 tiles with a K tail
    (508, 2040, 208, 7944, 7, 64, 0.1, True),    # 256 x 256 tiles with a K tail
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_fp8w_cases(case):
    seed, n, d_in, d_out, n_slots, r_max, p_base, runs = case
    say("fp8w", case)
    w = wl.make_random(seed, n, d_in, d_out, n_slots, r_max, p_base=p_base, dtype="bf16", runs=runs)
    if n_slots > 2:
        w.slot_rank[1] = 0
    codes, scale = wl.make_fp8_weight(seed, d_out, d_in)
    Yf, Yb = _run(w, codes, scale)
    e = _check(w, codes, scale, Yf, Yb)
    say("fp8w errors", e)


@pytest.mark.parametrize("n", [96, 1100])
def test_fp8w_b_layouts_give_identical_bits(n):
    w = wl.make_random(510, n, 256, 264, 9, 32, p_base=0.1, dtype="bf16", runs=True)
    codes, scale = wl.make_fp8_weight(510, w.d_out, w.d_in)
    Yf1, _ = _run(w, codes, scale, natural_b=True)
    Yf2, _ = _run(w, codes, scale, natural_b=False)
    assert torch.equal(Yf1, Yf2)


@pytest.mark.parametrize("n", [40, 600])
def test_fp8w_exact_on_small_integers(n):
    """X in {-1, 0, 1}, codes of -2..2, power-of-two scales, no adapters: every
    product and partial sum is a small integer times a power of two, so the
    result is exact and must equal the oracle's to the bit."""
    rng = np.random.default_rng(n)
    d_in, d_out = 32, 136
    w = wl.make_random(511, n, d_in, d_out, 2, 8, p_base=1.0, dtype="bf16")
    w.X = wl._encode(rng.integers(-1, 2, size=(n, d_in)).astype(np.float32), "bf16")
    ints = rng.integers(-2, 3, size=(d_out, d_in))
    code = {0: 0x00, 1: 0x38, 2: 0x40}
    codes = np.vectorize(lambda v: code[abs(v)] | (0x80 if v < 0 else 0))(ints).astype(np.uint8)
    scale = np.exp2(rng.integers(-2, 2, size=d_out)).astype(np.float32)
    Yf, Yb = _run(w, codes, scale)
    Y, _, _ = oracle.lora_forward_fp8w(w.X, codes, scale, w.A, w.B, w.row_slot, w.slot_rank,
                                       w.slot_alpha, w.r_max, "bf16")
    assert np.array_equal(to_f64(Yb), Y) and np.array_equal(to_f64(Yf), Y)


def test_fp8w_decode_workload():
    w = wl.make_workload("decode")
    codes, scale = wl.make_fp8_weight(2, w.d_out, w.d_in)
    Yf, Yb = _run(w, codes, scale)
    say("fp8w decode", _check(w, codes, scale, Yf, Yb))


def test_fp8w_prefill_sampled():
    w = wl.make_workload("prefill")
    codes, scale = wl.make_fp8_weight(3, w.d_out, w.d_in)
    Yf, Yb = _run(w, codes, scale)
    meta = oracle.segment_metadata(w.row_slot, w.slot_rank, w.slot_alpha, w.r_max)
    rows = sample_rows(w, meta, 256)
    say("fp8w prefill", _check(w, codes, scale, Yf, Yb, rows=rows))
    assert torch.isfinite(Yf.float()).all()
