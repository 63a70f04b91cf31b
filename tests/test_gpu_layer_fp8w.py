"""GPU parity of the one-call layer with an FP8 E4M3 base weight,
lora_layer_fused_fp8w (adapter-batching page, sections "Segmented Kernel
需要哪些 Metadata" and "Quantized Base Model 与 LoRA 的 Dtype 边界": the base
weight is W = w_scale * e4m3(Wq), the adapters stay bf16).  Against the
oracle's lora_forward_fp8w: the segment metadata bit for bit, H on the
written entries only, Y within the bf16 tolerance, and the LoRA increment
alone (all weight codes zero, so Y is the rounded increment) within the
same tolerance of the increment;
base-only and rank-0 rows equal lora_base_gemm_fp8w bit for bit; with and
without a sync buffer the same bits; repeated calls on one sync buffer; the
two-launch fallback past 512 rows.
"""
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


def run(w, codes, scale, sync=True, sync_buf=None, d=None):
    d = d or wl.device_tensors(w, DEV)
    Wq = torch.from_numpy(codes).to(DEV)
    ws = torch.from_numpy(scale).to(DEV)
    pool = srg.Pool(d["A"], d["Bt"], d["slot_rank"], w.slot_alpha)
    seg = srg.Segments(w.n, w.n_slots, DEV)
    H = torch.full((w.n, pool.r_max), float("nan"), dtype=torch.float32, device=DEV)
    Y = torch.empty((w.n, pool.d_out), dtype=torch.bfloat16, device=DEV)
    sy = sync_buf if sync_buf is not None else (srg.layer_sync(DEV) if sync else None)
    srg.lora_layer_fused_fp8w(d["row_slot"], d["X"], Wq, ws, pool, seg, H, Y, sy)
    Yb = torch.empty_like(Y)
    srg.lora_base_gemm_fp8w(d["X"], Wq, ws, Yb)
    torch.cuda.synchronize()
    return dict(H=H, Y=Y, Yb=Yb, meta=seg.to_host(), d=d, pool=pool, Wq=Wq, ws=ws)


def check(w, codes, scale, r):
    ref = oracle.segment_metadata(w.row_slot, w.slot_rank, w.slot_alpha, w.r_max)
    m = r["meta"]
    assert m["num_segments"] == int(ref["num_segments"])
    for k in ("segment_offsets", "segment_slots", "segment_ranks", "token_indices", "row_segment"):
        assert np.array_equal(m[k], ref[k]), k
    assert m["status"] == int(ref["status"])
    Y, dY, Hr = oracle.lora_forward_fp8w(w.X, codes, scale, w.A, w.B, w.row_slot, w.slot_rank,
                                         w.slot_alpha, w.r_max, w.dtype)
    keys, _ = oracle.validate_rows(w.row_slot, w.slot_rank, w.r_max)
    Hg = to_f64(r["H"])
    mask = np.zeros_like(Hg, dtype=bool)
    for i, a in enumerate(keys):
        if a >= 0:
            mask[i, :int(w.slot_rank[a])] = True
    assert np.all(np.isnan(Hg[~mask])), "H written outside [0, rank)"
    e = {"H": normwise(np.where(mask, Hg, 0.0), Hr), "Y": normwise(to_f64(r["Y"]), Y)}
    for k, v in e.items():
        assert v <= TOL["bf16"], (k, v)
    base = [i for i, a in enumerate(keys) if a < 0 or int(w.slot_rank[a]) == 0]
    if base:
        tb = torch.as_tensor(base, device=DEV)
        assert torch.equal(r["Y"][tb], r["Yb"][tb])
    return e


CASES = [
    # seed, n, d_in, d_out, n_slots, r_max, p_base
    (651, 1, 64, 72, 3, 8, 0.0),
    (652, 7, 144, 200, 5, 16, 0.3),
    (653, 256, 512, 4096, 40, 16, 0.1),     # decode shape, one launch
    (654, 300, 528, 264, 40, 64, 0.1),      # row-only workgroups, K tail
    (655, 512, 256, 4104, 60, 32, 0.1),     # more tiles than CUs, N tail
    (656, 700, 208, 136, 7, 64, 0.1),       # past 512 rows: the two calls
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_cases(case):
    seed, n, d_in, d_out, n_slots, r_max, p_base = case
    say("layer fp8w", case)
    w = wl.make_random(seed, n, d_in, d_out, n_slots, r_max, p_base=p_base)
    w.slot_rank[min(2, n_slots - 1)] = 0
    codes, scale = wl.make_fp8_weight(seed, d_out, d_in)
    a = run(w, codes, scale, sync=True)
    say("errors", check(w, codes, scale, a))
    b = run(w, codes, scale, sync=False, d=a["d"])
    assert torch.equal(a["Y"], b["Y"])
    assert torch.equal(a["H"].nan_to_num(7.0), b["H"].nan_to_num(7.0))
    # the increment alone: a zero base weight
    z = run(w, np.zeros_like(codes), scale, d=a["d"])
    _, dY, _ = oracle.lora_forward_fp8w(w.X, np.zeros_like(codes), scale, w.A, w.B, w.row_slot,
                                        w.slot_rank, w.slot_alpha, w.r_max, w.dtype)
    e = normwise(to_f64(z["Y"]), dY)
    assert e <= TOL["bf16"], e
    say("increment error", e)


def test_repeated_calls_on_one_sync_buffer():
    sy = srg.layer_sync(DEV)
    for k in range(3):
        w = wl.make_random(660 + k, 200, 256, 512, 20, 32, p_base=0.1)
        codes, scale = wl.make_fp8_weight(660 + k, w.d_out, w.d_in)
        r = run(w, codes, scale, sync_buf=sy)
        check(w, codes, scale, r)
        say("repeat", k, "ok")
