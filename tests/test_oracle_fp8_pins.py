"""Pins of the quantized-base part of the oracle: FP8 E4M3 decoding (OCP
8-bit floating point specification) and the layer with W = w_scale * e4m3(Wq)
(adapter-batching page, "Quantized Base Model 与 LoRA 的 Dtype 边界").

The decoder is checked against torch's float8_e4m3fn conversion for all 256
codes (a library routine), against values the specification fixes, and by
planted mistakes; the layer against the plain oracle on weights that both
formats hold exactly, and by linearity in the scale."""
import inspect
import textwrap

import numpy as np
import pytest
import torch

import oracle
import oracle.lora_oracle as lo
import workloads as wl


def _torch_decode():
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _same(a, b):
    return np.array_equal(np.nan_to_num(a, nan=1e300), np.nan_to_num(b, nan=1e300))


def test_decode_matches_torch_for_every_code():
    assert _same(oracle.decode_fp8_e4m3(np.arange(256, dtype=np.uint8)), _torch_decode())


def test_decode_specification_values():
    d = oracle.decode_fp8_e4m3
    cases = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0xC0: -2.0, 0x7E: 448.0, 0xFE: -448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x3C: 1.5}
    for code, val in cases.items():
        assert d(np.array([code], np.uint8))[0] == val, hex(code)
    assert np.isnan(d(np.array([0x7F, 0xFF], np.uint8))).all()
    assert np.signbit(d(np.array([0x80], np.uint8))[0])
    # 254 finite codes, strictly increasing over the non-negative half
    pos = d(np.arange(0x00, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


MUTATIONS = {
    "bias_8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "no_subnormals": ("v = np.where(e == 0, sub, normal)", "v = normal"),
    "sign_dropped": ("sign = np.where(c & 0x80, -1.0, 1.0)", "sign = np.ones(c.shape)"),
    "mantissa_over_16": ("m / 8.0) * np.exp2(e", "m / 16.0) * np.exp2(e"),
    "no_nan": ("return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)", "return v"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_decode_mutants_fail(name):
    old, new = MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(lo.decode_fp8_e4m3))
    assert old in src, name
    ns = dict(vars(lo))
    exec(src.replace(old, new), ns)
    assert not _same(ns["decode_fp8_e4m3"](np.arange(256, dtype=np.uint8)), _torch_decode())


_INT_CODE = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_integer_weights_equal_the_plain_layer(dtype):
    """Small-integer weights are exact both as E4M3 codes with scale 1 and
    as bf16/fp32: the quantized-base layer equals the plain one."""
    rng = np.random.default_rng(3)
    w = wl.make_random(21, n=40, d_in=48, d_out=24, n_slots=4, r_max=16, p_base=0.2, dtype=dtype)
    ints = rng.integers(-4, 5, size=(w.d_out, w.d_in))
    codes = np.vectorize(lambda v: _INT_CODE[abs(v)] | (0x80 if v < 0 else 0))(ints).astype(np.uint8)
    w.W = wl._encode(ints.astype(np.float32), dtype)
    Y, dY, H = oracle.lora_forward(w.X, w.W, w.A, w.B, w.row_slot, w.slot_rank, w.slot_alpha,
                                   w.r_max, dtype)
    Yq, dYq, Hq = oracle.lora_forward_fp8w(w.X, codes, np.ones(w.d_out, np.float32), w.A, w.B,
                                          w.row_slot, w.slot_rank, w.slot_alpha, w.r_max, dtype)
    np.testing.assert_array_equal(Yq, Y)
    np.testing.assert_array_equal(dYq, dY)
    np.testing.assert_array_equal(Hq, H)


def test_scale_is_per_output_row_and_linear():
    w = wl.make_random(22, n=30, d_in=64, d_out=40, n_slots=3, r_max=8, dtype="bf16")
    codes, scale = wl.make_fp8_weight(22, w.d_out, w.d_in)
    Y, dY, _ = oracle.lora_forward_fp8w(w.X, codes, scale, w.A, w.B, w.row_slot, w.slot_rank,
                                        w.slot_alpha, w.r_max, w.dtype)
    s2 = scale.copy()
    s2[7] *= 4.0                              # exact in float32
    Y2, dY2, _ = oracle.lora_forward_fp8w(w.X, codes, s2, w.A, w.B, w.row_slot, w.slot_rank,
                                          w.slot_alpha, w.r_max, w.dtype)
    np.testing.assert_array_equal(dY2, dY)
    other = [j for j in range(w.d_out) if j != 7]
    np.testing.assert_array_equal(Y2[:, other], Y[:, other])
    np.testing.assert_allclose(Y2[:, 7] - dY[:, 7], 4.0 * (Y[:, 7] - dY[:, 7]), rtol=1e-12,
                               atol=1e-15)


def test_row_subset_and_generator():
    w = wl.make_random(23, n=50, d_in=64, d_out=32, n_slots=5, r_max=16, dtype="bf16")
    codes, scale = wl.make_fp8_weight(23, w.d_out, w.d_in)
    assert codes.dtype == np.uint8 and codes.shape == (32, 64)
    assert not np.isnan(oracle.decode_fp8_e4m3(codes)).any()
    Y, _, _ = oracle.lora_forward_fp8w(w.X, codes, scale, w.A, w.B, w.row_slot, w.slot_rank,
                                       w.slot_alpha, w.r_max, w.dtype)
    rows = [4, 0, 31]
    Yr, _, _ = oracle.lora_forward_fp8w(w.X, codes, scale, w.A, w.B, w.row_slot, w.slot_rank,
                                        w.slot_alpha, w.r_max, w.dtype, rows=rows)
    np.testing.assert_allclose(Yr, Y[rows], rtol=1e-13, atol=1e-15)
