"""Pins for the oracle's scalar numerics: own exp and sigmoid, bf16 and E4M3.

Each check compares against something other than the oracle itself: float64
libm/numpy values, closed forms, or torch's own CPU conversions (library routines).
"""
import math

import numpy as np
import pytest
import torch


def ulp32(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


def test_exp_spec_exact_points(orc):
    assert orc.exp_spec(0.0) == 1.0
    assert orc.exp_spec(-0.0) == 1.0
    # exp(k ln2) for integer k is 2^k up to the rounding of the argument
    for k in range(-100, 101, 7):
        a = np.float32(k * math.log(2.0))
        ref = math.exp(float(a))
        got = orc.exp_spec(float(a))
        assert abs(got - ref) <= 2 * ulp32(ref), (k, got, ref)


def test_exp_spec_sweep_within_2ulp(orc):
    rng = np.random.default_rng(0)
    a = np.concatenate([np.linspace(-80, 80, 200001, dtype=np.float32),
                        rng.uniform(-80, 80, 100000).astype(np.float32),
                        rng.uniform(-1, 1, 50000).astype(np.float32)])
    got = orc.exp_spec_array(a).astype(np.float64)
    ref = np.exp(a.astype(np.float64))
    err = np.abs(got - ref) / ulp32(ref)
    assert err.max() <= 2.0, err.max()


def test_sigmoid_closed_forms(orc):
    assert orc.sigmoid(0.0) == 0.5
    # clamp at +-80: beyond it the value does not change and stays positive
    assert orc.sigmoid(1000.0) == orc.sigmoid(80.0) == 1.0
    assert orc.sigmoid(-1000.0) == orc.sigmoid(-80.0)
    assert 0.0 < orc.sigmoid(-80.0) < 1e-34


def test_sigmoid_sweep_symmetry_monotone(orc):
    z = np.linspace(-30, 30, 120001, dtype=np.float32)
    s = orc.sigmoid_array(z).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    assert (np.abs(s - ref) / ulp32(ref)).max() <= 3.0
    sm = orc.sigmoid_array(-z).astype(np.float64)
    # s(z) + s(-z) = 1 up to one rounding of each term
    assert np.abs(s + sm - 1.0).max() <= 2 * 2.0 ** -24
    assert np.all(np.diff(s) >= 0)


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(1)
    v = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact midpoints between neighbouring bf16 values (ties go to even)
    base = (rng.integers(0x3000, 0x5000, 20000).astype(np.uint32) << 16)
    mid = (base | 0x8000).view(np.float32)
    v = np.concatenate([v, mid, -mid, np.array([0.0, -0.0, 1.0, 65504.0], np.float32)])
    got = orc.bf16_from_f64_array(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_widening_exact(orc):
    codes = np.arange(0, 65536, 7, dtype=np.uint16)
    codes = codes[((codes >> 7) & 0xFF) != 0xFF]  # finite only
    w = orc.bf16_to_f32(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


def test_e4m3_decode_table(orc):
    # OCP E4M3: bias 7, 3 mantissa bits, subnormal m/8 * 2^-6, max 448, S.1111.111 = NaN
    assert orc.e4m3_to_f32(0x00) == 0.0
    assert orc.e4m3_to_f32(0x01) == 2.0 ** -9
    assert orc.e4m3_to_f32(0x07) == 7 * 2.0 ** -9
    assert orc.e4m3_to_f32(0x08) == 2.0 ** -6
    assert orc.e4m3_to_f32(0x38) == 1.0
    assert orc.e4m3_to_f32(0x7E) == 448.0
    assert orc.e4m3_to_f32(0xFE) == -448.0
    assert math.isnan(orc.e4m3_to_f32(0x7F))
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([orc.e4m3_to_f32(int(c)) for c in codes], np.float32)
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~fin)
    assert np.array_equal(got[fin], ref[fin])


def test_e4m3_encode_roundtrip_ties_and_saturation(orc):
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    for c in finite:
        v = orc.e4m3_to_f32(c)
        assert orc.e4m3_from_f32(v) == c, hex(c)
    # midpoints between neighbouring positive codes round to the even mantissa
    for c in range(0, 0x7E):
        lo, hi = orc.e4m3_to_f32(c), orc.e4m3_to_f32(c + 1)
        mid = np.float32((lo + hi) / 2)
        want = c if c % 2 == 0 else c + 1
        assert orc.e4m3_from_f32(float(mid)) == want, hex(c)
    assert orc.e4m3_from_f32(449.0) == 0x7E
    assert orc.e4m3_from_f32(1e9) == 0x7E
    assert orc.e4m3_from_f32(-1e9) == 0xFE
    assert orc.e4m3_from_f32(2.0 ** -11) == 0x00          # below half the smallest subnormal
    assert orc.e4m3_from_f32(3 * 2.0 ** -11) == 0x01      # rounds up to 2^-9


def test_e4m3_encode_matches_torch_on_clamped_inputs(orc):
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(100000) * 100, rng.standard_normal(50000) * 0.01,
                        rng.uniform(-448, 448, 50000)]).astype(np.float32)
    v = np.clip(v, -448.0, 448.0)  # torch's cast does not saturate; compare inside the range
    got = orc.e4m3_from_f32_array(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
