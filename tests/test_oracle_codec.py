"""Pins of the oracle's e4m3 codec, quantisation and scale calibration against
what the pages and the format definition fix (no GPU).

Sources: "FP8量化与长上下文推理" section 1 (format table) and 1.1 (s = max_abs /
448, round(x / s)); "cooking-agi: FP8 and the KV cache", sections "dynamic vs
static scale" (worked example, saturation) and "how to enable it in the
engine" (smallest subnormal, scale 1.0 remark).
"""

import json
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3_table


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f32_div(a, b):
    return float(np.float32(a) / np.float32(b))


# ---------------------------------------------------------------- decode ---
def test_decode_matches_formula_table_and_torch():
    c_tab = oracle.e4m3_decode_all()
    py_tab = e4m3_table.table()
    codes = torch.arange(256, dtype=torch.uint8)
    torch_tab = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        a, b, t = c_tab[c], py_tab[c], torch_tab[c]
        if math.isnan(b):
            assert math.isnan(a) and math.isnan(t), c
        else:
            assert a == b == t, (c, a, b, t)
            assert math.copysign(1, a) == math.copysign(1, b), c


def test_format_constants():
    tab = oracle.e4m3_decode_all()
    assert tab[0x7E] == 448.0 and tab[0xFE] == -448.0          # largest finite
    assert tab[0x01] == 2.0 ** -9                               # smallest subnormal
    assert abs(tab[0x01] - 0.00195) < 5e-6                      # printed "≈0.00195"
    assert np.isfinite(tab).sum() == 254
    assert [c for c in range(256) if math.isnan(tab[c])] == [0x7F, 0xFF]
    assert tab[0x08] == 2.0 ** -6                               # smallest normal
    # 4 exponent bits, 3 mantissa bits: 8 codes per binade above the subnormals
    pos = tab[:0x7F]
    assert np.all(np.diff(pos) > 0)


# ---------------------------------------------------------------- encode ---
def test_encode_round_trip_all_finite_codes():
    tab = oracle.e4m3_decode_all()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(float(tab[c])) == c, hex(c)


def test_encode_special_values():
    assert oracle.e4m3_encode(float("inf")) == 0x7E
    assert oracle.e4m3_encode(float("-inf")) == 0xFE
    assert oracle.e4m3_encode(500.0) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(float("nan")) == 0x7F
    assert oracle.e4m3_encode(-float("nan")) == 0xFF
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-30) == 0x80
    # midpoint between 448 and the next binade step (480) still rounds to 448
    assert oracle.e4m3_encode(463.99) == 0x7E


def test_encode_ties_go_to_even_code():
    tab = oracle.e4m3_decode_all()
    for c in range(0, 0x7E):
        mid = 0.5 * (tab[c] + tab[c + 1])
        if f32(mid) != mid:
            continue
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == want, hex(c)
        assert oracle.e4m3_encode(-mid) == want | 0x80, hex(c)
        # just off the midpoint goes to the nearer side
        below = float(np.nextafter(np.float32(mid), np.float32(0)))
        above = float(np.nextafter(np.float32(mid), np.float32(1e9)))
        assert oracle.e4m3_encode(below) == c
        assert oracle.e4m3_encode(above) == c + 1


def test_encode_matches_python_brute_force_on_samples():
    r = np.random.default_rng(7)
    xs = np.concatenate([
        r.standard_normal(300) * 10.0,
        r.standard_normal(200) * 1e-3,
        r.uniform(-500, 500, 200),
        r.standard_normal(100) * 1e-6,
    ]).astype(np.float32)
    for x in xs:
        x = float(x)
        assert oracle.e4m3_encode(x) == e4m3_table.nearest_code(x), x


def test_encode_scan_and_table_agree_on_samples():
    r = np.random.default_rng(11)
    bits = r.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    xs = bits.view(np.float32)
    for x in xs[:5000]:
        x = float(x)
        assert oracle.e4m3_encode(x) == oracle.e4m3_encode_scan(x)


def test_encode_matches_torch_on_preclamped_inputs():
    # torch's float8_e4m3fn cast rounds to nearest even but does not saturate
    # (values past 464 become NaN), so inputs are clamped to +-448 first.
    r = np.random.default_rng(3)
    xs = np.concatenate([
        r.standard_normal(20000) * 50,
        r.standard_normal(20000) * 0.01,
        r.standard_normal(5000) * 1e-4,
        np.ldexp(1.0, np.arange(-14, 9)),                      # binade edges
    ]).astype(np.float32)
    xs = np.clip(xs, -448, 448)
    t = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.quantize(xs, 1.0)
    assert np.array_equal(t, ours)


@pytest.mark.slow
def test_encoders_agree_on_all_2_pow_32_inputs():
    bad, first = oracle.sweep_encoders(0, 1 << 32)
    assert bad == 0, hex(first)


def test_encoders_agree_on_sub_ranges():
    # quick version of the exhaustive sweep for the default CPU run: the
    # subnormal range, the top binades, negative values and Inf/NaN patterns
    bad, first = oracle.sweep_encoders(0x3A800000, 0x3A800000 + (1 << 24))
    assert bad == 0, hex(first)
    bad, first = oracle.sweep_encoders(0x43000000, 0x43000000 + (1 << 24))
    assert bad == 0, hex(first)
    bad, first = oracle.sweep_encoders(0xBB000000, 0xBB000000 + (1 << 24))
    assert bad == 0, hex(first)
    bad, first = oracle.sweep_encoders(0x7F7F0000, 0x80000000 + (1 << 16))
    assert bad == 0, hex(first)


# --------------------------------------------------------- worked example --
def _golden(golden_dir):
    with open(os.path.join(golden_dir, "worked_scale_example.json")) as f:
        return json.load(f)


def _readback(x, s):
    return oracle.e4m3_decode_all()[oracle.quantize_one(x, s)] * s


def test_worked_example_dynamic_scales(golden_dir):
    g = _golden(golden_dir)
    A, B = g["tokens"]["A"], g["tokens"]["B"]
    dA, dB = g["dynamic_per_token"]["A"], g["dynamic_per_token"]["B"]
    sA = f32_div(dA["amax"], g["e4m3_max"])
    sB = f32_div(dB["amax"], g["e4m3_max"])
    assert abs(sA - dA["scale_printed"]) <= dA["scale_tol"]
    assert abs(sB - dB["scale_printed"]) <= dB["scale_tol"]
    # each token's maximum lands exactly on 448
    assert oracle.quantize_one(3.2, sA) == 0x7E
    assert oracle.quantize_one(180.0, sB) == 0x7E
    # 0.01 in A reads back 0.0098
    rb = _readback(0.01, sA)
    assert abs(rb - dA["readback_printed"]["0.01"]) <= dA["readback_tol"]
    # "all read back accurately": within half an e4m3 step (2^-4 relative)
    for x, s in [(v, sA) for v in A] + [(v, sB) for v in B]:
        assert abs(_readback(x, s) - x) <= abs(x) * 2.0 ** -4 + 1e-12, x


def test_worked_example_static_scale(golden_dir):
    g = _golden(golden_dir)["static_per_tensor"]
    s = f32_div(g["amax"], 448.0)
    assert abs(s - g["scale_printed"]) <= g["scale_tol"]
    rb = _readback(0.01, s)
    assert abs(rb - g["A_readback_printed"]["0.01"]) <= g["A_readback_tol"]
    assert abs((rb - 0.01) / 0.01 - g["A_rel_error_printed"]) <= g["A_rel_error_tol"]
    y = f32_div(180.0, s)
    assert abs(y - g["B_180_over_s_printed"]) <= g["B_180_over_s_tol"]
    code = oracle.quantize_one(180.0, s)
    assert oracle.e4m3_decode_all()[code] == g["B_180_saturates_to"]
    assert abs(_readback(180.0, s) - g["B_180_readback_printed"]) < 1e-4
    # "A is fine": within half an e4m3 step
    for x in (-0.8, 3.2):
        assert abs(_readback(x, s) - x) <= abs(x) * 2.0 ** -4


def test_worked_example_codes_derived_by_hand():
    # Each code below follows from the format by hand (value / s, then the
    # nearest of the representable values, ties to the even mantissa).
    sA, sB, sS = f32_div(3.2, 448), f32_div(180, 448), f32_div(120, 448)
    # 0.01 / sA = 1.4: between 1.375 (e=7,m=3) and 1.5 -> 1.375 = 0x3B
    assert oracle.quantize_one(0.01, sA) == 0x3B
    # -0.8 / sA = -112 = -1.75 * 2^6 (e=13, m=6) -> 0xEE
    assert oracle.quantize_one(-0.8, sA) == 0xEE
    # 2.0 / sB = 4.978: between 4.5 and 5.0 (=1.25 * 4, e=9, m=2) -> 0x4A
    assert oracle.quantize_one(2.0, sB) == 0x4A
    # 0.01 / sS = 0.03733 = 1.1947 * 2^-5: nearer 1.25 (m=2) -> e=2 -> 0x12
    assert oracle.quantize_one(0.01, sS) == 0x12
    # 2.0 / sS = 7.4667 = 1.8667 * 4 -> 1.875 (m=7), e=9 -> 0x4F
    assert oracle.quantize_one(2.0, sS) == 0x4F


def test_fp32_division_decides_the_tie():
    # -45 / fp32(120/448) is exactly -168.0 in fp32: the midpoint of 160
    # (mantissa 2) and 176 (mantissa 3), so the even code 0xF2 (-160) wins.
    # A float64 division gives -168.0000053 and would round to 0xF3 (-176).
    s = np.float32(120) / np.float32(448)
    assert np.float32(-45) / s == np.float32(-168.0)
    assert oracle.quantize_one(-45.0, float(s)) == 0xF2
    assert e4m3_table.nearest_code(-45.0 / float(s)) == 0xF3


def test_scale_one_subnormal_remark(golden_dir):
    g = _golden(golden_dir)["scale_one"]
    tab = oracle.e4m3_decode_all()
    c = oracle.quantize_one(g["x_rounds_up_to_min_subnormal"], 1.0)
    assert tab[c] == g["min_subnormal"]
    assert (tab[c] - 0.001) / 0.001 > 0.9                        # "nearly double"
    assert oracle.quantize_one(0.0009, 1.0) == 0x00              # "becomes 0"
    assert oracle.quantize_one(2.0 ** -10, 1.0) == 0x00          # tie -> even 0
    assert oracle.quantize_one(-0.0009, 1.0) == 0x80


def test_quantize_divides_in_fp32():
    r = np.random.default_rng(5)
    x = (r.standard_normal(4000) * 3).astype(np.float32)
    for s in (1.0, 0.0071428573, 0.2678571343, 3.0e-3):
        q = oracle.quantize(x, s)
        y = (x / np.float32(s)).astype(np.float32)
        want = np.array([e4m3_table.nearest_code(float(v)) for v in y[:400]])
        assert np.array_equal(q[:400], want)


# ----------------------------------------------------------- scale setup ---
def _bits(a):
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_scale_from_amax_worked_example():
    # the tokens of the worked example as one head ([T=2][H=1][D=3]); amax is
    # taken over bf16 values, so 180 is exact and s = 180/448 in fp32
    x = _bits([[[0.01, -0.8, 3.2]], [[2.0, -45.0, 180.0]]])
    s = oracle.scale_from_amax(x, per_head=True)
    assert s[0] == np.float32(180.0) / np.float32(448.0)
    assert abs(float(s[0]) - 0.402) < 5e-4


def test_scale_from_amax_per_head_and_per_tensor():
    r = np.random.default_rng(9)
    T, H, D = 37, 3, 64
    x = (r.standard_normal((T, H, D)) * np.array([1, 5, 0.1])[None, :, None])
    xb = _bits(x.astype(np.float32))
    vals = (xb.astype(np.uint32) << 16).view(np.float32)
    ph = oracle.scale_from_amax(xb, per_head=True)
    pt = oracle.scale_from_amax(xb, per_head=False)
    for h in range(H):
        assert ph[h] == np.float32(np.abs(vals[:, h, :]).max()) / np.float32(448)
    assert pt[0] == np.float32(np.abs(vals).max()) / np.float32(448)
    assert pt[0] == ph.max()


def test_scale_from_amax_degenerate():
    z = np.zeros((4, 2, 64), dtype=np.uint16)
    assert np.all(oracle.scale_from_amax(z, True) == 1.0)
    n = z.copy()
    n[1, 1, 3] = 0x7FC0                                           # NaN
    s = oracle.scale_from_amax(n, True)
    assert s[0] == 1.0 and math.isnan(s[1])
    # max maps to 448 exactly: quantising the amax value gives 0x7E
    xb = _bits(np.array([[[-7.5, 1.0]]], dtype=np.float32))
    s = oracle.scale_from_amax(xb, True)
    assert oracle.quantize_one(-7.5, float(s[0])) == 0xFE


def test_quantize_is_a_true_division_not_a_reciprocal_multiply():
    # x / s is exactly 1.9375 in IEEE fp32: the midpoint of 1.875 (0x3F) and
    # 2.0 (0x40), so the tie goes to the even code 0x40. Multiplying by the
    # fp32 reciprocal of s lands one ulp below and would give 0x3F.
    x = np.array([0x40136FCC], np.uint32).view(np.float32)[0]
    s = np.array([0x3F983157], np.uint32).view(np.float32)[0]
    assert x / s == np.float32(1.9375)
    assert x * (np.float32(1) / s) != np.float32(1.9375)
    assert oracle.quantize_one(float(x), float(s)) == 0x40
