"""Pins of the oracle's E5M2 codec, quantisation, scale calibration and cache
write (no GPU).

Sources: "FP8量化与长上下文推理" section 1 (format table: 5 exponent bits, 2
mantissa bits, range about +-57344) and section 1.1 (s = max_abs / fmax,
round(x / s)); "cooking-agi: FP8 and the KV cache", section "how to enable it
in the engine" (fp8_e5m2 as a KV-cache dtype) and section "dynamic vs static
scale" (saturating conversion). Bias 15, infinities and NaN patterns are the
OCP definition.
"""

import math
import struct

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import e4m3_table as tables
from oracle import BF16, E5M2


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bits(x_f32):
    return synth.bf16_bits(np.asarray(x_f32, np.float32))


# ---------------------------------------------------------------- decode ---
def test_decode_matches_formula_table_and_torch():
    c_tab = oracle.e5m2_decode_all()
    py_tab = tables.e5m2_table()
    torch_tab = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()
    for c in range(256):
        a, b, t = c_tab[c], py_tab[c], torch_tab[c]
        if math.isnan(b):
            assert math.isnan(a) and math.isnan(t), c
        else:
            assert a == b == t, (c, a, b, t)
            assert math.copysign(1, a) == math.copysign(1, b), c


def test_format_constants():
    tab = oracle.e5m2_decode_all()
    assert tab[0x7B] == 57344.0 and tab[0xFB] == -57344.0      # largest finite
    assert tab[0x01] == 2.0 ** -16                              # smallest subnormal
    assert tab[0x04] == 2.0 ** -14                              # smallest normal
    assert tab[0x7C] == math.inf and tab[0xFC] == -math.inf
    assert [c for c in range(256) if math.isnan(tab[c])] == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]
    assert np.isfinite(tab).sum() == 248
    pos = tab[:0x7C]
    assert np.all(np.diff(pos) > 0)
    # 2 mantissa bits: 4 codes per binade above the subnormals
    assert tab[0x44] == 2 * tab[0x40] and tab[0x41] == 1.25 * tab[0x40]


# ---------------------------------------------------------------- encode ---
def test_encode_round_trip_all_finite_codes():
    tab = oracle.e5m2_decode_all()
    for c in range(256):
        if not np.isfinite(tab[c]):
            continue
        assert oracle.e5m2_encode(float(tab[c])) == c, hex(c)


def test_encode_special_values():
    assert oracle.e5m2_encode(float("inf")) == 0x7B                 # saturates
    assert oracle.e5m2_encode(float("-inf")) == 0xFB
    assert oracle.e5m2_encode(60000.0) == 0x7B
    assert oracle.e5m2_encode(-1e30) == 0xFB
    assert oracle.e5m2_encode(float("nan")) == 0x7F
    assert oracle.e5m2_encode(-float("nan")) == 0xFF
    assert oracle.e5m2_encode(0.0) == 0x00
    assert oracle.e5m2_encode(-0.0) == 0x80
    assert oracle.e5m2_encode(-1e-30) == 0x80
    assert oracle.e5m2_encode(2.0 ** -17) == 0x00                   # tie to even 0
    assert oracle.e5m2_encode(1.5 * 2.0 ** -16) == 0x02             # tie to even 2


def test_encode_ties_go_to_even_code():
    tab = oracle.e5m2_decode_all()
    for c in range(0, 0x7B):
        mid = 0.5 * (tab[c] + tab[c + 1])
        if f32(mid) != mid:
            continue
        want = c if c % 2 == 0 else c + 1
        assert oracle.e5m2_encode(mid) == want, hex(c)
        assert oracle.e5m2_encode(-mid) == want | 0x80, hex(c)
        below = float(np.nextafter(np.float32(mid), np.float32(0)))
        above = float(np.nextafter(np.float32(mid), np.float32(1e9)))
        assert oracle.e5m2_encode(below) == c
        assert oracle.e5m2_encode(above) == c + 1


def test_encode_matches_python_brute_force_on_samples():
    r = np.random.default_rng(17)
    xs = np.concatenate([
        r.standard_normal(300) * 1000.0,
        r.standard_normal(200) * 1e-3,
        r.uniform(-60000, 60000, 200),
        r.standard_normal(100) * 1e-5,
    ]).astype(np.float32)
    for x in xs:
        x = float(x)
        assert oracle.e5m2_encode(x) == tables.e5m2_nearest_code(x), x


def test_encode_scan_and_table_agree_on_samples():
    r = np.random.default_rng(19)
    xs = r.integers(0, 2 ** 32, size=5000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    for x in xs:
        x = float(x)
        assert oracle.e5m2_encode(x) == oracle.e5m2_encode_scan(x)


def test_encode_matches_torch_on_preclamped_inputs():
    # torch's float8_e5m2 cast rounds to nearest even but overflows to Inf,
    # so inputs are clamped to +-57344 first
    r = np.random.default_rng(23)
    xs = np.concatenate([
        r.standard_normal(20000) * 3000,
        r.standard_normal(20000) * 0.01,
        r.standard_normal(5000) * 1e-5,
        np.ldexp(1.0, np.arange(-18, 16)),
    ]).astype(np.float32)
    xs = np.clip(xs, -57344, 57344)
    t = torch.from_numpy(xs).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(t, oracle.quantize(xs, 1.0, fmt=E5M2))


def test_encoders_agree_on_sub_ranges():
    for lo in (0x37000000, 0x47000000, 0xB8000000):               # subnormals, top, negative
        bad, first = oracle.sweep_encoders(lo, lo + (1 << 24), fmt=E5M2)
        assert bad == 0, hex(first)
    bad, first = oracle.sweep_encoders(0x7F7F0000, 0x80000000 + (1 << 16), fmt=E5M2)
    assert bad == 0, hex(first)


@pytest.mark.slow
def test_encoders_agree_on_all_2_pow_32_inputs():
    bad, first = oracle.sweep_encoders(0, 1 << 32, fmt=E5M2)
    assert bad == 0, hex(first)


# ----------------------------------------------------------- quantisation --
def test_quantize_divides_in_fp32():
    # x / s in fp32 is exactly 1.875, the midpoint of 1.75 (0x3F) and 2.0
    # (0x40); the exact quotient lies just below it. An fp32 division ties to
    # the even code 0x40, a wider division would give 0x3F.
    x = struct.unpack("<f", struct.pack("<I", 0x3FD8F3F1))[0]
    s = struct.unpack("<f", struct.pack("<I", 0x3F676A9B))[0]
    assert float(np.float32(x) / np.float32(s)) == 1.875
    assert x / s < 1.875
    assert oracle.quantize_one(x, s, fmt=E5M2) == 0x40


def test_scale_from_amax_uses_the_e5m2_maximum():
    x = np.zeros((3, 2, 64), np.float32)
    x[1, 0, 5] = -3.2
    x[2, 1, 7] = 180.0
    s = oracle.scale_from_amax(bits(x), True, fmt=E5M2)
    k0 = (bits(np.array([-3.2], np.float32)).astype(np.uint32) << 16).view(np.float32)[0]
    assert s[0] == np.float32(abs(k0)) / np.float32(57344.0)
    assert s[1] == np.float32(180.0) / np.float32(57344.0)
    # the largest value lands on the largest finite code
    assert oracle.quantize_one(180.0, float(s[1]), fmt=E5M2) == 0x7B
    t = oracle.scale_from_amax(bits(x), False, fmt=E5M2)
    assert t.shape == (1,) and t[0] == s[1]


# ------------------------------------------------------------ cache write --
def test_cache_write_e5m2_touches_only_its_row():
    H, D, P = 2, 64, 3
    r = np.random.default_rng(29)
    k = bits(r.standard_normal((2, H, D)).astype(np.float32) * 100)
    v = bits(r.standard_normal((2, H, D)).astype(np.float32) * 100)
    slots = np.array([2 * 16 + 9, -1], dtype=np.int64)
    kc = synth.poisoned_cache(P, H, D, True)
    vc = synth.poisoned_cache(P, H, D, True)
    ks = np.array([0.5, 0.25], np.float32)
    vs = np.array([0.125, 2.0], np.float32)
    oracle.kv_cache_write(kc, vc, k, v, slots, E5M2, True, ks, vs)
    ref_k = synth.poisoned_cache(P, H, D, True)
    ref_v = synth.poisoned_cache(P, H, D, True)
    kf = (k.astype(np.uint32) << 16).view(np.float32)
    vf = (v.astype(np.uint32) << 16).view(np.float32)
    for h in range(H):
        for d in range(D):
            ref_k[2, h, oracle.k_offset(9, d, 1)] = tables.e5m2_nearest_code(
                float(np.float32(kf[0, h, d]) / np.float32(ks[h])))
            ref_v[2, h, oracle.v_offset(9, d, 1)] = tables.e5m2_nearest_code(
                float(np.float32(vf[0, h, d]) / np.float32(vs[h])))
    assert np.array_equal(kc, ref_k) and np.array_equal(vc, ref_v)


def test_single_position_attention_returns_the_dequantised_e5m2_value():
    # one attended position: the output is decode(code) * s_v exactly
    H, D = 1, 64
    tab = tables.e5m2_table()
    codes = np.array([c for c in range(256) if np.isfinite(tab[c])], np.uint8)
    kc = np.zeros((1, H, 16 * D), np.uint8)
    vc = np.zeros((1, H, 16 * D), np.uint8)
    for i in range(0, len(codes), D):
        chunk = codes[i:i + D]
        for d, c in enumerate(chunk):
            vc[0, 0, oracle.v_offset(0, d, 1)] = c
        q = bits(np.ones((1, 1, D), np.float32))
        out = oracle.attention(q, kc, vc, np.zeros((1, 1), np.int32), np.array([1], np.int32),
                               1, E5M2, True, 0, 0.0, np.array([1.0], np.float32),
                               np.array([0.5], np.float32))
        for d, c in enumerate(chunk):
            assert out[0, 0, d] == tab[c] * 0.5, hex(c)
