"""Pins of the oracle's dynamic per-token scales (no GPU).

Every new token gets its own scale, computed when it is written
("FP8量化与长上下文推理" section 2.2, per-token dynamic quantisation of the KV
cache); the token's largest magnitude lands on the format's largest value
("cooking-agi: FP8 and the KV cache", section "dynamic vs static scale",
worked example of tokens A and B). PER_TOKEN takes one scale per token over
all of its KV heads; PER_TOKEN_HEAD one per token and KV head. The scale of a
slot is stored beside the page: pool[page][head][row], one per K and V.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from test_oracle_attention import manual_case

E4M3, E5M2 = oracle.FP8, oracle.E5M2
PT, PTH = oracle.PER_TOKEN, oracle.PER_TOKEN_HEAD


def write_dyn(case, mode, dtype=E4M3):
    kc = synth.poisoned_cache(case.num_pages, case.num_kv_heads, case.head_dim, True)
    vc = synth.poisoned_cache(case.num_pages, case.num_kv_heads, case.head_dim, True)
    kp, vp = oracle.scale_pools(case.num_pages, case.num_kv_heads)
    oracle.kv_cache_write_dyn(kc, vc, case.k_new, case.v_new, case.slots, dtype, mode, kp, vp)
    return kc, vc, kp, vp


def codes_of(cache, is_v, D):
    """Codes of every (page, head, row, dim) through the layout: [P][H][16][D]."""
    off = np.array([[(oracle.v_offset if is_v else oracle.k_offset)(r, d, 1)
                     for d in range(D)] for r in range(16)])
    return cache[:, :, off]


def slot_view(arr, slots):
    """[P][H][16](...) -> [T][H](...) at the given slots."""
    return arr[slots // 16, :, slots % 16]


def bf16_row(vals, D):
    row = np.zeros(D, np.float32)
    row[:len(vals)] = vals
    return synth.bf16_bits(row)


# ------------------------------------------------ the worked example -------
@pytest.mark.parametrize("mode", [PT, PTH])
def test_worked_example_tokens(golden_dir, mode):
    with open(os.path.join(golden_dir, "worked_scale_example.json")) as f:
        g = json.load(f)
    D = 64
    A, B = g["tokens"]["A"], g["tokens"]["B"]
    # head 0 holds the page's token, head 1 smaller values of its own
    k = np.stack([np.stack([bf16_row(A, D), bf16_row([0.5, -0.25], D)]),
                  np.stack([bf16_row(B, D), bf16_row([1.0, 3.0], D)])])
    case = manual_case(1, 2, D, 2, synth.bits_to_f32(k), synth.bits_to_f32(k), np.zeros((1, D)))
    kc, vc, kp, vp = write_dyn(case, mode)
    dec = oracle.e4m3_decode_all()
    ks = slot_view(kp, case.slots)                     # [2 tokens][2 heads]
    assert np.array_equal(ks, slot_view(vp, case.slots))
    a_max = float(synth.bits_to_f32(bf16_row([3.2], 1))[0])
    assert ks[0, 0] == np.float32(a_max) / np.float32(448.0)
    assert ks[1, 0] == np.float32(180.0) / np.float32(448.0)
    dyn = g["dynamic_per_token"]
    assert abs(ks[1, 0] - dyn["B"]["scale_printed"]) <= dyn["B"]["scale_tol"]
    # per token: one scale for both heads; per token and head: head 1 its own
    if mode == PT:
        assert ks[0, 1] == ks[0, 0] and ks[1, 1] == ks[1, 0]
    else:
        assert ks[0, 1] == np.float32(0.5) / np.float32(448.0)
        assert ks[1, 1] == np.float32(3.0) / np.float32(448.0)
    for cache, is_v in ((kc, False), (vc, True)):
        c = slot_view(codes_of(cache, is_v, D), case.slots)     # [2][2][D]
        # A: 0.01 -> 0x3B (1.375), -0.8 -> -112, 3.2 -> 448; B: 2 -> 5, -45 -> -112, 180 -> 448
        assert list(c[0, 0, :3]) == [0x3B, 0xEE, 0x7E]
        assert list(c[1, 0, :3]) == [0x4A, 0xEE, 0x7E]
        # "0.01 reads back 0.0098"
        rb = dec[c[0, 0, 0]] * float(ks[0, 0])
        assert abs(rb - dyn["A"]["readback_printed"]["0.01"]) <= dyn["A"]["readback_tol"]
        # every value of both tokens reads back within half an e4m3 step
        x = synth.bits_to_f32(case.k_new).astype(np.float64)
        back = dec[c] * ks[:, :, None].astype(np.float64)
        nz = x != 0
        assert np.all(np.abs(back - x)[nz] <= np.abs(x[nz]) / 16 + 1e-300)


# ------------------------------------------------------ properties ---------
@pytest.mark.parametrize("mode", [PT, PTH])
@pytest.mark.parametrize("dtype", [E4M3, E5M2])
def test_each_token_max_lands_on_the_format_max(mode, dtype):
    case = synth.decode_case(71, 8, 4, 64, [300, 45], values="spread", shuffle=True,
                             spare_frac=0.2)
    kc, vc, kp, vp = write_dyn(case, mode, dtype)
    top = 0x7E if dtype == E4M3 else 0x7B
    dec = oracle.e4m3_decode_all() if dtype == E4M3 else oracle.e5m2_decode_all()
    fmax = 448.0 if dtype == E4M3 else 57344.0
    for cache, pool, x_bits, is_v in ((kc, kp, case.k_new, False), (vc, vp, case.v_new, True)):
        c = slot_view(codes_of(cache, is_v, 64), case.slots)       # [T][H][D]
        s = slot_view(pool, case.slots).astype(np.float64)         # [T][H]
        x = synth.bits_to_f32(x_bits).astype(np.float64)
        ax = np.abs(x)
        if mode == PT:
            amax = ax.max(axis=(1, 2))[:, None] * np.ones((1, x.shape[1]))
        else:
            amax = ax.max(axis=2)
        # the stored scale is fp32(amax) / fmax, and the largest element's code is the top one
        assert np.array_equal(s, (amax.astype(np.float32) / np.float32(fmax)).astype(np.float64))
        is_max = ax == amax[:, :, None]
        assert np.all((c[is_max] & 0x7F) == top)
        # every element reads back within half a step of its format (normal range)
        back = dec[c] * s[:, :, None]
        step = 1 / 16 if dtype == E4M3 else 1 / 8
        normal = ax >= (2.0 ** -6 if dtype == E4M3 else 2.0 ** -14) * s[:, :, None]
        assert np.all(np.abs(back - x)[normal] <= ax[normal] * step)


def test_per_token_and_per_token_head_agree_with_one_head():
    case = synth.decode_case(72, 2, 1, 128, [100], values="spread")
    a = write_dyn(case, PT)
    b = write_dyn(case, PTH)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_zero_and_nan_tokens():
    D = 64
    k = np.zeros((3, 1, D), np.float32)
    k[1, 0, 3] = 2.0
    k[2, 0, :] = 1.0
    k[2, 0, 7] = np.nan
    case = manual_case(1, 1, D, 3, k, k, np.zeros((1, D)))
    kc, vc, kp, vp = write_dyn(case, PTH)
    s = slot_view(kp, case.slots)[:, 0]
    c = slot_view(codes_of(kc, False, D), case.slots)[:, 0]
    assert s[0] == 1.0 and np.all(c[0] == 0)              # all-zero token: scale 1
    assert s[1] == np.float32(2.0) / np.float32(448.0) and c[1, 3] == 0x7E
    assert math.isnan(s[2]) and np.all((c[2] & 0x7F) == 0x7F)   # NaN scale, NaN codes


def test_skipped_slots_leave_cache_and_pools_alone():
    case = synth.decode_case(73, 4, 2, 64, [40])
    slots = case.slots.copy()
    slots[5] = -1
    slots[6] = case.num_pages * 16 + 3
    kc = synth.poisoned_cache(case.num_pages, 2, 64, True)
    vc = kc.copy()
    kp, vp = oracle.scale_pools(case.num_pages, 2)
    kp[:] = 7.0
    oracle.kv_cache_write_dyn(kc, vc, case.k_new, case.v_new, slots, E4M3, PTH, kp, vp)
    p, r = case.slots[5] // 16, case.slots[5] % 16
    assert np.all(kp[p, :, r] == 7.0)
    assert np.all(codes_of(kc, False, 64)[p, :, r] == synth.POISON_FP8)


# ------------------------------------------------------- attention ---------
def attend(case, kc, vc, mode, ks, vs, window=0):
    return oracle.attention(case.q, kc, vc, case.block_tables, case.lens, case.num_kv_heads,
                            E4M3, mode, window, 0.0, ks, vs)


def test_attention_with_equal_token_scales_is_the_static_attention():
    # every (token, head) row has the same largest magnitude (dim 0 = +-5),
    # so every dynamic scale is 5/448: the same codes and the same arithmetic
    # as a static per-head scale of 5/448
    case = synth.decode_case(74, 8, 2, 64, [200, 33], shuffle=True)
    for x in (case.k_new, case.v_new):
        f = np.clip(synth.bits_to_f32(x), -4.0, 4.0)
        f[:, :, 0] = np.where(f[:, :, 0] < 0, -5.0, 5.0)
        x[:] = synth.bf16_bits(f)
    kc, vc, kp, vp = write_dyn(case, PTH)
    s = np.full(2, np.float32(5.0) / np.float32(448.0), np.float32)
    kc2 = synth.poisoned_cache(case.num_pages, 2, 64, True)
    vc2 = kc2.copy()
    oracle.kv_cache_write(kc2, vc2, case.k_new, case.v_new, case.slots, E4M3, True, s, s)
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)
    assert np.array_equal(attend(case, kc, vc, PTH, kp, vp), attend(case, kc2, vc2, True, s, s))


@pytest.mark.parametrize("mode", [PT, PTH])
def test_attention_reads_each_slots_own_scale(mode):
    # brute force from the definition: every attended value is decode(code)
    # times the scale stored for its own (page, head, row), read here through
    # the layout; logits and softmax in float64
    case = synth.decode_case(75, 8, 2, 64, [700, 90], values="spread", shuffle=True,
                             spare_frac=0.1)
    kc, vc, kp, vp = write_dyn(case, mode)
    dec = oracle.e4m3_decode_all()
    kx = dec[slot_view(codes_of(kc, False, 64), case.slots)] * \
        slot_view(kp, case.slots)[:, :, None].astype(np.float64)
    vx = dec[slot_view(codes_of(vc, True, 64), case.slots)] * \
        slot_view(vp, case.slots)[:, :, None].astype(np.float64)
    qf = synth.bits_to_f32(case.q).astype(np.float64)
    for window in (0, 50):
        out = attend(case, kc, vc, mode, kp, vp, window)
        start = 0
        for b, L in enumerate(case.lens):
            lo = max(0, L - window) if window else 0
            for i in range(8):
                z = kx[start + lo:start + L, i // 4] @ qf[b, i] / 8.0
                ref = oracle.softmax_weighted_sum(z, vx[start + lo:start + L, i // 4])
                assert np.allclose(out[b, i], ref, rtol=1e-9, atol=1e-12), (b, i, window)
            start += L


def test_small_tokens_keep_their_precision_with_dynamic_scales():
    # The contrast of the worked example and of the scale-1.0 remark
    # ("cooking-agi", sections "dynamic vs static scale" and "how to enable
    # it in the engine") in attention form: one large V token (about 1e3)
    # sets a static per-head scale below whose smallest subnormal every other
    # token (about 1e-4) falls, so they read back as zero; a window that skips
    # the large token attends only to small ones. Reference: float64
    # attention over the bf16 values.
    L, D, W = 300, 64, 299
    r = np.random.default_rng(11)
    k = r.standard_normal((L, 1, D)) * 0.5
    v = r.standard_normal((L, 1, D)) * 1e-4
    v[0] *= 1e7
    q = r.standard_normal((4, D))
    case = manual_case(4, 1, D, L, k, v, q)
    kf = synth.bits_to_f32(case.k_new).astype(np.float64)
    vf = synth.bits_to_f32(case.v_new).astype(np.float64)
    qf = synth.bits_to_f32(case.q).astype(np.float64)
    ref = np.stack([oracle.softmax_weighted_sum(kf[L - W:, 0] @ qf[0, i] / 8.0, vf[L - W:, 0])
                    for i in range(4)])
    kc, vc, kp, vp = write_dyn(case, PTH)
    err_dyn = np.abs(attend(case, kc, vc, PTH, kp, vp, W)[0] - ref).max()
    s_k = oracle.scale_from_amax(case.k_new, True)
    s_v = oracle.scale_from_amax(case.v_new, True)
    kc2 = synth.poisoned_cache(case.num_pages, 1, D, True)
    vc2 = kc2.copy()
    oracle.kv_cache_write(kc2, vc2, case.k_new, case.v_new, case.slots, E4M3, True, s_k, s_v)
    err_static = np.abs(attend(case, kc2, vc2, True, s_k, s_v, W)[0] - ref).max()
    # each attended value reads back within 1/16 of itself, so the weighted
    # mean moves by at most 1/16 of the largest attended |v| (plus the K side)
    vmax = np.abs(vf[L - W:]).max()
    mag = np.abs(ref).max()
    assert err_dyn < vmax / 16, (err_dyn, vmax)
    assert err_static > 0.9 * mag, (err_static, mag)          # the output is lost
    assert np.all(attend(case, kc2, vc2, True, s_k, s_v, W) == 0.0)
