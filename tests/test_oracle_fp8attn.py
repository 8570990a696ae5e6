"""Pins of the oracle's all-FP8 attention variant (no GPU): the query
quantised to e4m3 per row (s_q = amax / 448) and the probabilities quantised
to e4m3 per aligned 32-position block relative to the block's largest logit,
the softmax normaliser summing the unquantised probabilities.

Sources: "State of FP8 KV cache and attention quantization in vLLM"
(introduction: QK and ScoreV products in FP8, e4m3 throughout; the fixes
section: query quantisation fused ahead of the kernel); "cooking-agi: FP8 and
the KV cache", section "dynamic vs static scale" (the worked example whose
read-back values are used below). The scale rule for q and the block
reference for P are this library's reading of what the pages leave open.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from test_oracle_attention import bits, manual_case

FP8 = oracle.FP8


def fill_unit(case):
    """fp8 caches written with scale 1 (codes = the values when exact)."""
    kc = synth.poisoned_cache(case.num_pages, case.num_kv_heads, case.head_dim, True)
    vc = synth.poisoned_cache(case.num_pages, case.num_kv_heads, case.head_dim, True)
    one = np.ones(case.num_kv_heads, np.float32)
    oracle.kv_cache_write(kc, vc, case.k_new, case.v_new, case.slots, FP8, True, one, one)
    return kc, vc, one


def att8(case, kc, vc, s, window=0, sm_scale=1.0):
    return oracle.attention_fp8attn(case.q, kc, vc, case.block_tables, case.lens,
                                    case.num_kv_heads, FP8, True, window, sm_scale, s, s)


def test_zero_query_gives_the_window_mean():
    # every logit is 0: each block's reference is 0, p~ = e4m3(1) = 1
    r = np.random.default_rng(5)
    L, D = 77, 64
    v = np.round(r.standard_normal((L, 1, D)) * 4) / 4           # e4m3-exact values
    case = manual_case(1, 1, D, L, r.standard_normal((L, 1, D)), v, np.zeros((1, D)))
    kc, vc, one = fill_unit(case)
    for W in (0, 5, 40):
        out = att8(case, kc, vc, one, window=W)[0, 0]
        lo = L - W if W else 0
        assert np.allclose(out, v[lo:, 0].mean(axis=0), rtol=0, atol=1e-12), W


def test_single_position_returns_the_value():
    D = 64
    v = np.zeros((1, 1, D)); v[0, 0, :4] = [1.5, -0.25, 3.0, 448.0]
    case = manual_case(1, 1, D, 1, np.ones((1, 1, D)), v, np.ones((1, D)))
    kc, vc, one = fill_unit(case)
    assert np.array_equal(att8(case, kc, vc, one)[0, 0], v[0, 0])


def test_two_positions_in_one_block_quantise_p_but_not_the_normaliser():
    # q = 1.75 e_0: s_q = 1.75/448 = 2^-8 exactly and its code reads back
    # 1.75 exactly. k_0 = e_0, k_1 = 0.5 e_0, sm_scale 1: z = (1.75, 0.875).
    # In one block the reference is 1.75, so p = (1, e^-0.875 = 0.4169) and
    # p~ = (1, 0.40625), the nearest e4m3 value (0.40625 < 0.4169 < the
    # midpoint 0.421875 of 0.40625 and 0.4375).
    D = 64
    k = np.zeros((2, 1, D)); k[0, 0, 0] = 1.0; k[1, 0, 0] = 0.5
    v = np.zeros((2, 1, D)); v[0, 0, 1] = 2.0; v[1, 0, 1] = -4.0; v[1, 0, 2] = 1.0
    q = np.zeros((1, D)); q[0, 0] = 1.75
    case = manual_case(1, 1, D, 2, k, v, q)
    kc, vc, one = fill_unit(case)
    out = att8(case, kc, vc, one)[0, 0]
    e = math.exp(-0.875)
    assert 0.40625 < e < 0.421875
    want1 = (2.0 + 0.40625 * -4.0) / (1.0 + e)
    want2 = 0.40625 / (1.0 + e)
    assert abs(out[1] - want1) < 1e-14 and abs(out[2] - want2) < 1e-14
    # the unquantised softmax would give a different mix
    assert abs(out[1] - (2.0 + e * -4.0) / (1.0 + e)) > 1e-3


def test_positions_in_different_blocks_are_not_quantised_against_each_other():
    # window of 2 at positions 31, 32 (blocks 0 and 1): each block has one
    # position, p~ = 1, and the blocks merge exactly - the softmax itself.
    # The same logits at positions 30, 31 (one block) quantise the smaller p.
    D = 64
    for L, same_block in ((33, False), (32, True)):
        k = np.zeros((L, 1, D)); k[L - 2, 0, 0] = 1.0; k[L - 1, 0, 0] = 0.5
        v = np.zeros((L, 1, D)); v[L - 2, 0, 1] = 2.0; v[L - 1, 0, 1] = -4.0
        q = np.zeros((1, D)); q[0, 0] = 1.75
        case = manual_case(1, 1, D, L, k, v, q)
        kc, vc, one = fill_unit(case)
        out = att8(case, kc, vc, one, window=2)[0, 0, 1]
        e = math.exp(-0.875)
        exact = (2.0 + e * -4.0) / (1.0 + e)
        quant = (2.0 + 0.40625 * -4.0) / (1.0 + e)
        assert abs(out - (quant if same_block else exact)) < 1e-14, L


def test_query_quantisation_follows_the_worked_example():
    # q = (3.2, 0.01, -0.8, 0...) as bf16 (3.1875, 0.0099487, -0.796875):
    # s_q = amax / 448, and 0.01 gets code 0x3B as in the pages' dynamic-scale
    # example (which reads it back as 0.0098214 for the exact inputs; here
    # 1.375 * s_q). With k_0 = e_1, k_1 = 0 and sm_scale 1 the logits are
    # (1.375 s_q, 0): one block, reference 1.375 s_q, and e^-(1.375 s_q) =
    # 0.9903 quantises to 1.0 - so out = v_0 / (1 + 0.9903).
    D = 64
    q = np.zeros((1, D), np.float32); q[0, :3] = [3.2, 0.01, -0.8]
    qb = (bits(q).astype(np.uint32) << 16).view(np.float32)      # the bf16 values
    s_q = np.float32(qb[0, 0]) / np.float32(448)
    code = oracle.quantize_one(float(qb[0, 1]), float(s_q))
    assert code == 0x3B
    q_read = 1.375 * float(s_q)
    assert abs(q_read - 0.0098214) / 0.0098214 < 0.01
    k = np.zeros((2, 1, D)); k[0, 0, 1] = 1.0
    v = np.zeros((2, 1, D)); v[0, 0, 0] = 1.0
    case = manual_case(1, 1, D, 2, k, v, q)
    kc, vc, one = fill_unit(case)
    out = att8(case, kc, vc, one)[0, 0, 0]
    pz = math.exp(-q_read)
    assert oracle.e4m3_encode(np.float32(pz)) == oracle.e4m3_encode(1.0)
    assert abs(out - 1.0 / (1.0 + pz)) < 1e-14


def test_close_to_plain_attention_on_random_data():
    # not a pin of the definition: the two variants differ only by the e4m3
    # rounding of q and of p, a few per cent per term
    case = synth.decode_case(60, 8, 2, 128, [300], values="normal")
    ks = oracle.scale_from_amax(case.k_new, True)
    vs = oracle.scale_from_amax(case.v_new, True)
    kc = synth.poisoned_cache(case.num_pages, 2, 128, True)
    vc = synth.poisoned_cache(case.num_pages, 2, 128, True)
    oracle.kv_cache_write(kc, vc, case.k_new, case.v_new, case.slots, FP8, True, ks, vs)
    a = oracle.attention(case.q, kc, vc, case.block_tables, case.lens, 2, FP8, True, 0, 0.0,
                         ks, vs)
    b = oracle.attention_fp8attn(case.q, kc, vc, case.block_tables, case.lens, 2, FP8, True,
                                 0, 0.0, ks, vs)
    d = np.abs(a - b)
    assert d.max() < 0.05 and d.max() > 0


# ------------------------------------ second formulation: numpy brute force --
def _e4m3_encode(x32):
    """Saturating round-to-nearest-even e4m3 codes of float32 values, written
    from the format's value table (torch's float8_e4m3fn decode of the 256
    codes, independent of the oracle's codec): the nearest representable
    magnitude, a tie going to the even code (even mantissa), |x| >= 448 to
    448, the sign bit from x."""
    from test_oracle_attention import _decode_table
    pos = _decode_table(FP8)[:0x7F]                       # codes 0x00..0x7E, 0 .. 448
    x32 = np.asarray(x32, np.float32)
    a = np.minimum(np.abs(x32.astype(np.float64)), 448.0)
    i = np.clip(np.searchsorted(pos, a), 1, 0x7E)        # pos[i-1] <= a <= pos[i]
    lo, hi = pos[i - 1], pos[i]
    up = (hi - a < a - lo) | ((hi - a == a - lo) & (i % 2 == 0))
    code = np.where(up, i, i - 1).astype(np.uint8)
    return np.where(np.signbit(x32), code | 0x80, code).astype(np.uint8)


def _fp8attn_brute(case, kc, vc, dtype, ks, vs, window, reference="block"):
    """All-FP8 decode attention in vectorised numpy float64, on the same cache
    codes: q per row as e4m3 codes of fp32(q / s_q), s_q = fp32(amax) / 448;
    logits (q~ s_q) . (k~ s_k) / sqrt(D); P = e4m3(fp32(exp(z - M))). With
    reference "block", M is the largest logit of the position's aligned
    32-position block and the blocks merge with weights e^(M_j - M); with
    "row", M is the row's largest logit (the plain reading). The normaliser
    sums the unquantised exp(z - M) either way."""
    from test_oracle_attention import _decode_table, _layout_offsets
    B, Hq, D = case.q.shape
    Hkv = case.num_kv_heads
    G = Hq // Hkv
    koff, voff = _layout_offsets(D, 1)
    tab = _decode_table(dtype)
    t8 = _decode_table(FP8)
    kx = tab[kc[:, :, koff]] * np.asarray(ks, np.float64)[None, :, None, None]
    vx = tab[vc[:, :, voff]] * np.asarray(vs, np.float64)[None, :, None, None]
    q32 = synth.bits_to_f32(case.q)
    sq = np.abs(q32).max(axis=2).astype(np.float32) / np.float32(448.0)         # [B][Hq]
    qv = t8[_e4m3_encode(q32 / sq[:, :, None])] * sq[:, :, None].astype(np.float64)
    out = np.zeros((B, Hq, D))
    for b, L in enumerate(case.lens):
        lo = max(0, L - window) if window else 0
        t = np.arange(lo, L)
        if t.size == 0:
            continue
        pages = case.block_tables[b, t // 16]
        for h in range(Hkv):
            kt = kx[pages, h, t % 16]
            vt = vx[pages, h, t % 16]
            z = qv[b, h * G:(h + 1) * G] @ kt.T / math.sqrt(D)                # [G][n]
            if reference == "row":
                e = np.exp(z - z.max(axis=1, keepdims=True))
                p = t8[_e4m3_encode(e.astype(np.float32))]
                out[b, h * G:(h + 1) * G] = (p @ vt) / e.sum(axis=1, keepdims=True)
                continue
            blk = t // 32 - t[0] // 32
            nb = blk[-1] + 1
            mb = np.full((G, nb), -np.inf)
            for j in range(nb):
                mb[:, j] = z[:, blk == j].max(axis=1)
            e = np.exp(z - mb[:, blk])
            p = t8[_e4m3_encode(e.astype(np.float32))]
            w = np.exp(mb - mb.max(axis=1, keepdims=True))[:, blk]             # e^(M_j - M)
            out[b, h * G:(h + 1) * G] = ((p * w) @ vt) / (e * w).sum(axis=1, keepdims=True)
    return out


def test_e4m3_encoder_of_the_brute_force():
    # the table encoder against the pages' worked example and the format's
    # rounding rules (ties to even, saturation, subnormals)
    assert _e4m3_encode(np.float32(0.01) / (np.float32(3.2) / np.float32(448))) == 0x3B
    assert _e4m3_encode(np.float32(0.40625)) == oracle.e4m3_encode(0.40625)
    assert _e4m3_encode(np.float32(1000.0)) == 0x7E and _e4m3_encode(np.float32(-500)) == 0xFE
    assert _e4m3_encode(np.float32(1.0625)) == 0x38       # tie 1.0 / 1.125 -> even code
    assert _e4m3_encode(np.float32(1.1875)) == 0x3A       # tie 1.125 / 1.25 -> even code
    assert _e4m3_encode(np.float32(2.0 ** -10)) == 0x00   # tie 0 / 2^-9 -> 0
    assert _e4m3_encode(np.float32(3 * 2.0 ** -10)) == 0x02
    r = np.random.default_rng(3)
    x = (r.standard_normal(20000) * 8).astype(np.float32)
    want = np.array([oracle.e4m3_encode(v) for v in x[:2000]], np.uint8)
    assert np.array_equal(_e4m3_encode(x[:2000]), want)


FP8ATTN_CASES = {
    # name: (seed, Hq, Hkv, D, lens, values, dtype, windows, k-scale factors, v-scale factors)
    "tiny": (61, 4, 2, 64, [256], "tiny", FP8, (0,), [1, 3], [2, 0.5]),
    "gqa4_ragged_window": (62, 16, 4, 64, [300, 77, 513, 16, 1], "tiny", FP8, (0, 100, 33),
                           [1, 2.5, 0.3, 7], [4, 0.2, 1, 9]),
    "g8_drift": (63, 16, 2, 128, [2100], "drift", FP8, (0,), [1, 0.5], [1, 2]),
    "e5m2": (64, 8, 2, 64, [150, 260], "tiny", oracle.E5M2, (0,), [1, 40], [30, 1]),
}


@pytest.mark.parametrize("name", sorted(FP8ATTN_CASES))
def test_fp8attn_matches_a_numpy_brute_force(name):
    """The oracle's all-FP8 attention against a second, vectorised
    formulation on the same codes, with distinct static scales per KV head.
    The plain reading (P relative to the row's largest logit instead of its
    32-position block's) is computed beside it and its distance reported:
    both readings quantise the same products, and the block reading keeps
    more of each block's small probabilities above the e4m3 subnormal range."""
    seed, Hq, Hkv, D, lens, values, dtype, windows, kf, vf = FP8ATTN_CASES[name]
    case = synth.decode_case(seed, Hq, Hkv, D, lens, shuffle=True, spare_frac=0.2, values=values)
    ks = oracle.scale_from_amax(case.k_new, True, fmt=dtype) * np.array(kf, np.float32)
    vs = oracle.scale_from_amax(case.v_new, True, fmt=dtype) * np.array(vf, np.float32)
    kc = synth.poisoned_cache(case.num_pages, Hkv, D, True)
    vc = kc.copy()
    oracle.kv_cache_write(kc, vc, case.k_new, case.v_new, case.slots, dtype, True, ks, vs)
    for w in windows:
        got = oracle.attention_fp8attn(case.q, kc, vc, case.block_tables, case.lens, Hkv, dtype,
                                       True, w, 0.0, ks, vs)
        want = _fp8attn_brute(case, kc, vc, dtype, ks, vs, w)
        scale = max(1.0, np.max(np.abs(want)))
        assert np.max(np.abs(got - want)) / scale <= 1e-12, (name, w)
        plain = _fp8attn_brute(case, kc, vc, dtype, ks, vs, w, reference="row")
        exact = oracle.attention(case.q, kc, vc, case.block_tables, case.lens, Hkv, dtype,
                                 True, w, 0.0, ks, vs)
        e_block = np.abs(got - exact)
        e_plain = np.abs(plain - exact)
        print(f"[fp8attn {name} window {w}] block vs plain max {np.max(np.abs(got - plain)):.3e}; "
              f"vs bf16-arithmetic attention: block max {e_block.max():.3e} mean "
              f"{e_block.mean():.3e}, plain max {e_plain.max():.3e} mean {e_plain.mean():.3e} "
              f"(output scale {scale:.2f})")
        assert e_block.mean() <= e_plain.mean() * 1.5 + 1e-12, (name, w)
