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
