"""Pins of the oracle's cache write and decode attention (no GPU).

Each test checks the oracle against a closed form, an invariant of softmax
attention or a special case, chosen so that a plausible mistake (a dropped
scale, a wrong sign, a wrong head / page / row index, a transposed operand,
an off-by-one window) fails at least one of them.

Definitions: "State of FP8 KV cache and attention quantization in vLLM",
section "Kernel and vLLM improvements" (per-head scales, two-level
accumulation) and section "Single-request benchmark" (online softmax
rescaling); the in-page layout is the one the library header documents.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

FP8, BF16 = oracle.FP8, oracle.BF16


def bits(a):
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def fill(case, fp8=True, per_head=True, ks=None, vs=None):
    """Poisoned caches with every position of the case written."""
    kc = synth.poisoned_cache(case.num_pages, case.num_kv_heads, case.head_dim, fp8)
    vc = synth.poisoned_cache(case.num_pages, case.num_kv_heads, case.head_dim, fp8)
    if fp8:
        ks = oracle.scale_from_amax(case.k_new, per_head) if ks is None else ks
        vs = oracle.scale_from_amax(case.v_new, per_head) if vs is None else vs
    oracle.kv_cache_write(kc, vc, case.k_new, case.v_new, case.slots,
                          FP8 if fp8 else BF16, per_head, ks, vs)
    return kc, vc, ks, vs


def att(case, kc, vc, fp8=True, per_head=True, ks=None, vs=None, window=0,
        sm_scale=0.0, q=None, lens=None, bt=None):
    return oracle.attention(case.q if q is None else q, kc, vc,
                            case.block_tables if bt is None else bt,
                            case.lens if lens is None else lens,
                            case.num_kv_heads, FP8 if fp8 else BF16, per_head,
                            window, sm_scale, ks, vs)


def manual_case(Hq, Hkv, D, L, k_vals, v_vals, q_vals):
    """A one-sequence case with given float values (rounded to bf16)."""
    bt, npg = synth.make_pages(0, [L], shuffle=False)
    slots, so, po = synth.slots_for(bt, [L])
    return synth.DecodeCase(Hq, Hkv, D, np.array([L], np.int32),
                            bits(q_vals).reshape(1, Hq, D),
                            bits(k_vals).reshape(L, Hkv, D),
                            bits(v_vals).reshape(L, Hkv, D), slots, bt, npg, so, po)


# ---------------------------------------------------------------- layout ---
def test_layout_matches_header_examples(golden_dir):
    with open(os.path.join(golden_dir, "layout_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        e = 1 if c["dtype"] == "fp8" else 2
        assert oracle.k_offset(c["row"], c["dim"], e) == c["k"], c
        assert oracle.v_offset(c["row"], c["dim"], e) == c["v"], c


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("e", [1, 2])
def test_layout_is_a_bijection_of_the_block(D, e):
    pb = 16 * D * e
    ks = {oracle.k_offset(r, d, e) for r in range(16) for d in range(D)}
    vs = {oracle.v_offset(r, d, e) for r in range(16) for d in range(D)}
    assert len(ks) == len(vs) == 16 * D
    assert min(ks) == min(vs) == 0
    assert max(ks) == max(vs) == pb - e


# ----------------------------------------------------------- cache write ---
@pytest.mark.parametrize("fp8", [True, False])
def test_cache_write_touches_only_its_row(fp8):
    H, D, P = 2, 64, 3
    r = np.random.default_rng(1)
    k = bits(r.standard_normal((2, H, D)).astype(np.float32))
    v = bits(r.standard_normal((2, H, D)).astype(np.float32))
    slots = np.array([1 * 16 + 5, -1], dtype=np.int64)          # second skipped
    kc = synth.poisoned_cache(P, H, D, fp8)
    vc = synth.poisoned_cache(P, H, D, fp8)
    ks = np.array([0.5, 0.25], np.float32)
    vs = np.array([0.125, 2.0], np.float32)
    oracle.kv_cache_write(kc, vc, k, v, slots, FP8 if fp8 else BF16, True, ks, vs)
    ref_k = synth.poisoned_cache(P, H, D, fp8)
    ref_v = synth.poisoned_cache(P, H, D, fp8)
    e = 1 if fp8 else 2
    kf = (k.astype(np.uint32) << 16).view(np.float32)
    vf = (v.astype(np.uint32) << 16).view(np.float32)
    for h in range(H):
        for d in range(D):
            ko, vo = oracle.k_offset(5, d, e), oracle.v_offset(5, d, e)
            if fp8:
                ref_k[1, h, ko] = oracle.quantize_one(float(kf[0, h, d]), float(ks[h]))
                ref_v[1, h, vo] = oracle.quantize_one(float(vf[0, h, d]), float(vs[h]))
            else:
                ref_k[1, h, ko:ko + 2] = np.frombuffer(k[0, h, d].tobytes(), np.uint8)
                ref_v[1, h, vo:vo + 2] = np.frombuffer(v[0, h, d].tobytes(), np.uint8)
    assert np.array_equal(kc, ref_k) and np.array_equal(vc, ref_v)


def test_cache_write_per_tensor_uses_one_scale():
    H, D = 2, 64
    x = np.full((1, H, D), 3.0, np.float32)
    kc = synth.poisoned_cache(1, H, D, True)
    vc = synth.poisoned_cache(1, H, D, True)
    oracle.kv_cache_write(kc, vc, bits(x), bits(x), np.array([0], np.int64), FP8,
                          False, np.array([0.5, 99.0], np.float32),
                          np.array([2.0, 99.0], np.float32))
    # 3/0.5 = 6 = 1.5 * 4 (e=9, m=4) -> 0x4C ; 3/2 = 1.5 (e=7, m=4) -> 0x3C
    assert kc[0, 1, oracle.k_offset(0, 0, 1)] == 0x4C
    assert vc[0, 1, oracle.v_offset(0, 0, 1)] == 0x3C


# ------------------------------------------------------ softmax identities --
def test_softmax_closed_form_weights():
    z = np.array([0.0, math.log(2.0), math.log(3.0)])
    p = oracle.softmax_weighted_sum(z, np.eye(3))
    assert np.allclose(p, [1 / 6, 2 / 6, 3 / 6], rtol=0, atol=1e-15)


def test_softmax_shift_invariance_and_normalisation():
    r = np.random.default_rng(2)
    z = r.standard_normal(500) * 4
    v = r.standard_normal((500, 8))
    a = oracle.softmax_weighted_sum(z, v)
    b = oracle.softmax_weighted_sum(z + 123.25, v)
    assert np.allclose(a, b, rtol=0, atol=1e-13)
    p = oracle.softmax_weighted_sum(z[:40], np.eye(40))
    assert abs(p.sum() - 1.0) < 1e-14 and np.all(p >= 0)
    assert np.allclose(oracle.softmax_weighted_sum(z, np.ones((500, 3))), 1.0,
                       atol=1e-14)


# --------------------------------------------- attention closed forms ------
def test_single_position_returns_the_dequantised_value():
    r = np.random.default_rng(4)
    D = 64
    case = manual_case(2, 1, D, 1, r.standard_normal(D), r.standard_normal(D) * 3,
                       r.standard_normal(2 * D))
    kc, vc, ks, vs = fill(case)
    o = att(case, kc, vc, ks=ks, vs=vs)
    tab = oracle.e4m3_decode_all()
    want = np.array([tab[vc[0, 0, oracle.v_offset(0, d, 1)]] * float(vs[0])
                     for d in range(D)])
    assert np.array_equal(o[0, 0], want) and np.array_equal(o[0, 1], want)


def test_two_positions_closed_form():
    # q = 4 e0, k0 = 1 e0, k1 = 2 e0 (exact codes, scale 1), D = 64:
    # z0 = 4*1/8 = 0.5, z1 = 4*2/8 = 1.0 ; v0 = e0, v1 = e1
    D = 64
    k = np.zeros((2, D)); k[0, 0], k[1, 0] = 1.0, 2.0
    v = np.zeros((2, D)); v[0, 0], v[1, 1] = 1.0, 1.0
    q = np.zeros(D); q[0] = 4.0
    case = manual_case(1, 1, D, 2, k, v, q)
    one = np.array([1.0], np.float32)
    kc, vc, _, _ = fill(case, ks=one, vs=one)
    o = att(case, kc, vc, ks=one, vs=one)[0, 0]
    p1 = math.exp(1.0) / (math.exp(0.5) + math.exp(1.0))
    assert abs(o[0] - (1 - p1)) < 1e-15 and abs(o[1] - p1) < 1e-15
    assert np.all(o[2:] == 0)
    # an explicit softmax scale replaces 1/sqrt(D)
    o = att(case, kc, vc, ks=one, vs=one, sm_scale=0.25)[0, 0]
    p1 = math.exp(2.0) / (math.exp(1.0) + math.exp(2.0))
    assert abs(o[1] - p1) < 1e-15
    # the K scale multiplies the logits: s_k = 2 doubles them
    two = np.array([2.0], np.float32)
    o = att(case, kc, vc, ks=two, vs=one)[0, 0]
    p1 = math.exp(2.0) / (math.exp(1.0) + math.exp(2.0))
    assert abs(o[1] - p1) < 1e-15
    # the V scale multiplies the output
    o = att(case, kc, vc, ks=one, vs=np.array([0.5], np.float32))[0, 0]
    p1 = math.exp(1.0) / (math.exp(0.5) + math.exp(1.0))
    assert abs(o[1] - 0.5 * p1) < 1e-15


def test_gqa_query_head_i_uses_kv_head_i_div_G():
    Hq, Hkv, D, L = 8, 2, 64, 20
    r = np.random.default_rng(6)
    k = r.standard_normal((L, Hkv, D))
    v = np.zeros((L, Hkv, D)); v[:, 0, :] = 1.0; v[:, 1, :] = 2.0
    case = manual_case(Hq, Hkv, D, L, k, v, r.standard_normal(Hq * D))
    one = np.ones(Hkv, np.float32)
    kc, vc, _, _ = fill(case, ks=one, vs=one)
    o = att(case, kc, vc, ks=one, vs=one)
    for i in range(Hq):
        assert np.all(o[0, i] == (i // 4) + 1.0), i


@pytest.mark.parametrize("L,W", [(37, 0), (37, 5), (64, 16), (100, 50), (3, 8)])
def test_zero_query_gives_window_mean(L, W):
    # q = 0 makes every logit 0, so the output is the plain mean of the
    # values over the attended positions [max(0, L-W), L)
    D = 64
    v = np.zeros((L, 1, D))
    v[:, 0, 0] = np.arange(L) % 16              # exact in e4m3 with scale 1
    v[:, 0, 1] = (np.arange(L) // 16) + 1
    case = manual_case(1, 1, D, L, np.ones((L, 1, D)), v, np.zeros(D))
    one = np.array([1.0], np.float32)
    kc, vc, _, _ = fill(case, ks=one, vs=one)
    o = att(case, kc, vc, ks=one, vs=one, window=W)[0, 0]
    lo = max(0, L - W) if W > 0 else 0
    t = np.arange(lo, L)
    assert abs(o[0] - np.mean(t % 16)) < 1e-13
    assert abs(o[1] - np.mean(t // 16 + 1)) < 1e-13


def test_empty_context_gives_zeros():
    case = synth.decode_case(0, 4, 2, 64, [40, 0])
    kc, vc, ks, vs = fill(case)
    o = att(case, kc, vc, ks=ks, vs=vs)
    assert np.all(o[1] == 0) and np.all(np.isfinite(o[0]))


# ------------------------------------------------------------ invariants ---
def test_shuffled_block_table_gives_identical_output():
    lens = [50, 33]
    a = synth.decode_case(21, 8, 2, 64, lens, shuffle=False)
    b = synth.decode_case(21, 8, 2, 64, lens, shuffle=True, spare_frac=0.5)
    assert not np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.k_new, b.k_new)
    ka, va, ks, vs = fill(a)
    kb, vb, _, _ = fill(b, ks=ks, vs=vs)
    oa = att(a, ka, va, ks=ks, vs=vs)
    ob = att(b, kb, vb, ks=ks, vs=vs)
    assert np.array_equal(oa, ob)


def test_scaling_k_up_and_q_down_keeps_the_output():
    case = synth.decode_case(22, 4, 2, 64, [70])
    kc, vc, ks, vs = fill(case)
    o1 = att(case, kc, vc, ks=ks, vs=vs)
    q2 = bits(((case.q.astype(np.uint32) << 16).view(np.float32)) / 2)
    o2 = att(case, kc, vc, ks=ks * 2, vs=vs, q=q2)
    assert np.array_equal(o1, o2)


def test_duplicate_query_heads_give_identical_rows():
    case = synth.decode_case(23, 4, 2, 64, [90])
    q = case.q.copy()
    q[0, 1] = q[0, 0]
    q[0, 3] = q[0, 2]
    kc, vc, ks, vs = fill(case)
    o = att(case, kc, vc, ks=ks, vs=vs, q=q)
    assert np.array_equal(o[0, 0], o[0, 1]) and np.array_equal(o[0, 2], o[0, 3])
    assert not np.array_equal(o[0, 0], o[0, 2])


@pytest.mark.parametrize("part", [1, 7, 16, 100, 1000])
def test_split_merge_equals_unsplit(part):
    case = synth.decode_case(24, 8, 2, 64, [300, 17, 1], values="tiny")
    kc, vc, ks, vs = fill(case)
    full = att(case, kc, vc, ks=ks, vs=vs)
    split = oracle.attention_split(case.q, kc, vc, case.block_tables, case.lens,
                                   2, FP8, part, True, 0, 0.0, ks, vs)
    assert np.max(np.abs(full - split)) <= 1e-13 * max(1.0, np.max(np.abs(full)))


def test_bf16_layer_uses_the_bf16_bits_unscaled():
    case = synth.decode_case(25, 4, 2, 128, [45])
    kc, vc, _, _ = fill(case, fp8=False)
    # a scale array must not matter for a bf16 layer
    o1 = att(case, kc, vc, fp8=False, ks=np.array([7.0, 7.0], np.float32),
             vs=np.array([3.0, 3.0], np.float32))
    o2 = att(case, kc, vc, fp8=False)
    assert np.array_equal(o1, o2)
    # L = 1 returns the bf16 value itself
    one = synth.decode_case(26, 4, 2, 128, [1])
    kc, vc, _, _ = fill(one, fp8=False)
    o = att(one, kc, vc, fp8=False)
    vf = (one.v_new.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(o[0, 0], vf[0, 0].astype(np.float64))
    assert np.array_equal(o[0, 2], vf[0, 1].astype(np.float64))


def test_nan_codes_propagate():
    case = synth.decode_case(27, 2, 1, 64, [20])
    kc, vc, ks, vs = fill(case)
    v2 = vc.copy()
    v2[0, 0, oracle.v_offset(3, 10, 1)] = 0x7F
    o = att(case, kc, v2, ks=ks, vs=vs)
    assert np.isnan(o[0, 0, 10]) and np.all(np.isfinite(np.delete(o[0, 0], 10)))
    k2 = kc.copy()
    k2[0, 0, oracle.k_offset(3, 10, 1)] = 0x7F
    o = att(case, k2, vc, ks=ks, vs=vs)
    assert np.all(np.isnan(o[0]))
    # poison outside the window / beyond the context is never read
    o = att(case, k2, v2, ks=ks, vs=vs, window=16)
    assert np.all(np.isfinite(o))


# ------------------------------------------------- accumulation control ----
def test_low_precision_single_level_accumulation_drifts():
    """Negative control: summing P*V over 128k positions in one accumulator
    that keeps ~14 significand bits (the H800 FP8 GEMM figure in "cooking-agi:
    FP8 and the KV cache", training-recipes section) misses the 1e-2 gate,
    while the same low precision inside 128-position tiles promoted into a
    wide accumulator (two-level accumulation) meets it. The size of the
    drift itself is not pinned by the pages."""
    L = 131072
    case = synth.decode_case(synth.LLAMA70B, 8, 1, 128, [L], values="drift")
    kc, vc, ks, vs = fill(case)
    ref = att(case, kc, vc, ks=ks, vs=vs)
    one = oracle.attention_lowprec(case.q, kc, vc, case.block_tables, case.lens,
                                   1, FP8, 14, 0, True, 0, 0.0, ks, vs)
    two = oracle.attention_lowprec(case.q, kc, vc, case.block_tables, case.lens,
                                   1, FP8, 14, 128, True, 0, 0.0, ks, vs)
    e1 = np.max(np.abs(one - ref))
    e2 = np.max(np.abs(two - ref))
    assert e1 > 1e-2, e1
    assert e2 < 1e-2, e2


# ------------------------------------ second formulation: numpy brute force --
def _decode_table(dtype):
    """Values of all 256 codes from torch's float8 types (a library routine,
    independent of the oracle's codec): e4m3fn for e4m3, e5m2 for e5m2."""
    import torch
    t = torch.float8_e5m2 if dtype == oracle.E5M2 else torch.float8_e4m3fn
    return torch.arange(256, dtype=torch.uint8).view(t).to(torch.float64).numpy()


def _layout_offsets(D, e):
    """Byte offsets of (row, dim) inside one (page, head) block, written out
    from the layout the library header documents (K: 16-byte chunks of 16/e
    dims per row, chunk-major; V: 1 KiB groups of 64/e dims, row quads)."""
    r = np.arange(16)[:, None]
    d = np.arange(D)[None, :]
    ce, db = 16 // e, 64 // e
    k = ((d // ce) * 16 + r) * 16 + (d % ce) * e
    v = (d // db) * 1024 + (r // 4) * 256 + (d % db) * 4 * e + (r % 4) * e
    return k, v


def _brute_force_attention(case, kc, vc, dtype, per_head, ks, vs, window):
    """Decode attention written out in vectorised numpy float64: every
    attended position's value is decode(code) * s[h] (s[0] per tensor),
    gathered through the block table and the layout; logits
    q . k / sqrt(D); softmax; weighted sum of the values."""
    B, Hq, D = case.q.shape
    Hkv = case.num_kv_heads
    G = Hq // Hkv
    e = 2 if dtype == BF16 else 1
    koff, voff = _layout_offsets(D, e)
    if dtype == BF16:
        def values(cache, off):
            lo = cache[:, :, off].astype(np.uint32)
            hi = cache[:, :, off + 1].astype(np.uint32)
            return ((hi << 24) | (lo << 16)).view(np.float32).astype(np.float64)
        kx, vx = values(kc, koff), values(vc, voff)          # [P][H][16][D]
    else:
        tab = _decode_table(dtype)
        kx, vx = tab[kc[:, :, koff]], tab[vc[:, :, voff]]
        hs = np.arange(Hkv) if per_head else np.zeros(Hkv, int)
        kx = kx * np.asarray(ks, np.float64)[hs][None, :, None, None]
        vx = vx * np.asarray(vs, np.float64)[hs][None, :, None, None]
    qf = synth.bits_to_f32(case.q).astype(np.float64)
    out = np.zeros((B, Hq, D))
    for b, L in enumerate(case.lens):
        lo = max(0, L - window) if window else 0
        t = np.arange(lo, L)
        if t.size == 0:
            continue
        pages = case.block_tables[b, t // 16]
        rows = t % 16
        for h in range(Hkv):
            kt = kx[pages, h, rows]                          # [n][D]
            vt = vx[pages, h, rows]
            z = qf[b, h * G:(h + 1) * G] @ kt.T / math.sqrt(D)   # [G][n]
            p = np.exp(z - z.max(axis=1, keepdims=True))
            out[b, h * G:(h + 1) * G] = (p @ vt) / p.sum(axis=1, keepdims=True)
    return out


def test_brute_force_tables_match_the_format():
    # the brute force's two inputs checked against the header's worked
    # example and the format's extremes
    koff, voff = _layout_offsets(128, 1)
    assert koff[5, 17] == 337 and voff[5, 17] == 325
    t = _decode_table(FP8)
    assert t[0x7E] == 448.0 and t[0x01] == 2.0 ** -9 and np.isnan(t[0x7F])


@pytest.mark.parametrize("name", ["tiny", "gqa4_ragged_window", "per_tensor", "e5m2", "bf16"])
def test_attention_matches_a_numpy_brute_force(name):
    """The oracle's attention against a second, vectorised formulation on
    the same codes, with distinct static scales per KV head (the per-head
    scales of "State of FP8 KV cache and attention quantization in vLLM",
    section "Kernel and vLLM improvements"; per tensor or per attention
    head in "cooking-agi: FP8 and the KV cache", section "how to enable it
    in the engine"). A head that read another head's K or V scale, or the
    first head's for all, moves the output by far more than 1e-12."""
    dtype, per_head, windows = FP8, True, (0,)
    if name == "tiny":                       # the tiny workload itself
        case = synth.decode_case(synth.TINY, **synth.WORKLOADS[synth.TINY])
        ks = np.array([1.0 / 448, 5.0 / 448], np.float32)
        vs = np.array([3.0 / 448, 0.5 / 448], np.float32)
        ks = ks * oracle.scale_from_amax(case.k_new, True) * 448 / 10
        vs = vs * oracle.scale_from_amax(case.v_new, True) * 448 / 10
    elif name == "gqa4_ragged_window":      # G = 4, ragged batch, shuffled pool
        case = synth.decode_case(31, 16, 4, 64, [300, 77, 513, 16, 1], shuffle=True,
                                 spare_frac=0.3, values="tiny")
        ks = oracle.scale_from_amax(case.k_new, True) * np.array([1, 2.5, 0.3, 7], np.float32)
        vs = oracle.scale_from_amax(case.v_new, True) * np.array([4, 0.2, 1, 9], np.float32)
        windows = (0, 100, 16, 1)
    elif name == "per_tensor":
        case = synth.decode_case(32, 8, 2, 128, [200, 45])
        per_head = False
        ks = np.array([0.037], np.float32)
        vs = np.array([0.011], np.float32)
    elif name == "e5m2":
        case = synth.decode_case(33, 8, 2, 64, [150, 260], shuffle=True, values="tiny")
        dtype = oracle.E5M2
        ks = oracle.scale_from_amax(case.k_new, True, fmt=dtype) * np.array([1, 40], np.float32)
        vs = oracle.scale_from_amax(case.v_new, True, fmt=dtype) * np.array([30, 1], np.float32)
    else:
        case = synth.decode_case(34, 8, 2, 128, [90, 33], shuffle=True)
        dtype, ks, vs = BF16, None, None
    assert per_head is False or ks is None or len(set(ks.tolist())) == len(ks)
    kc = synth.poisoned_cache(case.num_pages, case.num_kv_heads, case.head_dim, dtype != BF16)
    vc = kc.copy()
    oracle.kv_cache_write(kc, vc, case.k_new, case.v_new, case.slots, dtype, per_head, ks, vs)
    for w in windows:
        got = oracle.attention(case.q, kc, vc, case.block_tables, case.lens, case.num_kv_heads,
                               dtype, per_head, w, 0.0, ks, vs)
        want = _brute_force_attention(case, kc, vc, dtype, per_head, ks, vs, w)
        err = np.max(np.abs(got - want)) / max(1.0, np.max(np.abs(want)))
        assert err <= 1e-12, (name, w, err)
