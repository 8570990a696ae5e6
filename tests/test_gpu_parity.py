"""GPU parity: the HIP library (through its C ABI) against the oracle on the
same seeded inputs.

Bars: cache bytes bit-exact (whole caches, poison included); scales
bit-exact; the flat quantiser bit-exact on all 2^32 fp32 inputs; attention
within max-abs 1e-2 and mean-abs 1e-3 of the float64 oracle (the gate), plus
a tighter bound that the kernel's arithmetic should meet (P is carried as
bf16 hi + lo, ~2^-18 relative), and bit-exact where the result is exact
(one attended position).
"""

import os
import sys

import numpy as np
import pytest
import torch

import fp8_kv_cache_write_amd as kv
import oracle
import synth
from _gpu import (BF16, FP8, GATE_MAX_ABS, GATE_MEAN_ABS, GpuLayer, OracleLayer,
                  bf16_dev, check_guards, dev, errors, guarded, host, i32_dev, i64_dev,
                  unquantised_reference)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(kv.LIB_PATH):
        from fp8_kv_cache_write_amd import build
        build.build()
    yield


def tight_bound(ref):
    return 2e-4 * max(1.0, float(np.nanmax(np.abs(ref))) if ref.size else 1.0)


def check_attention(g, o, label, out_dtype=torch.float32, tight=True):
    out = g.attend(out_dtype)
    ref = o.attend()
    mx, mean = errors(out, ref)
    say(f"[{label}] max_abs={mx:.3e} mean_abs={mean:.3e}")
    got = host(out.float()).astype(np.float64)
    assert np.all(np.isfinite(got)), label
    if out_dtype == torch.float32:
        # the parity gate, on the fp32 output
        assert mx <= GATE_MAX_ABS and mean <= GATE_MEAN_ABS, (label, mx, mean)
        if tight:
            assert mx <= tight_bound(ref), (label, mx)
    else:
        # a bf16 output is the fp32 result rounded once: within one bf16 ulp
        # (2^-8 relative) of the oracle plus the fp32 kernel error
        excess = np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + tight_bound(ref))
        assert np.all(excess <= 0), (label, float(excess.max()))
    return out, ref


# --------------------------------------------------------------- codec ------
def test_quantize_all_fp32_patterns_scale_one():
    scale = torch.ones(1, dtype=torch.float32, device=dev())
    chunk = 1 << 28
    for start in range(0, 1 << 32, chunk):
        say(f"quantize chunk {start:#x}")
        x = torch.arange(start, start + chunk, dtype=torch.int64, device=dev())
        x = x.to(torch.int32).view(torch.float32)
        out = torch.empty(chunk, dtype=torch.uint8, device=dev())
        kv.e4m3_quantize(x, scale, out)
        got = host(out)
        xs = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        want = oracle.quantize(xs, 1.0)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, [(hex(start + int(i)), hex(got[i]), hex(want[i])) for i in bad[:8]]
        del x, out


@pytest.mark.parametrize("scale", [0.0071428573, 0.2678571343, 0.4017857015, 3.0,
                                   1.2742863893508911, 1e-3])
def test_quantize_random_patterns_with_scales(scale):
    r = np.random.default_rng(int(scale * 1e6) + 1)
    bits = r.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    # plus values that land exactly on e4m3 midpoints after the division
    tab = oracle.e4m3_decode_all()
    mids = np.array([0.5 * (tab[c] + tab[c + 1]) for c in range(0x7E)], np.float64)
    near = (mids * np.float32(scale)).astype(np.float32)
    xs = np.concatenate([bits.view(np.float32), near, -near])
    out = torch.empty(xs.size, dtype=torch.uint8, device=dev())
    kv.e4m3_quantize(torch.from_numpy(xs).to(dev()),
                     torch.tensor([scale], dtype=torch.float32, device=dev()), out)
    assert np.array_equal(host(out), oracle.quantize(xs, scale))


def test_division_tie_case_from_the_worked_example():
    # -45 / fp32(120/448) = -168.0 exactly -> tie -> even code 0xF2
    s = np.float32(120) / np.float32(448)
    x = torch.tensor([-45.0, 180.0, 0.01, -0.8, 3.2, 2.0], dtype=torch.float32, device=dev())
    out = torch.empty(6, dtype=torch.uint8, device=dev())
    kv.e4m3_quantize(x, torch.tensor([s], dtype=torch.float32, device=dev()), out)
    assert list(host(out)) == [0xF2, 0x7E, 0x12, 0xC4, 0x54, 0x4F]


# ---------------------------------------------------------- scale setup -----
@pytest.mark.parametrize("per_head", [True, False])
def test_scale_from_amax_bit_exact(per_head):
    case = synth.decode_case(31, 8, 4, 128, [300, 77], values="tiny")
    k = case.k_new.copy()
    k[5, 2, 7] = 0x7FC0                       # NaN in head 2
    k[:, 3, :] = 0                            # all-zero head 3
    k[9, 1, 3] = 0xFF80                       # -Inf in head 1: its scale is +Inf
    desc = kv.layer_desc(8, 4, 128, scale_mode="per_kv_head" if per_head else "per_tensor")
    out = torch.empty(4 if per_head else 1, dtype=torch.float32, device=dev())
    kv.kv_scale_from_amax(desc, bf16_dev(k), out)
    want = oracle.scale_from_amax(k, per_head)
    got = host(out)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (got, want)
    k2 = case.k_new
    kv.kv_scale_from_amax(desc, bf16_dev(k2), out)
    assert np.array_equal(host(out), oracle.scale_from_amax(k2, per_head))
    # many work-groups per scale: a long tensor
    big = synth.decode_case(32, 8, 4, 128, [20000, 3001], values="normal").k_new
    kv.kv_scale_from_amax(desc, bf16_dev(big), out)
    assert np.array_equal(host(out), oracle.scale_from_amax(big, per_head))


# ---------------------------------------------------------- cache write -----
WRITE_CASES = [
    # (label, Hq, Hkv, D, lens, fp8, per_head, shuffle, values)
    ("tiny", 4, 2, 64, [256], True, True, False, "tiny"),
    ("d128-ragged-shuffled", 32, 8, 128, [100, 33, 1], True, True, True, "normal"),
    ("d256", 8, 2, 256, [70], True, True, True, "normal"),
    ("per-tensor", 32, 8, 128, [45], True, False, False, "normal"),
    ("bf16-d64", 64, 8, 64, [40, 17], False, True, True, "normal"),
    ("bf16-d256", 8, 2, 256, [33], False, True, False, "normal"),
]


@pytest.mark.parametrize("label,Hq,Hkv,D,lens,fp8,per_head,shuffle,values", WRITE_CASES,
                         ids=[c[0] for c in WRITE_CASES])
def test_kv_cache_write_bit_exact(label, Hq, Hkv, D, lens, fp8, per_head, shuffle, values):
    say(f"write {label}")
    case = synth.decode_case(40, Hq, Hkv, D, lens, shuffle=shuffle, spare_frac=0.3,
                             values=values)
    g = GpuLayer(case, fp8=fp8, per_head=per_head)
    o = OracleLayer(case, fp8=fp8, per_head=per_head)
    torch.cuda.synchronize()
    if fp8:
        ks, vs = g.scales_host()
        assert np.array_equal(ks, o.ks) and np.array_equal(vs, o.vs)
    assert np.array_equal(host(g.k_cache), o.k_cache), label
    assert np.array_equal(host(g.v_cache), o.v_cache), label


def test_kv_cache_write_skips_negative_slots():
    case = synth.decode_case(41, 4, 2, 64, [20])
    case.slots = case.slots.copy()
    case.slots[3] = -1
    case.slots[10] = -7
    g = GpuLayer(case)
    o = OracleLayer(case)
    torch.cuda.synchronize()
    assert np.array_equal(host(g.k_cache), o.k_cache)
    assert np.array_equal(host(g.v_cache), o.v_cache)


@pytest.mark.parametrize("fp8", [True, False])
def test_kv_cache_write_mixed_slot_runs(fp8):
    # The write stores a V row quad in 16-byte pieces only when four
    # consecutive tokens go to four consecutive slots starting at a multiple
    # of 4; every other pattern takes the byte stores. A mix of both, with
    # skipped slots, runs broken inside a quad, runs starting off a quad, a
    # quad split across tokens of different pages and a ragged tail (T % 4 =
    # 3), against the oracle's whole caches (poison included).
    Hkv, D, npg = 3, 128, 12
    slots = ([0, 1, 2, 3] + [20, 21, 22, 23] +          # aligned runs
             [5, 6, 7, 8] +                            # a run starting off a quad
             [36, 37, -1, 39] +                        # a skipped slot inside a quad
             [44, 45, 47, 46] +                        # a quad in the wrong order
             [60, 61, 62, 63] + [64, 65, 66, 67] +     # the last quad of one page, the first of the next
             [12, 13, 14, 15 + 16 * 11] +              # a run leaving the page in its last token
             [100, 101, 102, 103] + [181, 182, 183])   # aligned, then a ragged tail
    T = len(slots)
    r = np.random.default_rng(11)
    k = synth.bf16_bits(r.standard_normal((T, Hkv, D)).astype(np.float32) * 3)
    v = synth.bf16_bits(r.standard_normal((T, Hkv, D)).astype(np.float32) * 3)
    desc = kv.layer_desc(Hkv, Hkv, D, "fp8_e4m3" if fp8 else "bf16")
    pc = synth.poisoned_cache(npg, Hkv, D, fp8)
    kc, vc = torch.from_numpy(pc).to(dev()), torch.from_numpy(pc).to(dev())
    sl = np.array(slots, np.int64)
    ks = vs = None
    oks = ovs = None
    if fp8:
        oks = oracle.scale_from_amax(k, True)
        ovs = oracle.scale_from_amax(v, True)
        ks = torch.from_numpy(oks).to(dev())
        vs = torch.from_numpy(ovs).to(dev())
    kv.kv_cache_write(desc, bf16_dev(k), bf16_dev(v), i64_dev(sl), kc, vc, ks, vs)
    torch.cuda.synchronize()
    okc, ovc = pc.copy(), pc.copy()
    oracle.kv_cache_write(okc, ovc, k, v, sl, oracle.FP8 if fp8 else oracle.BF16, True, oks, ovs)
    assert np.array_equal(host(kc), okc)
    assert np.array_equal(host(vc), ovc)


@pytest.mark.parametrize("scale", [1.0, 0.0071428573, 0.2678571343, 7.0])
def test_kv_cache_write_every_bf16_value(scale):
    # all 65536 bf16 patterns (NaN, Inf, subnormals included) as K and V
    Hkv, D = 2, 128
    T = 65536 // (Hkv * D)
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(T, Hkv, D)
    bt, npg = synth.make_pages(0, [T], shuffle=True)
    slots, so, po = synth.slots_for(bt, [T])
    case = synth.DecodeCase(Hkv, Hkv, D, np.array([T], np.int32), np.zeros((1, Hkv, D), np.uint16),
                            allbits, allbits[::-1].copy(), slots, bt, npg, so, po)
    sc = ([scale, scale], [scale, scale])
    g = GpuLayer(case, scales=sc)
    o = OracleLayer(case, scales=sc)
    torch.cuda.synchronize()
    assert np.array_equal(host(g.k_cache), o.k_cache)
    assert np.array_equal(host(g.v_cache), o.v_cache)


# ------------------------------------------------------------ attention -----
def test_single_position_is_exact_for_every_code():
    # V holds every e4m3 code once (two heads x 128 dims); with one attended
    # position p = 1 exactly, so out = decode(code) * s_v bit for bit.
    Hkv, D = 2, 128
    codes = np.arange(256, dtype=np.int64)
    vals = oracle.e4m3_decode_all()[codes].astype(np.float32)      # exact bf16 values
    vbits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    vbits[0x7F], vbits[0xFF] = 0x7FC0, 0xFFC0                       # NaN codes
    v = vbits.reshape(1, Hkv, D)
    r = np.random.default_rng(3)
    k = synth.bf16_bits(r.standard_normal((1, Hkv, D)).astype(np.float32))
    q = synth.bf16_bits(r.standard_normal((1, 8, D)).astype(np.float32))
    bt, npg = synth.make_pages(0, [1], shuffle=False)
    slots, so, po = synth.slots_for(bt, [1])
    case = synth.DecodeCase(8, Hkv, D, np.array([1], np.int32), q, k, v, slots, bt, npg, so, po)
    sc = ([1.0, 1.0], [1.0, 1.0])                  # codes written unchanged
    g = GpuLayer(case, scales=sc)
    o = OracleLayer(case, scales=sc)
    torch.cuda.synchronize()
    assert np.array_equal(host(g.v_cache), o.v_cache)
    for s_v in (1.0, 0.3):
        g.v_scale.fill_(s_v)
        o.vs = np.full(2, s_v, np.float32)
        out = host(g.attend())
        ref = o.attend().astype(np.float32)
        same = (out == ref) | (np.isnan(out) & np.isnan(ref))
        assert same.all(), np.argwhere(~same)[:5]


SMALL_CASES = [
    # (label, workload, Hq, Hkv, D, lens, fp8, per_head, window, shuffle, values, scales)
    ("tiny-identity", synth.TINY, 4, 2, 64, [256], True, True, 0, False, "tiny", None),
    ("tiny-shuffled", synth.TINY, 4, 2, 64, [256], True, True, 0, True, "tiny", None),
    ("8b-ragged", synth.LLAMA8B, 32, 8, 128, [1000, 4099], True, True, 0, True, "normal", None),
    ("8b-scale1", synth.LLAMA8B, 32, 8, 128, [3001], True, False, 0, False, "normal", ([1.0], [1.0])),
    ("8b-bf16", synth.LLAMA8B, 32, 8, 128, [2049, 77], False, True, 0, True, "normal", None),
    ("batched", synth.BATCHED, 32, 8, 128, list(synth.batched_lens(num_seqs=8, lo=1800, hi=2200)),
     True, True, 0, True, "normal", None),
    ("70b-drift", synth.LLAMA70B, 64, 8, 128, [8195], True, True, 0, False, "drift", None),
    ("hd256", synth.HD256, 8, 2, 256, [6001], True, True, 0, False, "normal", None),
    ("hd256-bf16", synth.HD256, 8, 2, 256, [3003], False, True, 0, False, "normal", None),
    ("gptoss-full", synth.GPTOSS, 64, 8, 64, [3001], True, True, 0, False, "normal", None),
    ("gptoss-sw-bf16", synth.GPTOSS, 64, 8, 64, [3001, 100], False, True, 128, False, "normal", None),
    ("gptoss-sw-fp8", synth.GPTOSS, 64, 8, 64, [3001, 129], True, True, 128, True, "normal", None),
    ("group3", 50, 6, 2, 128, [517], True, True, 0, False, "normal", None),
    ("group1", 51, 4, 4, 64, [300], True, True, 0, False, "normal", None),
]


@pytest.mark.parametrize("label,wl,Hq,Hkv,D,lens,fp8,per_head,window,shuffle,values,scales",
                         SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_attention_small(label, wl, Hq, Hkv, D, lens, fp8, per_head, window, shuffle, values,
                         scales):
    say(f"attention {label}")
    case = synth.decode_case(wl, Hq, Hkv, D, lens, shuffle=shuffle, spare_frac=0.1,
                             values=values)
    g = GpuLayer(case, fp8=fp8, per_head=per_head, window=window, scales=scales)
    o = OracleLayer(case, fp8=fp8, per_head=per_head, window=window, scales=scales)
    check_attention(g, o, label)
    check_attention(g, o, label + "-bf16out", out_dtype=torch.bfloat16)


@pytest.mark.parametrize("ppw", [1, 2, 3, 8])
def test_attention_forced_split_partitions(ppw, tune):
    tune("pages_per_wave", int(ppw))
    for fp8, window, lens in ((True, 0, [700, 1, 0, 33]), (True, 100, [700, 90]),
                              (False, 37, [513, 16, 17])):
        label = f"split ppw={ppw} fp8={fp8} window={window}"
        say(label)
        case = synth.decode_case(60 + ppw, 16, 4, 128, lens, shuffle=True, spare_frac=0.2)
        g = GpuLayer(case, fp8=fp8, window=window)
        o = OracleLayer(case, fp8=fp8, window=window)
        check_attention(g, o, label)


REDUCE_CASES = [
    # (longest context, other lengths): with 1 page per wave a partition is 4
    # pages, so these give 16, 17, 32, 33, 64, 65 and 130 partitions: every
    # chunk size of the reduce kernel, its edges, and two and three chunks
    (1024, [3, 0]), (1040, [700]), (2048, [1]), (2064, [1000]), (4096, [64]),
    (4112, [17]), (8320, [4111]),
]


@pytest.mark.parametrize("longest,others", REDUCE_CASES, ids=[str(c[0]) for c in REDUCE_CASES])
def test_reduce_chunks(longest, others, tune):
    # The largest logit of sequence 0 sits near its end (a key equal to the
    # first query of each group), so a later chunk raises the running max and
    # rescales what the earlier ones summed; sequence 1 has it at position 10,
    # so the later chunks add with small weights. Shorter sequences leave
    # partitions that hold only an empty partial.
    tune("pages_per_wave", 1)
    lens = [longest] + others
    case = synth.decode_case(75, 16, 4, 128, lens, shuffle=True, spare_frac=0.1)
    k = synth.bits_to_f32(case.k_new).copy()
    q = synth.bits_to_f32(case.q)
    for b, pos in ((0, longest - 30), (1, 10)):
        if b < len(lens) and pos < lens[b]:
            r = int(np.flatnonzero((case.seq_of_row == b) & (case.pos_of_row == pos))[0])
            for h in range(4):
                k[r, h] = q[b, 4 * h]
    case.k_new = synth.bf16_bits(k)
    for fp8 in (True, False):
        label = f"reduce chunks L={longest} fp8={fp8}"
        say(label)
        g = GpuLayer(case, fp8=fp8)
        o = OracleLayer(case, fp8=fp8)
        check_attention(g, o, label)
        check_attention(g, o, label + "-bf16out", out_dtype=torch.bfloat16)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("fp8", [True, False])
def test_attention_boundary_lengths(D, fp8):
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 49, 0, 65]
    for window in (0, 5, 16, 17, 40):
        label = f"lens D={D} fp8={fp8} window={window}"
        say(label)
        case = synth.decode_case(70, 8, 2, D, lens, shuffle=True, spare_frac=0.2)
        g = GpuLayer(case, fp8=fp8, window=window)
        o = OracleLayer(case, fp8=fp8, window=window)
        out, _ = check_attention(g, o, label)
        assert np.all(host(out)[11] == 0)            # empty context -> zeros


def test_explicit_softmax_scale():
    case = synth.decode_case(71, 32, 8, 128, [500])
    for sm in (0.05, 0.3):
        g = GpuLayer(case, sm_scale=sm)
        o = OracleLayer(case, sm_scale=sm)
        check_attention(g, o, f"sm_scale={sm}")


def test_shuffled_and_identity_tables_give_identical_bits():
    lens = [600, 257]
    a = synth.decode_case(72, 32, 8, 128, lens, shuffle=False)
    b = synth.decode_case(72, 32, 8, 128, lens, shuffle=True, spare_frac=0.5)
    ga, gb = GpuLayer(a), GpuLayer(b)
    oa, ob = host(ga.attend()), host(gb.attend())
    assert np.array_equal(oa, ob)


# ------------------------------------------------------- full-size cases ----
def full_case(workload, Hq, Hkv, D, lens, **kw):
    say(f"generating workload {workload} lens={list(lens)[:4]}...")
    return synth.decode_case(workload, Hq, Hkv, D, lens, **kw)


@pytest.fixture(scope="module")
def llama8b_128k():
    return full_case(synth.LLAMA8B, 32, 8, 128, [131072])


@pytest.mark.parametrize("variant", ["fp8-per-head", "fp8-scale1", "bf16"])
def test_full_llama8b_128k(llama8b_128k, variant):
    case = llama8b_128k
    fp8 = variant != "bf16"
    per_head = variant == "fp8-per-head"
    scales = ([1.0], [1.0]) if variant == "fp8-scale1" else None
    say(f"full 8B 128k {variant}: gpu")
    g = GpuLayer(case, fp8=fp8, per_head=per_head, scales=scales)
    say(f"full 8B 128k {variant}: oracle")
    o = OracleLayer(case, fp8=fp8, per_head=per_head, scales=scales)
    assert np.array_equal(host(g.k_cache), o.k_cache)
    assert np.array_equal(host(g.v_cache), o.v_cache)
    out, ref = check_attention(g, o, f"8B-128k-{variant}")
    if fp8:
        unq = unquantised_reference(case)
        d = np.abs(host(out).astype(np.float64) - unq)
        say(f"[8B-128k-{variant}] error vs unquantised bf16 attention: max={d.max():.3e} "
            f"mean={d.mean():.3e} (reported, not gated)")


@pytest.mark.parametrize("L", [8192, 32768])
@pytest.mark.parametrize("variant", ["fp8-per-head", "fp8-scale1"])
def test_full_llama8b_mid_contexts_decode_step(L, variant):
    """The 8B layer at 8192 and 32768 positions (the plan's LDS-staged runs
    of 4 and 16 pages) through kvq_decode_step with the default plan: the
    cache holds positions 0 .. L-2, the step writes position L-1 and attends
    over all L. Cache bytes bit-exact against the oracle's write of every
    position; attention to the gate and the tight bound."""
    case = full_case(synth.LLAMA8B, 32, 8, 128, [L])
    per_head = variant == "fp8-per-head"
    scales = ([1.0], [1.0]) if variant == "fp8-scale1" else None
    o = OracleLayer(case, per_head=per_head, scales=scales)
    import copy
    pre = copy.copy(case)
    pre.k_new, pre.v_new, pre.slots = case.k_new[:-1], case.v_new[:-1], case.slots[:-1]
    sc = (o.ks, o.vs) if per_head else scales
    g = GpuLayer(pre, per_head=per_head, scales=sc)
    out = run_decode_step(g, case, case.k_new[-1:], case.v_new[-1:])
    assert np.array_equal(host(g.k_cache), o.k_cache)
    assert np.array_equal(host(g.v_cache), o.v_cache)
    ref = o.attend()
    mx, mean = errors(out, ref)
    label = f"8B-{L}-{variant}-decode-step"
    say(f"[{label}] max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert mx <= GATE_MAX_ABS and mean <= GATE_MEAN_ABS, (label, mx, mean)
    assert mx <= tight_bound(ref), (label, mx)
    unq = unquantised_reference(case)
    d = np.abs(host(out).astype(np.float64) - unq)
    say(f"[{label}] error vs unquantised bf16 attention: max={d.max():.3e} "
        f"mean={d.mean():.3e} (reported, not gated)")


@pytest.mark.timeout(900)
def test_full_llama8b_1m_decode_step():
    """The 8B layer at 1048576 positions (65536 pages, 2 GiB of fp8 cache)
    through kvq_decode_step with the default plan: the longest context any
    test runs. There the plan finds no co-resident run of at most 64 pages
    and falls back to 64-page runs in 256 partitions per KV head, read into
    registers; the reduce merges 256 partitions per row. Cache bytes
    bit-exact against the oracle's write of every position; attention to
    the gate and the tight bound: the two-level FP32 sums do not drift over
    a million positions."""
    L = 1 << 20
    case = full_case(synth.LLAMA8B, 32, 8, 128, [L])
    say("1M: oracle write")
    o = OracleLayer(case)
    import copy
    pre = copy.copy(case)
    pre.k_new, pre.v_new, pre.slots = case.k_new[:-1], case.v_new[:-1], case.slots[:-1]
    say("1M: gpu write + decode step")
    g = GpuLayer(pre, scales=(o.ks, o.vs))
    out = run_decode_step(g, case, case.k_new[-1:], case.v_new[-1:])
    assert np.array_equal(host(g.k_cache), o.k_cache)
    assert np.array_equal(host(g.v_cache), o.v_cache)
    say("1M: oracle attention")
    ref = o.attend()
    mx, mean = errors(out, ref)
    say(f"[8B-1M-decode-step] max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert mx <= GATE_MAX_ABS and mean <= GATE_MEAN_ABS, (mx, mean)
    assert mx <= tight_bound(ref), mx


def test_full_batched_concurrency8_with_step_write():
    lens = synth.batched_lens()
    case = full_case(synth.BATCHED, 32, 8, 128, lens, shuffle=True, spare_frac=0.1)
    # the cache holds every position but the newest of each sequence; the
    # step then writes the 8 new tokens in one call and attends
    last = np.cumsum(case.lens.astype(np.int64)) - 1
    keep = np.ones(case.slots.size, bool)
    keep[last] = False
    import copy
    pre = copy.copy(case)
    pre.k_new, pre.v_new, pre.slots = case.k_new[keep], case.v_new[keep], case.slots[keep]
    o = OracleLayer(case)                      # scales over all positions
    desc = kv.layer_desc(32, 8, 128)
    ks = torch.empty(8, dtype=torch.float32, device=dev())
    vs = torch.empty(8, dtype=torch.float32, device=dev())
    kv.kv_scale_from_amax(desc, bf16_dev(case.k_new), ks)
    kv.kv_scale_from_amax(desc, bf16_dev(case.v_new), vs)
    assert np.array_equal(host(ks), o.ks) and np.array_equal(host(vs), o.vs)
    g = GpuLayer(pre, scales=(host(ks), host(vs)))
    kv.kv_cache_write(g.desc, bf16_dev(case.k_new[last]), bf16_dev(case.v_new[last]),
                      i64_dev(case.slots[last]), g.k_cache, g.v_cache, g.k_scale, g.v_scale)
    torch.cuda.synchronize()
    assert np.array_equal(host(g.k_cache), o.k_cache)
    assert np.array_equal(host(g.v_cache), o.v_cache)
    g.case = case
    g.block_tables = i32_dev(case.block_tables)
    g.context_lens = i32_dev(case.lens)
    check_attention(g, o, "batched-8x20k")


def test_full_llama70b_128k_drift():
    case = full_case(synth.LLAMA70B, 64, 8, 128, [131072], values="drift")
    g = GpuLayer(case)
    o = OracleLayer(case)
    out, ref = check_attention(g, o, "70B-128k-drift")
    unq = unquantised_reference(case)
    d = np.abs(host(out).astype(np.float64) - unq)
    say(f"[70B-128k] error vs unquantised bf16 attention: max={d.max():.3e} mean={d.mean():.3e}")


def test_full_hd256_64k():
    case = full_case(synth.HD256, 8, 2, 256, [65536])
    g = GpuLayer(case)
    o = OracleLayer(case)
    check_attention(g, o, "hd256-64k")


def test_full_gptoss_hybrid_32k():
    case = full_case(synth.GPTOSS, 64, 8, 64, [32768])
    g = GpuLayer(case)
    o = OracleLayer(case)
    check_attention(g, o, "gptoss-full-32k")
    gs = GpuLayer(case, fp8=False, window=128)
    os_ = OracleLayer(case, fp8=False, window=128)
    check_attention(gs, os_, "gptoss-sw128-bf16-32k")


VARIANTS = ["2x1", "2x2", "4x1", "2x1s1", "2x1s2", "4x1s1"]


def shape_fits(variant, D, fp8):
    """Whether a split-kernel shape (TPxRING[sSLOTS]) is offered for this
    head dim and cache dtype: the LDS ring of 4 waves must stay within the
    first 64 KiB of LDS (direct-to-LDS loads)."""
    tp = int(variant.split("x")[0])
    slots = int(variant.split("s")[1]) if "s" in variant else 0
    return 4 * slots * tp * 2 * 16 * D * (1 if fp8 else 2) <= 64 * 1024


@pytest.mark.parametrize("variant", VARIANTS)
def test_attention_every_tile_variant(variant, tune):
    # every compiled (pages per tile x register ring) shape of the split
    # kernel, on ragged lengths, a window and both cache dtypes
    tune("split_shape", variant)
    for D, fp8, window, lens in ((128, True, 0, [1000, 37, 1]), (64, True, 50, [700, 129]),
                                 (128, False, 0, [515, 64]), (256, True, 0, [333]),
                                 (256, False, 21, [300, 16])):
        if not shape_fits(variant, D, fp8):
            continue
        label = f"variant {variant} D={D} fp8={fp8} window={window}"
        say(label)
        case = synth.decode_case(80, 4 * (D // 64), D // 64, D, lens, shuffle=True,
                                 spare_frac=0.2)
        g = GpuLayer(case, fp8=fp8, window=window)
        o = OracleLayer(case, fp8=fp8, window=window)
        check_attention(g, o, label)
        tune("pages_per_wave", 3)
        check_attention(g, o, label + " ppw=3")
        tune("pages_per_wave", None)


# ------------------------------------------------------ fused decode step ---
def split_newest(case):
    """(case holding every position but each sequence's newest, rows of the
    newest positions in case order)."""
    import copy
    ends = np.cumsum(case.lens.astype(np.int64))
    newest = [int(e) - 1 for e, L in zip(ends, case.lens) if L > 0]
    keep = np.ones(case.slots.size, bool)
    keep[newest] = False
    pre = copy.copy(case)
    pre.k_new, pre.v_new, pre.slots = case.k_new[keep], case.v_new[keep], case.slots[keep]
    return pre


def newest_rows(case):
    """bf16 [B][Hkv][D] of every sequence's newest position (zeros when the
    sequence is empty)."""
    B, H, D = case.num_seqs, case.num_kv_heads, case.head_dim
    k = np.zeros((B, H, D), np.uint16)
    v = np.zeros((B, H, D), np.uint16)
    ends = np.cumsum(case.lens.astype(np.int64))
    for b, (e, L) in enumerate(zip(ends, case.lens)):
        if L > 0:
            k[b], v[b] = case.k_new[e - 1], case.v_new[e - 1]
    return k, v


def run_decode_step(g, case, knew, vnew, out_dtype=torch.float32):
    reg = list(g.guards)
    out = guarded((case.num_seqs, case.num_q_heads, case.head_dim), out_dtype, None, reg)
    n = kv.decode_workspace_bytes(g.desc, case.num_seqs, case.max_context_len)
    ws = guarded((n,), torch.uint8, None, reg) if n else None
    kv.decode_step(g.desc, bf16_dev(knew), bf16_dev(vnew), g.k_cache, g.v_cache, out, g.q,
                   i32_dev(case.block_tables), i32_dev(case.lens), case.max_context_len,
                   g.k_scale, g.v_scale, ws)
    check_guards(reg, "decode step")
    return out


DECODE_STEP_CASES = [
    # (label, Hq, Hkv, D, lens, fp8, window)
    ("d128-fp8", 32, 8, 128, [1000, 4099, 1, 0, 17], True, 0),
    ("d128-bf16", 32, 8, 128, [513, 16, 33], False, 0),
    ("d64-fp8-window", 16, 2, 64, [700, 129, 3], True, 100),
    ("d64-bf16-sw128", 64, 8, 64, [3001, 100], False, 128),
    ("d256-fp8", 8, 2, 256, [777, 31], True, 0),
    ("d256-bf16", 8, 2, 256, [300, 15], False, 21),
    ("g8-fp8", 64, 8, 128, [2050, 48], True, 0),
    ("g16-fp8", 64, 4, 128, [1500, 33], True, 0),
    # head_dim 64 fp8 with LDS-staged runs of 4 and 8 pages: 4-page tiles
    ("d64-fp8-g8-4page", 64, 8, 64, [8192], True, 0),
    ("d64-fp8-g8-4page-ragged", 64, 8, 64, [8192, 3000], True, 0),
    ("g12-bf16-window", 48, 4, 64, [900, 200], False, 77),
]


@pytest.mark.parametrize("label,Hq,Hkv,D,lens,fp8,window", DECODE_STEP_CASES,
                         ids=[c[0] for c in DECODE_STEP_CASES])
def test_decode_step_equals_write_then_attend(label, Hq, Hkv, D, lens, fp8, window):
    say(f"decode step {label}")
    case = synth.decode_case(90, Hq, Hkv, D, lens, shuffle=True, spare_frac=0.2)
    pre = split_newest(case)
    knew, vnew = newest_rows(case)
    # scales from the whole layer (both sides calibrate on all positions)
    o = OracleLayer(case, fp8=fp8, window=window)
    ref_gpu = GpuLayer(case, fp8=fp8, window=window)       # the two-call path
    sc = ref_gpu.scales_host() if fp8 else None
    if fp8:
        assert np.array_equal(sc[0], o.ks) and np.array_equal(sc[1], o.vs)
    g = GpuLayer(pre, fp8=fp8, window=window, scales=sc)
    g.case = case
    g.q = bf16_dev(case.q)
    out = run_decode_step(g, case, knew, vnew)
    assert np.array_equal(host(g.k_cache), o.k_cache), label
    assert np.array_equal(host(g.v_cache), o.v_cache), label
    two_call = ref_gpu.attend()
    assert np.array_equal(host(out), host(two_call)), label
    ref = o.attend()
    mx, mean = errors(out, ref)
    say(f"[{label}] max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert mx <= GATE_MAX_ABS and mean <= GATE_MEAN_ABS and mx <= tight_bound(ref)


def test_decode_step_max_batch():
    """65535 sequences (the most one call takes) of 0 to 40 positions each,
    one decode step: 131070 (sequence, KV head) work-groups in one launch,
    batch index up to the grid's limit in the write, the split kernel and
    the output rows. Cache bytes bit-exact against the oracle, the step equal
    to the two-call path bit for bit, attention to the gate and the tight
    bound; empty sequences give zero rows."""
    B = 65535
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, 65535])))
    lens = [int(x) for x in r.integers(0, 41, size=B)]
    say(f"max batch: {B} sequences, {sum(lens)} positions")
    case = synth.decode_case(93, 8, 2, 64, lens, shuffle=True, spare_frac=0.1)
    pre = split_newest(case)
    knew, vnew = newest_rows(case)
    o = OracleLayer(case)
    ref_gpu = GpuLayer(case)
    sc = ref_gpu.scales_host()
    assert np.array_equal(sc[0], o.ks) and np.array_equal(sc[1], o.vs)
    g = GpuLayer(pre, scales=sc)
    g.case = case
    g.q = bf16_dev(case.q)
    out = run_decode_step(g, case, knew, vnew)
    assert np.array_equal(host(g.k_cache), o.k_cache)
    assert np.array_equal(host(g.v_cache), o.v_cache)
    assert np.array_equal(host(out), host(ref_gpu.attend()))
    got = host(out)
    empty = np.asarray(lens) == 0
    assert np.all(got[empty] == 0.0)
    ref = o.attend()
    mx, mean = errors(out, ref)
    say(f"[max-batch] max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert mx <= GATE_MAX_ABS and mean <= GATE_MEAN_ABS and mx <= tight_bound(ref)


@pytest.mark.parametrize("variant", VARIANTS)
def test_decode_step_every_tile_variant(variant, tune):
    tune("split_shape", variant)
    for ppw in ("auto", "1", "3"):
        if ppw == "auto":
            tune("pages_per_wave", None)
        else:
            tune("pages_per_wave", int(ppw))
        for D, fp8 in ((128, True), (64, False)):
            if not shape_fits(variant, D, fp8):
                continue
            label = f"decode step variant={variant} ppw={ppw} D={D} fp8={fp8}"
            say(label)
            case = synth.decode_case(91, 4 * (D // 64), D // 64, D, [333, 32, 1], shuffle=True,
                                     spare_frac=0.2)
            pre = split_newest(case)
            knew, vnew = newest_rows(case)
            ref_gpu = GpuLayer(case, fp8=fp8)
            g = GpuLayer(pre, fp8=fp8, scales=ref_gpu.scales_host() if fp8 else None)
            g.q = bf16_dev(case.q)
            out = run_decode_step(g, case, knew, vnew)
            torch.cuda.synchronize()
            assert np.array_equal(host(g.k_cache), host(ref_gpu.k_cache)), label
            assert np.array_equal(host(g.v_cache), host(ref_gpu.v_cache)), label
            assert np.array_equal(host(out), host(ref_gpu.attend())), label


PARTITION_ORDER_CASES = [
    # (pages per wave, lengths): a ragged batch with empty and partial last
    # partitions, one sequence with 64-page runs, and the plan's own choice
    ("2", [1000, 4099, 1, 0, 17]), ("64", [9000]), ("auto", [6000, 4500, 7]),
]


@pytest.mark.parametrize("ppw,lens", PARTITION_ORDER_CASES,
                         ids=[c[0] for c in PARTITION_ORDER_CASES])
def test_partition_order_bit_identical(ppw, lens, tune):
    # The rotated and the plain partition order run the same partitions on
    # other work-groups: the outputs, caches and fused-step results agree
    # bit for bit, and both pass the oracle gate.
    if ppw == "auto":
        tune("pages_per_wave", None)
    else:
        tune("pages_per_wave", int(ppw))
    case = synth.decode_case(92, 32, 8, 128, lens, shuffle=True, spare_frac=0.2)
    pre = split_newest(case)
    knew, vnew = newest_rows(case)
    o = OracleLayer(case)
    ref = o.attend()
    got = {}
    for rot in ("0", "1"):
        tune("partition_rotate", int(rot))
        label = f"partition order rotate={rot} ppw={ppw} lens={lens}"
        say(label)
        full = GpuLayer(case)
        att = full.attend()
        g = GpuLayer(pre, scales=full.scales_host())
        g.q = bf16_dev(case.q)
        step = run_decode_step(g, case, knew, vnew)
        assert np.array_equal(host(g.k_cache), o.k_cache), label
        assert np.array_equal(host(g.v_cache), o.v_cache), label
        assert np.array_equal(host(step), host(att)), label
        mx, mean = errors(att, ref)
        say(f"[{label}] max_abs={mx:.3e} mean_abs={mean:.3e}")
        assert mx <= GATE_MAX_ABS and mean <= GATE_MEAN_ABS and mx <= tight_bound(ref), label
        got[rot] = host(att)
    assert np.array_equal(got["0"], got["1"])


WIDE_CASES = [
    # (label, wl, Hq, Hkv, D, lens, fp8, window, values): G = 9..16, where
    # the 16 MFMA columns hold queries and P*V runs once per half of P
    ("g16-d128-fp8", 190, 128, 8, 128, [3000, 1, 0, 257], True, 0, "normal"),
    ("g16-d128-bf16", 191, 64, 4, 128, [2000, 33], False, 0, "normal"),
    ("g12-d64-fp8-window", 192, 24, 2, 64, [1500, 300], True, 128, "normal"),
    ("g10-d256-fp8", 193, 20, 2, 256, [1200, 64], True, 0, "tiny"),
    ("g9-d128-fp8-drift", 194, 72, 8, 128, [4000], True, 0, "drift"),
    ("g16-d256-bf16-window", 195, 32, 2, 256, [700], False, 100, "normal"),
]


@pytest.mark.parametrize("label,wl,Hq,Hkv,D,lens,fp8,window,values", WIDE_CASES,
                         ids=[c[0] for c in WIDE_CASES])
def test_wide_groups(label, wl, Hq, Hkv, D, lens, fp8, window, values):
    say(f"wide group {label}")
    case = synth.decode_case(wl, Hq, Hkv, D, lens, shuffle=True, spare_frac=0.2, values=values)
    g = GpuLayer(case, fp8=fp8, window=window)
    o = OracleLayer(case, fp8=fp8, window=window)
    out, _ = check_attention(g, o, label, tight=values != "tiny")
    if values == "tiny":
        ref = o.attend()
        scale = max(1.0, float(np.abs(ref).max()))
        assert errors(out, ref)[0] <= 2e-4 * scale, label
    # a query head and its copy in another group position give the same row
    # only through their own columns: every head is checked above


@pytest.mark.parametrize("variant", ["2x1", "2x1s1"])
@pytest.mark.parametrize("ppw", ["1", "3", "auto"])
def test_wide_groups_shapes_and_runs(variant, ppw, tune):
    tune("split_shape", variant)
    if ppw == "auto":
        tune("pages_per_wave", None)
    else:
        tune("pages_per_wave", int(ppw))
    case = synth.decode_case(196, 64, 4, 128, [1000, 129, 2], shuffle=True, spare_frac=0.2)
    g = GpuLayer(case)
    o = OracleLayer(case)
    check_attention(g, o, f"wide shapes {variant} ppw={ppw}")
