"""GPU parity of the e5m2 cache dtype (fp8_e5m2: "cooking-agi: FP8 and the KV
cache", section "how to enable it in the engine") against the oracle: the
codec on every fp32 input, the amax/57344 scales, the cache write on every
bf16 value, and decode attention and the fused decode step on e5m2 caches."""

import os

import numpy as np
import pytest
import torch

import fp8_kv_cache_write_amd as kv
import oracle
import synth
from _gpu import E5M2, GpuLayer, OracleLayer, bf16_dev, dev, errors, host
from test_gpu_parity import (GATE_MAX_ABS, GATE_MEAN_ABS, VARIANTS, check_attention,
                             newest_rows, run_decode_step, say, shape_fits, split_newest,
                             tight_bound)

pytestmark = pytest.mark.gpu
FMT = "fp8_e5m2"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(kv.LIB_PATH):
        from fp8_kv_cache_write_amd import build
        build.build()
    yield


# --------------------------------------------------------------- codec ------
def test_e5m2_quantize_all_fp32_patterns_scale_one():
    scale = torch.ones(1, dtype=torch.float32, device=dev())
    chunk = 1 << 28
    for start in range(0, 1 << 32, chunk):
        say(f"e5m2 quantize chunk {start:#x}")
        x = torch.arange(start, start + chunk, dtype=torch.int64, device=dev())
        x = x.to(torch.int32).view(torch.float32)
        out = torch.empty(chunk, dtype=torch.uint8, device=dev())
        kv.e5m2_quantize(x, scale, out)
        got = host(out)
        xs = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        want = oracle.quantize(xs, 1.0, fmt=E5M2)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, [(hex(start + int(i)), hex(got[i]), hex(want[i])) for i in bad[:8]]
        del x, out


@pytest.mark.parametrize("scale", [7.8e-5, 1.2742863893508911, 3.0, 1e-3])
def test_e5m2_quantize_random_patterns_with_scales(scale):
    r = np.random.default_rng(int(scale * 1e6) + 7)
    bits = r.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    tab = oracle.e5m2_decode_all()
    mids = np.array([0.5 * (tab[c] + tab[c + 1]) for c in range(0x7B)], np.float64)
    near = (mids * np.float32(scale)).astype(np.float32)
    xs = np.concatenate([bits.view(np.float32), near, -near])
    out = torch.empty(xs.size, dtype=torch.uint8, device=dev())
    kv.e5m2_quantize(torch.from_numpy(xs).to(dev()),
                     torch.tensor([scale], dtype=torch.float32, device=dev()), out)
    assert np.array_equal(host(out), oracle.quantize(xs, scale, fmt=E5M2))


@pytest.mark.parametrize("per_head", [True, False])
def test_e5m2_scale_from_amax_bit_exact(per_head):
    case = synth.decode_case(32, 8, 4, 128, [300, 77], values="tiny")
    k = case.k_new.copy()
    k[5, 2, 7] = 0x7FC0                       # NaN in head 2
    k[:, 3, :] = 0                            # all-zero head 3
    desc = kv.layer_desc(8, 4, 128, FMT, "per_kv_head" if per_head else "per_tensor")
    out = torch.empty(4 if per_head else 1, dtype=torch.float32, device=dev())
    kv.kv_scale_from_amax(desc, bf16_dev(k), out)
    want = oracle.scale_from_amax(k, per_head, fmt=E5M2)
    assert np.array_equal(host(out).view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------- cache write -----
@pytest.mark.parametrize("label,Hq,Hkv,D,lens,per_head,shuffle", [
    ("d64", 4, 2, 64, [256], True, False),
    ("d128-ragged-shuffled", 32, 8, 128, [100, 33, 1], True, True),
    ("d256", 8, 2, 256, [70], True, True),
    ("per-tensor", 32, 8, 128, [45], False, False),
])
def test_e5m2_kv_cache_write_bit_exact(label, Hq, Hkv, D, lens, per_head, shuffle):
    case = synth.decode_case(42, Hq, Hkv, D, lens, shuffle=shuffle, spare_frac=0.3)
    g = GpuLayer(case, per_head=per_head, fmt=FMT)
    o = OracleLayer(case, per_head=per_head, fmt=FMT)
    torch.cuda.synchronize()
    ks, vs = g.scales_host()
    assert np.array_equal(ks, o.ks) and np.array_equal(vs, o.vs)
    assert np.array_equal(host(g.k_cache), o.k_cache), label
    assert np.array_equal(host(g.v_cache), o.v_cache), label


@pytest.mark.parametrize("scale", [1.0, 7.8e-5, 0.25, 3.0])
def test_e5m2_kv_cache_write_every_bf16_value(scale):
    Hkv, D = 2, 128
    T = 65536 // (Hkv * D)
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(T, Hkv, D)
    bt, npg = synth.make_pages(0, [T], shuffle=True)
    slots, so, po = synth.slots_for(bt, [T])
    case = synth.DecodeCase(Hkv, Hkv, D, np.array([T], np.int32), np.zeros((1, Hkv, D), np.uint16),
                            allbits, allbits[::-1].copy(), slots, bt, npg, so, po)
    sc = ([scale, scale], [scale, scale])
    g = GpuLayer(case, scales=sc, fmt=FMT)
    o = OracleLayer(case, scales=sc, fmt=FMT)
    torch.cuda.synchronize()
    assert np.array_equal(host(g.k_cache), o.k_cache)
    assert np.array_equal(host(g.v_cache), o.v_cache)


# ------------------------------------------------------------ attention -----
def test_e5m2_single_position_is_exact_for_every_finite_code():
    # V holds every finite e5m2 value (248 of them, padded with zeros); with
    # one attended position p = 1 exactly, so out = decode(code) * s_v.
    Hkv, D = 2, 128
    tab = oracle.e5m2_decode_all()
    finite = np.array([tab[c] for c in range(256) if np.isfinite(tab[c])], np.float32)
    vals = np.zeros(Hkv * D, np.float32)
    vals[:finite.size] = finite
    vbits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    v = vbits.reshape(1, Hkv, D)
    r = np.random.default_rng(4)
    k = synth.bf16_bits(r.standard_normal((1, Hkv, D)).astype(np.float32))
    q = synth.bf16_bits(r.standard_normal((1, 8, D)).astype(np.float32))
    bt, npg = synth.make_pages(0, [1], shuffle=False)
    slots, so, po = synth.slots_for(bt, [1])
    case = synth.DecodeCase(8, Hkv, D, np.array([1], np.int32), q, k, v, slots, bt, npg, so, po)
    sc = ([1.0, 1.0], [1.0, 1.0])
    g = GpuLayer(case, scales=sc, fmt=FMT)
    o = OracleLayer(case, scales=sc, fmt=FMT)
    torch.cuda.synchronize()
    assert np.array_equal(host(g.v_cache), o.v_cache)
    for s_v in (1.0, 0.3):
        g.v_scale.fill_(s_v)
        o.vs = np.full(2, s_v, np.float32)
        out = host(g.attend())
        ref = o.attend().astype(np.float32)
        assert np.array_equal(out, ref), np.argwhere(out != ref)[:5]


E5M2_CASES = [
    # (label, workload, Hq, Hkv, D, lens, per_head, window, shuffle, values)
    ("tiny", synth.TINY, 4, 2, 64, [256], True, 0, True, "tiny"),
    ("8b-ragged", synth.LLAMA8B, 32, 8, 128, [1000, 4099], True, 0, True, "normal"),
    ("8b-per-tensor", synth.LLAMA8B, 32, 8, 128, [3001], False, 0, False, "normal"),
    ("70b-drift", synth.LLAMA70B, 64, 8, 128, [8195], True, 0, False, "drift"),
    ("hd256", synth.HD256, 8, 2, 256, [6001], True, 0, False, "normal"),
    ("gptoss-sw", synth.GPTOSS, 64, 8, 64, [3001, 129], True, 128, True, "normal"),
]


@pytest.mark.parametrize("label,wl,Hq,Hkv,D,lens,per_head,window,shuffle,values", E5M2_CASES,
                         ids=[c[0] for c in E5M2_CASES])
def test_e5m2_attention_small(label, wl, Hq, Hkv, D, lens, per_head, window, shuffle, values):
    case = synth.decode_case(wl, Hq, Hkv, D, lens, shuffle=shuffle, spare_frac=0.25,
                             values=values)
    g = GpuLayer(case, per_head=per_head, window=window, fmt=FMT)
    o = OracleLayer(case, per_head=per_head, window=window, fmt=FMT)
    assert np.array_equal(host(g.k_cache), o.k_cache)
    check_attention(g, o, f"e5m2-{label}")


def test_e5m2_attention_forced_split(tune):
    tune("pages_per_wave", 3)
    case = synth.decode_case(synth.LLAMA8B, 32, 8, 128, [2000, 37, 1], shuffle=True,
                             spare_frac=0.2)
    check_attention(GpuLayer(case, fmt=FMT), OracleLayer(case, fmt=FMT), "e5m2-forced-split")


def test_e5m2_full_llama8b_128k():
    case = synth.decode_case(synth.LLAMA8B, 32, 8, 128, [131072])
    say("full 8B 128k e5m2: gpu")
    g = GpuLayer(case, fmt=FMT)
    say("full 8B 128k e5m2: oracle")
    o = OracleLayer(case, fmt=FMT)
    assert np.array_equal(host(g.k_cache), o.k_cache)
    assert np.array_equal(host(g.v_cache), o.v_cache)
    check_attention(g, o, "8B-128k-e5m2")


@pytest.mark.parametrize("label,Hq,Hkv,D,lens,window", [
    ("d128", 32, 8, 128, [1000, 4099, 1, 0, 17], 0),
    ("d64-window", 16, 2, 64, [700, 129, 3], 100),
    ("d256", 8, 2, 256, [777, 31], 0),
])
def test_e5m2_decode_step_equals_write_then_attend(label, Hq, Hkv, D, lens, window):
    case = synth.decode_case(91, Hq, Hkv, D, lens, shuffle=True, spare_frac=0.2)
    pre = split_newest(case)
    knew, vnew = newest_rows(case)
    o = OracleLayer(case, window=window, fmt=FMT)
    ref_gpu = GpuLayer(case, window=window, fmt=FMT)
    sc = ref_gpu.scales_host()
    assert np.array_equal(sc[0], o.ks) and np.array_equal(sc[1], o.vs)
    g = GpuLayer(pre, window=window, scales=sc, fmt=FMT)
    g.case = case
    g.q = bf16_dev(case.q)
    out = run_decode_step(g, case, knew, vnew)
    assert np.array_equal(host(g.k_cache), o.k_cache), label
    assert np.array_equal(host(g.v_cache), o.v_cache), label
    assert np.array_equal(host(out), host(ref_gpu.attend())), label
    ref = o.attend()
    mx, mean = errors(out, ref)
    assert mx <= GATE_MAX_ABS and mean <= GATE_MEAN_ABS and mx <= tight_bound(ref)


@pytest.mark.parametrize("variant", VARIANTS)
def test_e5m2_every_tile_variant(variant, tune):
    tune("split_shape", variant)
    for D, lens in ((128, [1000, 37, 1]), (64, [700, 129])):
        if not shape_fits(variant, D, True):
            continue
        case = synth.decode_case(81, 4 * (D // 64), D // 64, D, lens, shuffle=True,
                                 spare_frac=0.2)
        check_attention(GpuLayer(case, fmt=FMT), OracleLayer(case, fmt=FMT),
                        f"e5m2 variant {variant} D={D}")
