"""GPU parity of dynamic per-token scales (KVQ_SCALE_PER_TOKEN and
KVQ_SCALE_PER_TOKEN_HEAD: every written token gets its own scale,
"FP8量化与长上下文推理" section 2.2; the token's largest value lands on the
format maximum, "cooking-agi: FP8 and the KV cache", section "dynamic vs
static scale") against the oracle: the write bit for bit (codes, poison and
the scale pools), the attention to the gate and the tight bound, the fused
decode step bit for bit against write-then-attend."""

import os

import numpy as np
import pytest
import torch

import fp8_kv_cache_write_amd as kv
import oracle
import synth
from _gpu import (GpuLayer, OracleLayer, bf16_dev, check_guards, dev, errors, guarded, host,
                  i32_dev)
from test_gpu_parity import (GATE_MAX_ABS, GATE_MEAN_ABS, newest_rows, say, split_newest)

pytestmark = pytest.mark.gpu
TIGHT = 2e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(kv.LIB_PATH):
        from fp8_kv_cache_write_amd import build
        build.build()
    yield


def same_bits(a, b):
    """Bit-identical scales; NaN matches NaN whatever its payload or sign."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    eq = (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
    return a.shape == b.shape and bool(eq.all())


def check(g, o, label, tight=True):
    out = g.attend()
    ref = o.attend()
    mx, mean = errors(out, ref)
    scale = max(1.0, float(np.abs(ref).max()))
    say(f"[{label}] max_abs={mx:.3e} mean_abs={mean:.3e} (output scale {scale:.2f})")
    assert np.all(np.isfinite(host(out))), label
    assert mx <= GATE_MAX_ABS * scale and mean <= GATE_MEAN_ABS * scale, (label, mx, mean)
    if tight:
        assert mx <= TIGHT * scale, (label, mx)
    return out, ref


WRITE_CASES = [
    # (label, Hq, Hkv, D, lens, fmt)
    ("d64-e4m3", 8, 2, 64, [300, 17], "fp8_e4m3"),
    ("d128-e4m3", 32, 8, 128, [1000, 33, 1], "fp8_e4m3"),
    ("d256-e5m2", 8, 2, 256, [500, 40], "fp8_e5m2"),
    ("d128-e5m2-h1", 4, 1, 128, [200], "fp8_e5m2"),
    # the most KV heads the dynamic modes take (per-head maxima in LDS)
    ("d128-h256", 256, 256, 128, [60, 9], "fp8_e4m3"),
]


@pytest.mark.parametrize("dyn", ["per_token", "per_token_head"])
@pytest.mark.parametrize("label,Hq,Hkv,D,lens,fmt", WRITE_CASES, ids=[c[0] for c in WRITE_CASES])
def test_dynamic_write_is_bit_exact(label, Hq, Hkv, D, lens, fmt, dyn):
    case = synth.decode_case(120, Hq, Hkv, D, lens, shuffle=True, spare_frac=0.25,
                             values="spread")
    g = GpuLayer(case, fmt=fmt, dyn=dyn)
    o = OracleLayer(case, fmt=fmt, dyn=dyn)
    torch.cuda.synchronize()
    assert np.array_equal(host(g.k_cache), o.k_cache), label
    assert np.array_equal(host(g.v_cache), o.v_cache), label
    assert same_bits(host(g.k_scale), o.ks), label      # untouched slots stay NaN on both
    assert same_bits(host(g.v_scale), o.vs), label


@pytest.mark.parametrize("dyn", ["per_token", "per_token_head"])
def test_dynamic_write_mixed_slot_runs(dyn):
    # 16-byte V stores for aligned runs of 4 slots, byte stores otherwise
    # (skipped slots, broken and misaligned runs, a run leaving its page, a
    # ragged tail), codes and scale pools against the oracle, poison included
    Hkv, D, npg = 3, 128, 12
    slots = ([0, 1, 2, 3] + [20, 21, 22, 23] + [5, 6, 7, 8] + [36, 37, -1, 39] +
             [44, 45, 47, 46] + [60, 61, 62, 63] + [64, 65, 66, 67] +
             [12, 13, 14, 15 + 16 * 11] + [100, 101, 102, 103] + [181, 182, 183])
    T = len(slots)
    r = np.random.default_rng(12)
    x = r.standard_normal((2, T, Hkv, D)).astype(np.float32)
    x *= np.exp2(r.integers(-6, 7, size=(2, T, Hkv, 1))).astype(np.float32)
    k, v = synth.bf16_bits(x[0]), synth.bf16_bits(x[1])
    desc = kv.layer_desc(Hkv, Hkv, D, "fp8_e4m3", dyn)
    pc = synth.poisoned_cache(npg, Hkv, D, True)
    kc, vc = torch.from_numpy(pc).to(dev()), torch.from_numpy(pc).to(dev())
    kpool = torch.full((npg, Hkv, 16), float("nan"), dtype=torch.float32, device=dev())
    vpool = kpool.clone()
    sl = np.array(slots, np.int64)
    kv.kv_cache_write_dynamic(desc, bf16_dev(k), bf16_dev(v), torch.from_numpy(sl).to(dev()),
                              kc, vc, kpool, vpool)
    torch.cuda.synchronize()
    okc, ovc = pc.copy(), pc.copy()
    okp = np.full((npg, Hkv, 16), np.nan, np.float32)
    ovp = okp.copy()
    mode = oracle.PER_TOKEN if dyn == "per_token" else oracle.PER_TOKEN_HEAD
    oracle.kv_cache_write_dyn(okc, ovc, k, v, sl, oracle.FP8, mode, okp, ovp)
    assert np.array_equal(host(kc), okc)
    assert np.array_equal(host(vc), ovc)
    assert same_bits(host(kpool), okp) and same_bits(host(vpool), ovp)


def test_dynamic_write_special_tokens():
    # all-zero token: scale 1; NaN element: NaN scale and NaN codes; a token
    # whose largest value is in another head (per token) or in its own head
    D, Hkv = 64, 2
    r = np.random.default_rng(3)
    k = r.standard_normal((6, Hkv, D)).astype(np.float32)
    k[1] = 0.0
    k[2, 1, 5] = np.nan
    k[3, 0, 9] = 1000.0
    k[4, 1, :] *= 1e-6
    bt, npg = synth.make_pages(0, [6], shuffle=False)
    slots, so, po = synth.slots_for(bt, [6])
    kb = synth.bf16_bits(k)
    case = synth.DecodeCase(4, Hkv, D, np.array([6], np.int32),
                            synth.bf16_bits(r.standard_normal((1, 4, D)).astype(np.float32)),
                            kb, kb.copy(), slots, bt, npg, so, po)
    for dyn in ("per_token", "per_token_head"):
        g = GpuLayer(case, dyn=dyn)
        o = OracleLayer(case, dyn=dyn)
        torch.cuda.synchronize()
        assert np.array_equal(host(g.k_cache), o.k_cache), dyn
        assert same_bits(host(g.k_scale), o.ks), dyn
        assert same_bits(host(g.v_scale), o.vs), dyn


ATT_CASES = [
    # (label, wl, Hq, Hkv, D, lens, fmt, window, values)
    ("tiny-spread", synth.TINY, 4, 2, 64, [256], "fp8_e4m3", 0, "spread"),
    ("8b-ragged", synth.LLAMA8B, 32, 8, 128, [1000, 4099, 1, 0, 17], "fp8_e4m3", 0, "spread"),
    ("8b-normal", synth.LLAMA8B, 32, 8, 128, [3000], "fp8_e4m3", 0, "normal"),
    ("8b-e5m2", synth.LLAMA8B, 32, 8, 128, [2001, 33], "fp8_e5m2", 0, "spread"),
    ("70b-g8-drift", synth.LLAMA70B, 64, 8, 128, [5000], "fp8_e4m3", 0, "drift"),
    ("hd256", synth.HD256, 8, 2, 256, [6001, 3], "fp8_e4m3", 0, "spread"),
    ("g1-d64", 121, 4, 4, 64, [300], "fp8_e4m3", 0, "spread"),
    ("window-odd", synth.GPTOSS, 64, 8, 64, [3001, 129, 40], "fp8_e4m3", 128, "spread"),
    ("window-113", 122, 16, 2, 128, [1000, 500], "fp8_e4m3", 113, "normal"),
    ("g16", 126, 64, 4, 128, [2000, 40], "fp8_e4m3", 0, "spread"),
]


@pytest.mark.parametrize("dyn", ["per_token", "per_token_head"])
@pytest.mark.parametrize("label,wl,Hq,Hkv,D,lens,fmt,window,values", ATT_CASES,
                         ids=[c[0] for c in ATT_CASES])
def test_dynamic_attention(label, wl, Hq, Hkv, D, lens, fmt, window, values, dyn):
    case = synth.decode_case(wl, Hq, Hkv, D, lens, shuffle=True, spare_frac=0.25, values=values)
    g = GpuLayer(case, window=window, fmt=fmt, dyn=dyn)
    o = OracleLayer(case, window=window, fmt=fmt, dyn=dyn)
    assert np.array_equal(host(g.k_cache), o.k_cache)
    check(g, o, f"dyn-{dyn}-{label}")


@pytest.mark.parametrize("variant", ["2x1", "2x1s1"])
@pytest.mark.parametrize("ppw", ["3", "4", "auto"])
def test_dynamic_shapes_and_runs(variant, ppw, tune):
    tune("split_shape", variant)
    if ppw != "auto":
        tune("pages_per_wave", int(ppw))
    case = synth.decode_case(123, 32, 4, 128, [1500, 37, 1], shuffle=True, spare_frac=0.2,
                             values="spread")
    check(GpuLayer(case, dyn="per_token_head"), OracleLayer(case, dyn="per_token_head"),
          f"dyn {variant} ppw={ppw}")


def test_dynamic_nan_token_makes_its_heads_nan():
    # a NaN element gives its token (per token) or its token's head (per
    # token and head) a NaN scale; every query head that attends to it is NaN
    case = synth.decode_case(124, 16, 4, 128, [700, 300], shuffle=True)
    kf = synth.bits_to_f32(case.k_new).copy()
    kf[100, 2, 7] = np.nan                  # sequence 0, KV head 2
    case.k_new = synth.bf16_bits(kf)
    for dyn, heads in (("per_token_head", [(0, 8), (0, 9), (0, 10), (0, 11)]),
                       ("per_token", [(0, i) for i in range(16)])):
        out = host(GpuLayer(case, dyn=dyn).attend())
        ref = OracleLayer(case, dyn=dyn).attend()
        nan_g = np.isnan(out).all(-1)
        assert np.array_equal(nan_g, np.isnan(ref).all(-1)), dyn
        assert sorted(map(tuple, np.argwhere(nan_g).tolist())) == heads, dyn
        fin = ~np.isnan(ref)
        assert np.abs(out[fin] - ref[fin]).max() <= TIGHT * max(1.0, np.abs(ref[fin]).max())


def run_decode_step_dynamic(g, case, knew, vnew):
    reg = list(g.guards)
    out = guarded((case.num_seqs, case.num_q_heads, case.head_dim), torch.float32, None, reg)
    n = kv.decode_workspace_bytes(g.desc, case.num_seqs, case.max_context_len)
    ws = guarded((n,), torch.uint8, None, reg) if n else None
    kv.decode_step_dynamic(g.desc, bf16_dev(knew), bf16_dev(vnew), g.k_cache, g.v_cache, out,
                           g.q, i32_dev(case.block_tables), i32_dev(case.lens),
                           case.max_context_len, g.k_scale, g.v_scale, ws)
    check_guards(reg, "dynamic decode step")
    return out


@pytest.mark.parametrize("dyn", ["per_token", "per_token_head"])
@pytest.mark.parametrize("label,Hq,Hkv,D,lens,fmt,window", [
    ("d128", 32, 8, 128, [1000, 4099, 1, 0, 17], "fp8_e4m3", 0),
    ("d64-window", 16, 2, 64, [700, 129, 3], "fp8_e4m3", 100),
    ("d256-e5m2", 8, 2, 256, [777, 31], "fp8_e5m2", 0),
    ("g8", 64, 8, 128, [2050, 48], "fp8_e4m3", 0),
    ("g16", 64, 4, 128, [1500, 20], "fp8_e4m3", 0),
    ("h256", 256, 256, 64, [300, 5, 0], "fp8_e4m3", 0),
])
def test_dynamic_decode_step_equals_write_then_attend(label, Hq, Hkv, D, lens, fmt, window, dyn):
    say(f"dynamic decode step {label} {dyn}")
    case = synth.decode_case(125, Hq, Hkv, D, lens, shuffle=True, spare_frac=0.2,
                             values="spread")
    pre = split_newest(case)
    knew, vnew = newest_rows(case)
    full = GpuLayer(case, window=window, fmt=fmt, dyn=dyn)
    g = GpuLayer(pre, window=window, fmt=fmt, dyn=dyn)
    g.case = case
    g.q = bf16_dev(case.q)
    out = run_decode_step_dynamic(g, case, knew, vnew)
    assert np.array_equal(host(g.k_cache), host(full.k_cache)), label
    assert np.array_equal(host(g.v_cache), host(full.v_cache)), label
    assert same_bits(host(g.k_scale), host(full.k_scale)), label
    assert same_bits(host(g.v_scale), host(full.v_scale)), label
    assert np.array_equal(host(out), host(full.attend())), label
    o = OracleLayer(case, window=window, fmt=fmt, dyn=dyn)
    ref = o.attend()
    mx, mean = errors(out, ref)
    scale = max(1.0, float(np.abs(ref).max()))
    assert mx <= TIGHT * scale and mean <= GATE_MEAN_ABS * scale, (label, mx, mean)


@pytest.mark.parametrize("dyn", ["per_token", "per_token_head"])
def test_dynamic_full_llama8b_128k(dyn):
    case = synth.decode_case(synth.LLAMA8B, 32, 8, 128, [131072], values="spread")
    say(f"full 8B 128k dynamic {dyn}: gpu")
    g = GpuLayer(case, dyn=dyn)
    say(f"full 8B 128k dynamic {dyn}: oracle")
    o = OracleLayer(case, dyn=dyn)
    assert np.array_equal(host(g.k_cache), o.k_cache)
    assert same_bits(host(g.k_scale), o.ks) and same_bits(host(g.v_scale), o.vs)
    check(g, o, f"8B-128k-dyn-{dyn}")


def test_dynamic_full_llama70b_128k_drift():
    case = synth.decode_case(synth.LLAMA70B, 64, 8, 128, [131072], values="drift")
    check(GpuLayer(case, dyn="per_token_head"), OracleLayer(case, dyn="per_token_head"),
          "70B-128k-drift-dyn")
