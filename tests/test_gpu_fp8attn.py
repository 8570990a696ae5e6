"""GPU parity of the all-FP8 attention mode (KVQ_ATTN_FP8: e4m3 query and
probabilities, fp8 MFMA; "State of FP8 KV cache and attention quantization in
vLLM", introduction) against the oracle's variant that quantises q and P by
the same rules (per-row s_q = amax / 448; P per aligned 32-position block
relative to the block's largest logit). Logits differ between the two only by
FP32 rounding, so a probability can land on the other side of an e4m3
rounding boundary now and then: the parity bar is the attention gate."""

import os

import numpy as np
import pytest
import torch

import fp8_kv_cache_write_amd as kv
import oracle
import synth
from _gpu import GpuLayer, OracleLayer, bf16_dev, errors, host
from test_gpu_parity import (GATE_MAX_ABS, GATE_MEAN_ABS, newest_rows, run_decode_step, say,
                             split_newest)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(kv.LIB_PATH):
        from fp8_kv_cache_write_amd import build
        build.build()
    yield


def check(g, o, label):
    """The attention gate, stated for unit-scale inputs, scaled by the
    output's magnitude on the workloads with outlier channels or rows: one
    probability rounded to the neighbouring e4m3 value moves the output by
    up to 1/8 of that position's weighted value."""
    out = g.attend()
    ref = o.attend()
    mx, mean = errors(out, ref)
    scale = max(1.0, float(np.abs(ref).max()))
    say(f"[{label}] max_abs={mx:.3e} mean_abs={mean:.3e} (output scale {scale:.2f})")
    assert np.all(np.isfinite(host(out))), label
    assert mx <= GATE_MAX_ABS * scale and mean <= GATE_MEAN_ABS * scale, (label, mx, mean)
    return out, ref


CASES = [
    # (label, workload, Hq, Hkv, D, lens, fmt, window, values)
    ("tiny-e4m3", synth.TINY, 4, 2, 64, [256], "fp8_e4m3", 0, "tiny"),
    ("8b-ragged", synth.LLAMA8B, 32, 8, 128, [1000, 4099, 1], "fp8_e4m3", 0, "normal"),
    ("8b-e5m2", synth.LLAMA8B, 32, 8, 128, [2001, 33], "fp8_e5m2", 0, "normal"),
    ("70b-g8-drift", synth.LLAMA70B, 64, 8, 128, [8195], "fp8_e4m3", 0, "drift"),
    ("g16", 55, 64, 4, 128, [3001, 100], "fp8_e4m3", 0, "normal"),
    ("g16-e5m2-d64", 56, 32, 2, 64, [777], "fp8_e5m2", 0, "normal"),
    ("hd256", synth.HD256, 8, 2, 256, [6001], "fp8_e4m3", 0, "normal"),
    ("g1", 57, 4, 4, 64, [300], "fp8_e4m3", 0, "normal"),
    ("window-odd-page", synth.GPTOSS, 64, 8, 64, [3001, 129, 40], "fp8_e4m3", 128, "normal"),
    ("window-113", 58, 16, 2, 128, [1000, 500], "fp8_e4m3", 113, "normal"),
]


@pytest.mark.parametrize("label,wl,Hq,Hkv,D,lens,fmt,window,values", CASES,
                         ids=[c[0] for c in CASES])
def test_fp8attn_small(label, wl, Hq, Hkv, D, lens, fmt, window, values):
    case = synth.decode_case(wl, Hq, Hkv, D, lens, shuffle=True, spare_frac=0.25, values=values)
    g = GpuLayer(case, window=window, fmt=fmt, attn="fp8")
    o = OracleLayer(case, window=window, fmt=fmt, attn="fp8")
    assert np.array_equal(host(g.k_cache), o.k_cache)
    check(g, o, f"fp8attn-{label}")


@pytest.mark.parametrize("variant", ["2x1", "2x1s1"])
@pytest.mark.parametrize("ppw", ["3", "4", "auto"])
def test_fp8attn_shapes_and_runs(variant, ppw, tune):
    # odd runs are rounded up to even ones (tiles stay on 32-position blocks)
    tune("split_shape", variant)
    if ppw != "auto":
        tune("pages_per_wave", int(ppw))
    case = synth.decode_case(59, 32, 4, 128, [1500, 37, 1], shuffle=True, spare_frac=0.2)
    check(GpuLayer(case, attn="fp8"), OracleLayer(case, attn="fp8"), f"fp8attn {variant} ppw={ppw}")


def test_fp8attn_single_position_is_exact():
    # one position: its block's p is exactly 1 (code 0x38), so out = v
    Hkv, D = 2, 128
    r = np.random.default_rng(9)
    v = synth.bf16_bits((np.round(r.standard_normal((1, Hkv, D)) * 8) / 8).astype(np.float32))
    k = synth.bf16_bits(r.standard_normal((1, Hkv, D)).astype(np.float32))
    q = synth.bf16_bits(r.standard_normal((1, 16, D)).astype(np.float32))
    bt, npg = synth.make_pages(0, [1], shuffle=False)
    slots, so, po = synth.slots_for(bt, [1])
    case = synth.DecodeCase(16, Hkv, D, np.array([1], np.int32), q, k, v, slots, bt, npg, so, po)
    sc = ([1.0, 1.0], [0.5, 0.5])
    g = GpuLayer(case, scales=sc, attn="fp8")
    o = OracleLayer(case, scales=sc, attn="fp8")
    out = host(g.attend())
    assert np.array_equal(out, o.attend().astype(np.float32))


def test_fp8attn_full_llama8b_128k():
    case = synth.decode_case(synth.LLAMA8B, 32, 8, 128, [131072])
    say("full 8B 128k fp8 attention: gpu")
    g = GpuLayer(case, attn="fp8")
    say("full 8B 128k fp8 attention: oracle")
    o = OracleLayer(case, attn="fp8")
    out, ref = check(g, o, "8B-128k-fp8attn")
    plain = OracleLayer(case).attend()
    d = np.abs(host(out).astype(np.float64) - plain)
    say(f"[8B-128k-fp8attn] vs bf16-arithmetic attention on the same codes: "
        f"max={d.max():.3e} mean={d.mean():.3e} (the e4m3 rounding of q and P; reported)")


@pytest.mark.timeout(900)
def test_fp8attn_full_llama8b_1m():
    # the all-FP8 arithmetic over 1048576 positions (32768 P blocks per
    # row, 256 partitions per KV head): each fp8 MFMA rounds its own
    # 32-product sum, every block's product joins the FP32 sum, and the
    # output stays within the gate of the float64 oracle
    case = synth.decode_case(synth.LLAMA8B, 32, 8, 128, [1 << 20])
    say("full 8B 1M fp8 attention: gpu")
    g = GpuLayer(case, attn="fp8")
    say("full 8B 1M fp8 attention: oracle")
    o = OracleLayer(case, attn="fp8")
    check(g, o, "8B-1M-fp8attn")


def test_fp8attn_full_llama70b_128k_drift():
    case = synth.decode_case(synth.LLAMA70B, 64, 8, 128, [131072], values="drift")
    g = GpuLayer(case, attn="fp8")
    o = OracleLayer(case, attn="fp8")
    check(g, o, "70B-128k-drift-fp8attn")


@pytest.mark.parametrize("label,Hq,Hkv,D,lens,window", [
    ("d128", 32, 8, 128, [1000, 4099, 1, 0, 17], 0),
    ("d64-window", 16, 2, 64, [700, 129, 3], 100),
    ("g16", 64, 4, 128, [513, 31], 0),
])
def test_fp8attn_decode_step_equals_write_then_attend(label, Hq, Hkv, D, lens, window):
    case = synth.decode_case(92, Hq, Hkv, D, lens, shuffle=True, spare_frac=0.2)
    pre = split_newest(case)
    knew, vnew = newest_rows(case)
    o = OracleLayer(case, window=window, attn="fp8")
    ref_gpu = GpuLayer(case, window=window, attn="fp8")
    sc = ref_gpu.scales_host()
    g = GpuLayer(pre, window=window, scales=sc, attn="fp8")
    g.case = case
    g.q = bf16_dev(case.q)
    out = run_decode_step(g, case, knew, vnew)
    assert np.array_equal(host(g.k_cache), o.k_cache), label
    assert np.array_equal(host(g.v_cache), o.v_cache), label
    assert np.array_equal(host(out), host(ref_gpu.attend())), label
    ref = o.attend()
    mx, mean = errors(out, ref)
    scale = max(1.0, float(np.abs(ref).max()))
    assert mx <= GATE_MAX_ABS * scale and mean <= GATE_MEAN_ABS * scale, (label, mx, mean)


@pytest.mark.parametrize("attn", ["fp8", "bf16"])
def test_fp8attn_tiny_zero_and_nan_query_rows(attn):
    # The kernel takes q / s_q by a reciprocal and one fma correction unless
    # a column of the wave has s_q < 2^-100, a non-finite s_q or a NaN
    # element; then the wave divides. Rows scaled by 2^-110 (exact in bf16)
    # take that path: all of KV head 0's group, one head of KV head 1's
    # (mixed wave). An all-zero row has s_q = 1 and attends uniformly.
    # A NaN element makes its head's output NaN on both sides (in both
    # attention modes: its running max never rises, so the merges must carry
    # the NaN).
    import dataclasses
    Hq, Hkv, D = 32, 8, 128
    case = synth.decode_case(61, Hq, Hkv, D, [1500, 77], shuffle=True, spare_frac=0.2)
    qf = synth.bits_to_f32(case.q).copy()
    G = Hq // Hkv
    qf[:, 0:G] *= np.float32(2.0 ** -110)
    qf[:, G] *= np.float32(2.0 ** -110)
    qf[:, 2 * G] = 0.0
    qf[1, 3 * G + 1, 5] = np.nan
    q = synth.bf16_bits(qf)
    assert np.array_equal(synth.bits_to_f32(q)[:, 0:G], qf[:, 0:G])   # scaling stayed exact
    case = dataclasses.replace(case, q=q)
    out = host(GpuLayer(case, attn=attn).attend())
    ref = OracleLayer(case, attn=attn).attend()
    nan_out = np.isnan(out)
    assert np.array_equal(nan_out, np.isnan(ref)), (np.argwhere(nan_out.any(-1)).tolist(),
                                                    np.argwhere(np.isnan(ref).any(-1)).tolist())
    assert nan_out[1, 3 * G + 1].all() and nan_out.sum() == D
    out[nan_out] = 0.0
    ref = np.where(np.isnan(ref), 0.0, ref)
    mx = float(np.abs(out.astype(np.float64) - ref).max())
    mean = float(np.abs(out.astype(np.float64) - ref).mean())
    say(f"[{attn} attention, tiny/zero/nan q] max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert mx <= GATE_MAX_ABS and mean <= GATE_MEAN_ABS
