"""Seeded random layer configurations against the oracle (GPU parity): head
dim, group size, KV heads, batch and ragged lengths, cache dtype (e4m3, e5m2,
bf16), scale mode (per tensor, per KV head, per token, per token and head),
sliding window, softmax scale, arithmetic (bf16 on exact codes, or all-FP8),
output dtype and page order drawn per case; a third of the static-scale cases
also run the fused decode step, which must equal the two-call path bit for
bit. Every configuration is one the library documents as supported. The
parity bars: the attention gate and the tight bound in the bf16-arithmetic
modes; in the all-FP8 mode (where FP32 against float64 logit rounding can
move a probability across an e4m3 rounding boundary, by at most an eighth of
it), the mean gate on cases of at least 64 (row, q head) pairs, the max
gate on rows of at least 512
attended positions, where a flip is diluted, and on every row the bound of
two flips: a quarter of the row's largest attended |v|."""

import numpy as np
import pytest
import torch

import synth
from _gpu import FLIP_DILUTION_PAIRS, GpuLayer, OracleLayer, bf16_dev, host
from test_gpu_parity import GATE_MAX_ABS, GATE_MEAN_ABS
from test_gpu_parity import check_attention, newest_rows, run_decode_step, say, split_newest

pytestmark = pytest.mark.gpu

NUM_CASES = 600


def draw(i):
    """Configuration i: a dict of the layer's parameters (deterministic)."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, 777, i])))
    D = int(r.choice([64, 128, 256]))
    Hkv = int(r.choice([1, 2, 4, 8] if D < 256 else [1, 2, 4]))
    G = int(r.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
    while G * Hkv > 64:
        G //= 2
    B = int(r.integers(1, 6))
    lmax = int(r.choice([64, 600, 3000]))
    lens = [int(x) for x in r.integers(0, lmax + 1, size=B)]
    lens[int(r.integers(0, B))] = max(lens[0], 1)          # at least one non-empty row
    fmt = str(r.choice(["fp8_e4m3", "fp8_e4m3", "fp8_e5m2", "bf16"]))
    fp8 = fmt != "bf16"
    scales = str(r.choice(["per_kv_head", "per_kv_head", "per_tensor", "per_token",
                           "per_token_head"])) if fp8 else "per_kv_head"
    dyn = scales in ("per_token", "per_token_head")
    attn = "fp8" if (fp8 and not dyn and r.random() < 0.6) else "bf16"
    window = int(r.integers(1, 400)) if r.random() < 0.3 else 0
    sm_scale = float(r.uniform(0.03, 0.2)) if r.random() < 0.2 else 0.0
    return dict(D=D, Hkv=Hkv, Hq=G * Hkv, lens=lens, fmt=fmt, scales=scales, dyn=dyn,
                attn=attn, window=window, sm_scale=sm_scale,
                out=str(r.choice(["f32", "bf16"])), shuffle=bool(r.random() < 0.6),
                values=str(r.choice(["normal", "tiny"])), step=bool(r.random() < 0.35))


def check_fp8attn_rows(g, o, case, window, label):
    out = g.attend()
    ref = o.attend()
    got = host(out).astype(np.float64)
    assert np.all(np.isfinite(got)), label
    d = np.abs(got - ref)
    scale = max(1.0, float(np.abs(ref).max()))
    say(f"[{label}] max_abs={d.max():.3e} mean_abs={d.mean():.3e} (output scale {scale:.2f})")
    if d.shape[0] * d.shape[1] >= FLIP_DILUTION_PAIRS:
        assert d.mean() <= GATE_MEAN_ABS * scale, label
    v = np.abs(synth.bits_to_f32(case.v_new)).astype(np.float64)       # [T][Hkv][D]
    G = case.num_q_heads // case.num_kv_heads
    for b, L in enumerate(case.lens):
        lo = max(0, int(L) - window) if window else 0
        rows = np.flatnonzero((case.seq_of_row == b) & (case.pos_of_row >= lo))
        if rows.size == 0:
            continue
        if rows.size >= 512:
            assert d[b].max() <= GATE_MAX_ABS * scale, (label, b)
        for h in range(case.num_kv_heads):
            # e4m3 rounding moves |v| by at most 1/16 of it
            bound = 0.25 * (17.0 / 16.0) * float(v[rows, h].max())
            assert d[b, h * G:(h + 1) * G].max() <= bound, (label, b, h)


def _label(i, c):
    return (f"random#{i} D={c['D']} Hq={c['Hq']} Hkv={c['Hkv']} lens={c['lens']} {c['fmt']} "
            f"{c['scales']} attn={c['attn']} W={c['window']} sm={c['sm_scale']:.3f} "
            f"out={c['out']} shuffle={c['shuffle']} values={c['values']} step={c['step']}")


@pytest.mark.parametrize("i", range(NUM_CASES))
def test_random_configuration(i):
    c = draw(i)
    label = _label(i, c)
    say(label)
    case = synth.decode_case(1000 + i, c["Hq"], c["Hkv"], c["D"], c["lens"],
                             shuffle=c["shuffle"], spare_frac=0.2, values=c["values"])
    kw = dict(fmt=c["fmt"], window=c["window"], sm_scale=c["sm_scale"], attn=c["attn"],
              per_head=c["scales"] != "per_tensor",
              dyn=c["scales"] if c["dyn"] else None)
    g = GpuLayer(case, **kw)
    o = OracleLayer(case, **kw)
    assert np.array_equal(host(g.k_cache), o.k_cache), label
    assert np.array_equal(host(g.v_cache), o.v_cache), label
    out_dtype = torch.float32 if c["out"] == "f32" else torch.bfloat16
    if c["attn"] == "fp8":
        check_fp8attn_rows(g, o, case, c["window"], label)
    else:
        check_attention(g, o, label, out_dtype=out_dtype)
    if c["step"] and not c["dyn"]:
        # the fused step on the same layer (the newest positions written by
        # the step itself) against the two-call path: identical bits
        pre = split_newest(case)
        sc = g.scales_host()
        gs = GpuLayer(pre, scales=sc if g.fp8 else None, **kw)
        gs.case = case
        gs.q = bf16_dev(case.q)
        knew, vnew = newest_rows(case)
        step_out = run_decode_step(gs, case, knew, vnew)
        assert np.array_equal(host(gs.k_cache), o.k_cache), label
        assert np.array_equal(host(gs.v_cache), o.v_cache), label
        two_call = g.attend()
        assert np.array_equal(host(step_out), host(two_call)), label
