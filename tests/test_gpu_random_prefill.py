"""Seeded random chunked-prefill configurations against the oracle (GPU
parity): head dim, group size, KV heads, batch, ragged context lengths and
chunk lengths (empty chunks, whole prompts, a few rows over a long context),
cache dtype (e4m3, e5m2, bf16), scale mode (per tensor, per KV head, per
token, per token and head), sliding window, softmax scale, arithmetic (bf16
on exact codes, or all-FP8), output dtype, page order, column groups per
wave, and the key split (no workspace, the plan's own split, or a forced
partition count) drawn per case. Every configuration is one the library
documents as supported; each row attends causally to its prefix, as the
prefill of "State of FP8 KV cache and attention quantization in vLLM"
(section "Single-request benchmark") reads its input.

The bars: in the bf16-arithmetic modes the attention gate and the P-rounding
bound (2^-8 of the largest attended |v|); in the all-FP8 mode the mean gate
on cases of at least 64 (row, q head) pairs, the max gate on rows of at
least 512 attended positions, and on every row the bound of two e4m3 flips
of a probability (a quarter of the row's largest attended |v| per KV
head)."""

import numpy as np
import pytest
import torch

import synth
from _gpu import FLIP_DILUTION_PAIRS, GpuLayer, OracleLayer, host
from test_gpu_parity import GATE_MAX_ABS, GATE_MEAN_ABS, say
from test_gpu_prefill import check, gpu_prefill, oracle_prefill

pytestmark = pytest.mark.gpu

NUM_CASES = 300
ORACLE_BUDGET = 3e8      # sum over rows of attended positions x Hq x D


def attended(lens, chunks, window):
    """Attended positions of every query row, in row order."""
    n = []
    for L, m in zip(lens, chunks):
        for j in range(m):
            pos = L - m + j
            n.append(min(pos + 1, window) if window else pos + 1)
    return np.array(n, dtype=np.int64)


def draw(i):
    """Configuration i: a dict of the layer's and the batch's parameters."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, 901, i])))
    D = int(r.choice([64, 128, 256]))
    Hkv = int(r.choice([1, 2, 4, 8] if D < 256 else [1, 2, 4]))
    G = int(r.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
    while G * Hkv > 64:
        G //= 2
    B = int(r.integers(1, 5))
    lmax = int(r.choice([64, 700, 2500]))
    lens = [int(x) for x in r.integers(1, lmax + 1, size=B)]
    chunks = []
    for L in lens:
        kind = r.random()
        if kind < 0.2:
            chunks.append(L)                                   # whole prompt
        elif kind < 0.35:
            chunks.append(int(r.integers(1, min(L, 16) + 1)))  # a few rows, long prefix
        elif kind < 0.45:
            chunks.append(0)                                   # nothing new
        else:
            chunks.append(int(r.integers(1, L + 1)))
    if sum(chunks) == 0:
        chunks[0] = lens[0]
    fmt = str(r.choice(["fp8_e4m3", "fp8_e4m3", "fp8_e5m2", "bf16"]))
    fp8 = fmt != "bf16"
    scales = str(r.choice(["per_kv_head", "per_kv_head", "per_tensor", "per_token",
                           "per_token_head"])) if fp8 else "per_kv_head"
    dyn = scales in ("per_token", "per_token_head")
    attn = "fp8" if (fp8 and not dyn and r.random() < 0.4) else "bf16"
    window = int(r.integers(1, 400)) if r.random() < 0.3 else 0
    sm_scale = float(r.uniform(0.03, 0.2)) if r.random() < 0.2 else 0.0
    split = str(r.choice(["none", "plan", "plan", "forced"]))
    parts = int(r.choice([2, 3, 7, 64])) if split == "forced" else None
    groups = int(r.choice([1, 2, 3])) if r.random() < 0.4 else None
    # bound the oracle's work: halve the chunks until it fits
    while (attended(lens, chunks, window).sum() * G * Hkv * D > ORACLE_BUDGET
           and max(chunks) > 1):
        chunks = [c // 2 if c > 1 else c for c in chunks]
    return dict(D=D, Hkv=Hkv, Hq=G * Hkv, lens=lens, chunks=chunks, fmt=fmt, scales=scales,
                dyn=dyn, attn=attn, window=window, sm_scale=sm_scale, split=split,
                parts=parts, groups=groups, out=str(r.choice(["f32", "bf16"])),
                shuffle=bool(r.random() < 0.6), values=str(r.choice(["normal", "tiny"])))


def check_fp8attn_rows(out, ref, case, chunks, window, label):
    got = host(out.float()).astype(np.float64)
    assert np.all(np.isfinite(got)), label
    d = np.abs(got - ref)
    scale = max(1.0, float(np.abs(ref).max()))
    say(f"[{label}] max_abs={d.max():.3e} mean_abs={d.mean():.3e} (output scale {scale:.2f})")
    if d.shape[0] * d.shape[1] >= FLIP_DILUTION_PAIRS:
        assert d.mean() <= GATE_MEAN_ABS * scale, label
    v = np.abs(synth.bits_to_f32(case.v_new)).astype(np.float64).max(axis=2)   # [T][Hkv]
    G = case.num_q_heads // case.num_kv_heads
    row = 0
    for b, (L, m) in enumerate(zip(case.lens, chunks)):
        # max |v| of sequence b's position p per KV head
        vb = np.zeros((int(L), case.num_kv_heads))
        sel = np.flatnonzero(case.seq_of_row == b)
        vb[case.pos_of_row[sel]] = v[sel]
        for j in range(m):
            pos = int(L) - m + j
            lo = max(0, pos + 1 - window) if window else 0
            if pos + 1 - lo >= 512:
                assert d[row].max() <= GATE_MAX_ABS * scale, (label, row)
            for h in range(case.num_kv_heads):
                # e4m3 rounding moves |v| by at most 1/16 of it
                bound = 0.25 * (17.0 / 16.0) * float(vb[lo:pos + 1, h].max())
                assert d[row, h * G:(h + 1) * G].max() <= bound, (label, row, h)
            row += 1


def _label(i, c):
    return (f"random-prefill#{i} D={c['D']} Hq={c['Hq']} Hkv={c['Hkv']} lens={c['lens']} "
            f"chunks={c['chunks']} {c['fmt']} {c['scales']} attn={c['attn']} W={c['window']} "
            f"sm={c['sm_scale']:.3f} split={c['split']}/{c['parts']} groups={c['groups']} "
            f"out={c['out']} shuffle={c['shuffle']} values={c['values']}")


@pytest.mark.parametrize("i", range(NUM_CASES))
def test_random_prefill_configuration(i, tune):
    c = draw(i)
    label = _label(i, c)
    say(label)
    tune("prefill_key_parts", c["parts"])
    tune("prefill_column_groups", c["groups"])
    case = synth.prefill_case(3000 + i, c["Hq"], c["Hkv"], c["D"], c["lens"], c["chunks"],
                              shuffle=c["shuffle"], spare_frac=0.2, values=c["values"])
    kw = dict(fmt=c["fmt"], window=c["window"], sm_scale=c["sm_scale"], attn=c["attn"],
              per_head=c["scales"] != "per_tensor",
              dyn=c["scales"] if c["dyn"] else None)
    g = GpuLayer(case, **kw)
    o = OracleLayer(case, **kw)
    assert np.array_equal(host(g.k_cache), o.k_cache), label
    assert np.array_equal(host(g.v_cache), o.v_cache), label
    split = c["split"] != "none"
    out = gpu_prefill(g, case, split=split)
    ref = oracle_prefill(o, case)
    if c["attn"] == "fp8":
        check_fp8attn_rows(out, ref, case, c["chunks"], c["window"], label)
    else:
        check(out, ref, o, case, label)
    if c["out"] == "bf16":
        # the bf16 output is the FP32 result rounded to nearest even
        b16 = gpu_prefill(g, case, torch.bfloat16, split=split)
        assert torch.equal(out.to(torch.bfloat16), b16), label
