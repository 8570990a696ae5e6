"""GPU parity of chunked-prefill attention (kvq_paged_prefill_attention)
against the oracle: every new row of a chunk attends causally to its
(window-limited) prefix ("State of FP8 KV cache and attention quantization in
vLLM", section "Single-request benchmark": prefill is self-attention over the
input).

Tolerance: the kernel rounds each probability to bf16 for the P*V product
(relative error <= 2^-8: bf16 keeps 8 significand bits) while the normaliser
sums the FP32 values, so an output moves by at most 2^-8 of the largest
attended |v| (the weights sum to one), plus FP32 rounding; the tests assert
that bound and the attention gate (scaled by the output's magnitude on
outlier data)."""

import os

import numpy as np
import pytest
import torch

import fp8_kv_cache_write_amd as kv
import oracle
import synth
from _gpu import GpuLayer, OracleLayer, check_guards, dev, guarded, host, i32_dev
from test_gpu_parity import GATE_MAX_ABS, GATE_MEAN_ABS, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(kv.LIB_PATH):
        from fp8_kv_cache_write_amd import build
        build.build()
    yield


def gpu_prefill(g, case, out_dtype=torch.float32, split=False, context_lens=None):
    # split: pass the workspace that lets the plan split the keys; the output
    # starts as NaN, so a row the kernels never write shows
    reg = list(g.guards)
    out = guarded((case.num_query_rows, case.num_q_heads, case.head_dim), out_dtype,
                  float("nan"), reg)
    ws = None
    if split:
        n = kv.prefill_workspace_bytes(g.desc, case.num_seqs, case.max_query_len,
                                       case.block_tables.shape[1])
        ws = guarded((n,), torch.uint8, None, reg) if n else None
    lens = g.context_lens if context_lens is None else i32_dev(context_lens)
    kv.paged_prefill_attention(g.desc, out, g.q, g.k_cache, g.v_cache, g.block_tables,
                               i32_dev(case.query_start), lens, case.max_query_len,
                               g.k_scale, g.v_scale, workspace=ws)
    check_guards(reg, "prefill attention")
    return out


def oracle_prefill(o, case, rows=None, lens=None):
    return oracle.prefill_attention(case.q, o.k_cache, o.v_cache, case.block_tables,
                                    case.query_start, case.lens if lens is None else lens,
                                    case.num_kv_heads, o.fmt, o.per_head, o.window, o.sm_scale,
                                    o.ks, o.vs, rows, fp8attn=o.attn == "fp8")


def vmax(o, case):
    """Largest |decoded v| of the written positions (bounds the P rounding)."""
    x = np.abs(synth.bits_to_f32(case.v_new)).max()
    return float(x) * 1.07     # the cache rounding moves a value by <= 1/16


def check(out, ref, o, case, label):
    g = host(out.float()).astype(np.float64)
    d = np.abs(g - ref)
    mx, mean = float(d.max()), float(d.mean())
    scale = max(1.0, float(np.abs(ref).max()))
    bound = 2.0 ** -8 * vmax(o, case) + 1e-5 * scale
    say(f"[{label}] max_abs={mx:.3e} mean_abs={mean:.3e} bound={bound:.3e} "
        f"(output scale {scale:.2f})")
    assert np.all(np.isfinite(g)), label
    assert mx <= GATE_MAX_ABS * scale and mean <= GATE_MEAN_ABS * scale, (label, mx, mean)
    assert mx <= bound, (label, mx, bound)


CASES = [
    # (label, wl, Hq, Hkv, D, lens, chunks, fmt, window, values)
    ("tiny-whole", synth.TINY, 4, 2, 64, [256], [256], "fp8_e4m3", 0, "tiny"),
    ("d128-g4-ragged", 140, 32, 8, 128, [300, 77, 16, 5], [300, 40, 16, 0], "fp8_e4m3", 0,
     "normal"),
    ("d128-chunk-at-end", 141, 32, 8, 128, [2000, 1500], [256, 513], "fp8_e4m3", 0, "normal"),
    ("d128-g8", 142, 64, 8, 128, [700], [700], "fp8_e4m3", 0, "drift"),
    ("d128-g1", 143, 8, 8, 128, [400, 33], [130, 33], "fp8_e4m3", 0, "normal"),
    ("d128-g3", 144, 6, 2, 128, [500], [250], "fp8_e4m3", 0, "normal"),
    ("d64-window128", synth.GPTOSS, 64, 8, 64, [1000, 129], [500, 129], "fp8_e4m3", 128,
     "normal"),
    ("d128-window113", 145, 16, 2, 128, [900, 300], [450, 7], "fp8_e4m3", 113, "normal"),
    ("d256", synth.HD256, 8, 2, 256, [600, 90], [600, 31], "fp8_e4m3", 0, "normal"),
    ("d128-e5m2", 146, 32, 8, 128, [800], [300], "fp8_e5m2", 0, "normal"),
    ("d128-bf16", 147, 32, 8, 128, [500, 64], [250, 64], "bf16", 0, "normal"),
    ("d64-bf16-sw", 148, 16, 2, 64, [700], [700], "bf16", 128, "normal"),
    ("d256-bf16", 149, 8, 2, 256, [300], [300], "bf16", 21, "normal"),
]


@pytest.mark.parametrize("label,wl,Hq,Hkv,D,lens,chunks,fmt,window,values", CASES,
                         ids=[c[0] for c in CASES])
def test_prefill(label, wl, Hq, Hkv, D, lens, chunks, fmt, window, values):
    case = synth.prefill_case(wl, Hq, Hkv, D, lens, chunks, shuffle=True, spare_frac=0.25,
                              values=values)
    g = GpuLayer(case, window=window, fmt=fmt)
    o = OracleLayer(case, window=window, fmt=fmt)
    assert np.array_equal(host(g.k_cache), o.k_cache)
    check(gpu_prefill(g, case), oracle_prefill(o, case), o, case, f"prefill-{label}")


@pytest.mark.parametrize("groups", ["1", "2", "3"])
@pytest.mark.parametrize("fmt,D,G", [("fp8_e4m3", 128, 4), ("fp8_e4m3", 64, 8),
                                     ("fp8_e5m2", 128, 2), ("bf16", 64, 4)])
def test_prefill_column_groups(groups, fmt, D, G, tune):
    # every column-group count of the kernel, all rows compared (counts above
    # what a shape supports fall back to its largest)
    tune("prefill_column_groups", int(groups))
    case = synth.prefill_case(153, 2 * G, 2, D, [700, 333], [700, 200], shuffle=True,
                              spare_frac=0.2)
    g = GpuLayer(case, fmt=fmt)
    o = OracleLayer(case, fmt=fmt)
    check(gpu_prefill(g, case), oracle_prefill(o, case), o, case,
          f"prefill {fmt} D={D} G={G} groups={groups}")


def test_prefill_bf16_output_is_the_rounded_f32_output():
    case = synth.prefill_case(150, 32, 8, 128, [600, 200], [300, 200], shuffle=True)
    g = GpuLayer(case)
    f = gpu_prefill(g, case)
    b = gpu_prefill(g, case, torch.bfloat16)
    assert torch.equal(f.to(torch.bfloat16), b)


def test_prefill_last_row_tracks_decode():
    # the last row of each chunk is the decode attention of its sequence;
    # the two kernels differ only in P's rounding (bf16 here)
    case = synth.prefill_case(151, 32, 8, 128, [3000, 1000], [64, 1000], shuffle=True)
    g = GpuLayer(case)
    pf = host(gpu_prefill(g, case))
    last = case.query_start[1:] - 1
    q_last = torch.from_numpy(np.ascontiguousarray(case.q[last]).view(np.int16)).to(dev()) \
        .view(torch.bfloat16)
    out = torch.empty((2, 32, 128), dtype=torch.float32, device=dev())
    ws = kv.alloc_workspace(g.desc, 2, int(case.lens.max()))
    kv.paged_decode_attention(g.desc, out, q_last, g.k_cache, g.v_cache, g.block_tables,
                              g.context_lens, int(case.lens.max()), g.k_scale, g.v_scale, ws)
    torch.cuda.synchronize()
    d = np.abs(pf[last] - host(out)).max()
    assert d <= 2.0 ** -8 * vmax(None, case) + 1e-5, d


def test_prefill_llama8b_8k_whole_prompt_sampled():
    case = synth.prefill_case(synth.LLAMA8B, 32, 8, 128, [8192], [8192])
    g = GpuLayer(case)
    out = host(gpu_prefill(g, case))
    o = OracleLayer(case)
    rows = np.array([0, 1, 15, 16, 31, 32, 1000, 4095, 4096, 8000, 8191], np.int32)
    ref = oracle_prefill(o, case, rows)
    check(torch.from_numpy(out[rows]), ref, o, case, "prefill-8B-8k-sampled")


def test_prefill_llama8b_32k_whole_prompt_every_query_block():
    """The 32768-token whole-prompt prefill of the 8B layer (the prefill the
    benchmark times): one row of every 48-row query block (the plan's block
    for this shape; its offset in the block varies) checked against the
    decode kernel, which the full-size decode tests pin to the oracle, at
    context pos + 1, all in one batched decode call; and 64 of those rows,
    spread from the first block to the last, against the oracle itself."""
    L = 32768
    case = synth.prefill_case(synth.LLAMA8B, 32, 8, 128, [L], [L])
    g = GpuLayer(case)
    out = host(gpu_prefill(g, case))
    blk = 48
    rows = np.array([b * blk + (7 * b) % blk for b in range(L // blk)] + [L - 1], np.int32)
    rows = np.unique(rows)
    B = rows.size
    q_rows = torch.from_numpy(np.ascontiguousarray(case.q[rows]).view(np.int16)).to(dev()) \
        .view(torch.bfloat16)
    bt = i32_dev(np.repeat(case.block_tables, B, axis=0))
    lens = i32_dev(rows + 1)
    dec = torch.empty((B, 32, 128), dtype=torch.float32, device=dev())
    ws = kv.alloc_workspace(g.desc, B, L)
    kv.paged_decode_attention(g.desc, dec, q_rows, g.k_cache, g.v_cache, bt, lens, L,
                              g.k_scale, g.v_scale, ws)
    torch.cuda.synchronize()
    d = np.abs(out[rows] - host(dec))
    bound = 2.0 ** -8 * vmax(None, case) + 1e-5
    say(f"[prefill-8B-32k-every-block] {B} rows vs decode: max_abs={d.max():.3e} bound={bound:.3e}")
    assert np.all(np.isfinite(out[rows])) and d.max() <= bound, (float(d.max()), bound)
    o = OracleLayer(case)
    sub = rows[np.linspace(0, B - 1, 64).round().astype(int)]
    ref = oracle_prefill(o, case, sub)
    check(torch.from_numpy(out[sub]), ref, o, case, "prefill-8B-32k-whole-sampled")


def test_prefill_llama8b_32k_chunk_sampled():
    # a 2048-row chunk at the end of a 32768-position context
    case = synth.prefill_case(synth.LLAMA8B, 32, 8, 128, [32768], [2048])
    g = GpuLayer(case)
    out = host(gpu_prefill(g, case))
    o = OracleLayer(case)
    rows = np.array([0, 1, 511, 512, 1024, 2047], np.int32)
    ref = oracle_prefill(o, case, rows)
    check(torch.from_numpy(out[rows]), ref, o, case, "prefill-8B-32k-chunk-sampled")


@pytest.mark.parametrize("split", [False, True])
def test_prefill_llama8b_one_wave_chunk_sampled(split):
    # a 2500-row chunk over 65536 positions: 424 work-groups of three column
    # groups, one wave (the plan keeps three groups for a chunk over a long
    # key range rather than 632 groups of two in a partial second wave);
    # with a workspace the plan may split the keys instead; rows from the
    # first, middle and last query blocks against the oracle
    case = synth.prefill_case(synth.LLAMA8B, 32, 8, 128, [65536], [2500])
    g = GpuLayer(case)
    out = host(gpu_prefill(g, case, split=split))
    o = OracleLayer(case)
    rows = np.array([0, 1, 47, 48, 1249, 1250, 2451, 2452, 2499], np.int32)
    ref = oracle_prefill(o, case, rows)
    check(torch.from_numpy(out[rows]), ref, o, case, f"prefill-8B-2500-over-64k split={split}")


@pytest.mark.parametrize("lens", [[16384, 2048], [4096, 4096, 4096]],
                         ids=["ragged", "equal"])
def test_prefill_llama8b_batch_sampled(lens):
    # whole prompts of several sequences, 16 or 24 (sequence, KV head) units
    # and two or more waves of work-groups: a ragged batch takes the
    # round-robin block order, a batch of equal prompts the XCD-grouped one;
    # rows from the first, middle and last query blocks of every sequence
    case = synth.prefill_case(synth.LLAMA8B, 32, 8, 128, lens, lens, shuffle=True)
    g = GpuLayer(case)
    out = host(gpu_prefill(g, case))
    o = OracleLayer(case)
    rows = []
    for b, n in enumerate(lens):
        q0 = int(case.query_start[b])
        rows += [q0, q0 + 47, q0 + 48, q0 + n // 2, q0 + n - 1]
    rows = np.array(rows, np.int32)
    ref = oracle_prefill(o, case, rows)
    check(torch.from_numpy(out[rows]), ref, o, case, f"prefill-8B-batch-{lens}")


@pytest.mark.parametrize("split", [False, True])
def test_prefill_max_batch(split):
    # 65535 sequences (the most one call takes) of 1 to 24 positions, each
    # with a chunk of 0 to 4 new rows at its end: the batch index up to the
    # grid's limit and the round-robin block order over 131070 (sequence,
    # KV head) units; empty chunks write nothing. Every row against the
    # oracle.
    B = 65535
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, 65535, 2])))
    lens = [int(x) for x in r.integers(1, 25, size=B)]
    chunks = [int(min(L, x)) for L, x in zip(lens, r.integers(0, 5, size=B))]
    say(f"prefill max batch: {B} sequences, {sum(chunks)} query rows, split={split}")
    case = synth.prefill_case(94, 8, 2, 64, lens, chunks, shuffle=True, spare_frac=0.1)
    g = GpuLayer(case)
    out = gpu_prefill(g, case, split=split)
    o = OracleLayer(case)
    check(out, oracle_prefill(o, case), o, case, f"prefill-max-batch-split={split}")


@pytest.mark.parametrize("fmt,attn", [("fp8_e4m3", "bf16"), ("bf16", "bf16"),
                                      ("fp8_e4m3", "fp8")])
def test_prefill_nan_rows(fmt, attn):
    # A NaN query element makes its (row, head) NaN; a NaN key element (code
    # 0x7F in an fp8 cache, scales fixed so the NaN does not reach them)
    # makes NaN exactly the rows that attend its position, for the query
    # heads of its KV head; every other row matches the oracle.
    case = synth.prefill_case(154, 16, 4, 128, [300, 200], [300, 100], shuffle=True)
    q = synth.bits_to_f32(case.q).copy()
    q[5, 3, 7] = np.nan                                   # sequence 0, row 5, head 3
    case.q = synth.bf16_bits(q)
    k = synth.bits_to_f32(case.k_new).copy()
    r = int(np.flatnonzero((case.seq_of_row == 1) & (case.pos_of_row == 150))[0])
    k[r, 2, 11] = np.nan                                  # sequence 1, position 150, KV head 2
    case.k_new = synth.bf16_bits(k)
    scales = ([0.05] * 4, [0.05] * 4)
    g = GpuLayer(case, fmt=fmt, attn=attn, scales=scales)
    o = OracleLayer(case, fmt=fmt, attn=attn, scales=scales)
    out = host(gpu_prefill(g, case)).astype(np.float64)
    ref = oracle_prefill(o, case)
    want = {(5, 3)} | {(300 + j, h) for j in range(100) for h in range(8, 12) if 100 + j >= 150}
    nan_g = np.isnan(out).all(-1)
    assert not np.any(np.isnan(out) & ~nan_g[..., None]), "partly NaN rows"
    assert set(map(tuple, np.argwhere(nan_g).tolist())) == want
    assert np.array_equal(nan_g, np.isnan(ref).all(-1))
    fin = ~nan_g
    d = np.abs(out[fin] - ref[fin])
    bound = 2.0 ** -8 * vmax(None, case) + 1e-5 * max(1.0, float(np.abs(ref[fin]).max()))
    if attn == "fp8":
        assert float(d.mean()) <= GATE_MEAN_ABS, (fmt, attn)
    else:
        assert float(d.max()) <= bound, (fmt, attn, float(d.max()))


def test_prefill_empty_and_argument_checks():
    case = synth.prefill_case(152, 8, 2, 64, [40], [0])
    g = GpuLayer(case)
    out = torch.zeros((0, 8, 64), dtype=torch.float32, device=dev())
    kv.paged_prefill_attention(g.desc, out, g.q, g.k_cache, g.v_cache, g.block_tables,
                               i32_dev(case.query_start), g.context_lens, 0, g.k_scale,
                               g.v_scale)
    bad = kv.layer_desc(8, 2, 64, "bf16", attn="fp8")      # FP8 attention needs an fp8 cache
    with pytest.raises(kv.Kvfp8Error):
        kv.paged_prefill_attention(bad, out, g.q, g.k_cache, g.v_cache, g.block_tables,
                                   i32_dev(case.query_start), g.context_lens, 1, g.k_scale,
                                   g.v_scale)


DYN_CASES = [
    # (label, wl, Hq, Hkv, D, lens, chunks, fmt, window, values)
    ("d128-spread", 160, 32, 8, 128, [900, 77, 5], [900, 40, 0], "fp8_e4m3", 0, "spread"),
    ("d128-chunk-at-end", 161, 32, 8, 128, [2000], [513], "fp8_e4m3", 0, "spread"),
    ("d64-window", synth.GPTOSS, 64, 8, 64, [1000, 129], [500, 129], "fp8_e4m3", 128, "spread"),
    ("d256-e5m2", synth.HD256, 8, 2, 256, [600, 90], [600, 31], "fp8_e5m2", 0, "spread"),
    ("d128-g1-normal", 162, 8, 8, 128, [400], [130], "fp8_e4m3", 0, "normal"),
]


@pytest.mark.parametrize("dyn", ["per_token", "per_token_head"])
@pytest.mark.parametrize("label,wl,Hq,Hkv,D,lens,chunks,fmt,window,values", DYN_CASES,
                         ids=[c[0] for c in DYN_CASES])
def test_prefill_dynamic_scales(label, wl, Hq, Hkv, D, lens, chunks, fmt, window, values, dyn):
    # every position attended with its own (dynamic, per-token) K and V scales
    case = synth.prefill_case(wl, Hq, Hkv, D, lens, chunks, shuffle=True, spare_frac=0.25,
                              values=values)
    g = GpuLayer(case, window=window, fmt=fmt, dyn=dyn)
    o = OracleLayer(case, window=window, fmt=fmt, dyn=dyn)
    assert np.array_equal(host(g.k_cache), o.k_cache)
    check(gpu_prefill(g, case), oracle_prefill(o, case), o, case, f"prefill-dyn-{dyn}-{label}")


@pytest.mark.parametrize("groups", ["1", "2", "3"])
def test_prefill_dynamic_column_groups(groups, tune):
    tune("prefill_column_groups", int(groups))
    case = synth.prefill_case(163, 16, 4, 128, [700, 333], [700, 200], shuffle=True,
                              spare_frac=0.2, values="spread")
    g = GpuLayer(case, dyn="per_token_head")
    o = OracleLayer(case, dyn="per_token_head")
    check(gpu_prefill(g, case), oracle_prefill(o, case), o, case, f"prefill-dyn groups={groups}")


def keys_per_row(case, window):
    """Number of attended positions of every query row."""
    n = []
    for b, L in enumerate(case.lens):
        m = case.query_start[b + 1] - case.query_start[b]
        for j in range(m):
            pos = L - m + j
            n.append(min(pos + 1, window) if window else pos + 1)
    return np.array(n)


def check_fp8attn(out, ref, case, window, label, outliers=False):
    """All-FP8 arithmetic: the oracle quantises q and P by the same rules, so
    the two differ where FP32 logit rounding (the oracle works in float64)
    moves a probability across an e4m3 rounding boundary: one code step, at
    most 1/8 of that p (p <= 1, and the normaliser is >= 1), so a row moves
    by at most 1/8 of twice its largest |v| per flip. Over a long window of
    unit-scale values a flip is diluted below the gate; a row that attends
    fewer than one 32-position block, or a sharp softmax over outlier values,
    is not. So: the mean gate (scaled by the output's magnitude) everywhere,
    the max gate on rows of at least 32 positions of unit-scale workloads,
    and the flip bound (two flips: 1/4 of the largest attended |v|) on every
    row."""
    g = host(out.float()).astype(np.float64)
    d = np.abs(g - ref)
    mean = float(d.mean())
    scale = max(1.0, float(np.abs(ref).max()))
    nk = keys_per_row(case, window)
    long_rows = nk >= 32
    mx_long = float(d[long_rows].max()) if long_rows.any() else 0.0
    mx_short = float(d[~long_rows].max()) if (~long_rows).any() else 0.0
    say(f"[{label}] max_abs={mx_long:.3e} (rows >= 32 positions) {mx_short:.3e} (shorter) "
        f"mean_abs={mean:.3e} (output scale {scale:.2f})")
    assert np.all(np.isfinite(g)), label
    assert mean <= GATE_MEAN_ABS * scale, (label, mean)
    if not outliers:
        assert mx_long <= GATE_MAX_ABS * scale, (label, mx_long)
    assert max(mx_long, mx_short) <= 0.25 * vmax(None, case), (label, mx_long, mx_short)


FP8ATTN_CASES = [
    # (label, wl, Hq, Hkv, D, lens, chunks, fmt, window, values)
    ("tiny", synth.TINY, 4, 2, 64, [256], [256], "fp8_e4m3", 0, "tiny"),
    ("d128-ragged", 170, 32, 8, 128, [900, 77, 5], [900, 40, 0], "fp8_e4m3", 0, "normal"),
    ("d128-chunk-at-end", 171, 32, 8, 128, [2000], [513], "fp8_e4m3", 0, "normal"),
    ("g16", 172, 64, 4, 128, [600], [600], "fp8_e4m3", 0, "normal"),
    ("d64-window", synth.GPTOSS, 64, 8, 64, [1000, 129], [500, 129], "fp8_e4m3", 128, "normal"),
    ("d256-e5m2", synth.HD256, 8, 2, 256, [600, 90], [600, 31], "fp8_e5m2", 0, "normal"),
    ("g8-drift", 173, 64, 8, 128, [700], [700], "fp8_e4m3", 0, "drift"),
]


@pytest.mark.parametrize("label,wl,Hq,Hkv,D,lens,chunks,fmt,window,values", FP8ATTN_CASES,
                         ids=[c[0] for c in FP8ATTN_CASES])
def test_prefill_fp8_attention(label, wl, Hq, Hkv, D, lens, chunks, fmt, window, values):
    case = synth.prefill_case(wl, Hq, Hkv, D, lens, chunks, shuffle=True, spare_frac=0.25,
                              values=values)
    g = GpuLayer(case, window=window, fmt=fmt, attn="fp8")
    o = OracleLayer(case, window=window, fmt=fmt, attn="fp8")
    check_fp8attn(gpu_prefill(g, case), oracle_prefill(o, case), case, window,
                  f"prefill-fp8attn-{label}", outliers=values == "tiny")


@pytest.mark.parametrize("groups", ["1", "2", "3"])
def test_prefill_fp8_attention_column_groups(groups, tune):
    tune("prefill_column_groups", int(groups))
    case = synth.prefill_case(174, 16, 4, 128, [700, 333], [700, 200], shuffle=True,
                              spare_frac=0.2)
    g = GpuLayer(case, attn="fp8")
    o = OracleLayer(case, attn="fp8")
    check_fp8attn(gpu_prefill(g, case), oracle_prefill(o, case), case, 0,
                  f"prefill-fp8attn groups={groups}")


def test_prefill_fp8_attention_last_row_is_the_decode_kernels():
    # same codes, same blocks, same logit arithmetic: the last row of each
    # chunk and the all-FP8 decode kernel differ only in FP32 summation order
    case = synth.prefill_case(175, 32, 8, 128, [3000, 1000], [64, 1000], shuffle=True)
    g = GpuLayer(case, attn="fp8")
    pf = host(gpu_prefill(g, case))
    last = case.query_start[1:] - 1
    q_last = torch.from_numpy(np.ascontiguousarray(case.q[last]).view(np.int16)).to(dev()) \
        .view(torch.bfloat16)
    out = torch.empty((2, 32, 128), dtype=torch.float32, device=dev())
    ws = kv.alloc_workspace(g.desc, 2, int(case.lens.max()))
    kv.paged_decode_attention(g.desc, out, q_last, g.k_cache, g.v_cache, g.block_tables,
                              g.context_lens, int(case.lens.max()), g.k_scale, g.v_scale, ws)
    torch.cuda.synchronize()
    d = np.abs(pf[last] - host(out)).max()
    say(f"[prefill vs decode, all-FP8] max_abs={d:.3e}")
    assert d <= 1e-5 * max(1.0, float(np.abs(host(out)).max())), d


SPLIT_CASES = [
    # (label, wl, Hq, Hkv, D, lens, chunks, fmt, window, values, attn, dyn)
    ("d128-chunk64", 180, 32, 8, 128, [6000], [64], "fp8_e4m3", 0, "normal", "bf16", None),
    ("d128-ragged", 181, 32, 8, 128, [5000, 3000, 100], [200, 1, 100], "fp8_e4m3", 0, "normal",
     "bf16", None),
    ("d128-window", 182, 32, 8, 128, [4000, 2100], [300, 33], "fp8_e4m3", 128, "normal", "bf16",
     None),
    ("d64-g8", synth.GPTOSS, 64, 8, 64, [3000], [96], "fp8_e4m3", 0, "normal", "bf16", None),
    ("d256", synth.HD256, 8, 2, 256, [4000], [40], "fp8_e4m3", 0, "normal", "bf16", None),
    ("bf16-cache", 183, 32, 8, 128, [3000], [100], "bf16", 0, "normal", "bf16", None),
    ("e5m2", 184, 32, 8, 128, [3000], [100], "fp8_e5m2", 0, "normal", "bf16", None),
    ("dyn", 185, 32, 8, 128, [4000, 1000], [64, 20], "fp8_e4m3", 0, "spread", "bf16",
     "per_token_head"),
    ("att8", 186, 32, 8, 128, [4000], [70], "fp8_e4m3", 0, "normal", "fp8", None),
    ("att8-g16", 187, 64, 4, 128, [2500], [50], "fp8_e4m3", 0, "normal", "fp8", None),
]


@pytest.mark.parametrize("label,wl,Hq,Hkv,D,lens,chunks,fmt,window,values,attn,dyn", SPLIT_CASES,
                         ids=[c[0] for c in SPLIT_CASES])
def test_prefill_key_split(label, wl, Hq, Hkv, D, lens, chunks, fmt, window, values, attn, dyn,
                           tune):
    # a short chunk over a long context: the plan splits the keys (the
    # workspace size says so), the merge gives the oracle's rows, and the
    # unsplit kernel agrees to the same bound
    tune("prefill_key_parts", None)
    case = synth.prefill_case(wl, Hq, Hkv, D, lens, chunks, shuffle=True, spare_frac=0.2,
                              values=values)
    g = GpuLayer(case, window=window, fmt=fmt, attn=attn, dyn=dyn)
    o = OracleLayer(case, window=window, fmt=fmt, attn=attn, dyn=dyn)
    assert kv.prefill_workspace_bytes(g.desc, case.num_seqs, case.max_query_len,
                                      case.block_tables.shape[1]) > 0
    ref = oracle_prefill(o, case)
    for split in (True, False):
        out = gpu_prefill(g, case, split=split)
        tag = f"prefill split={split} {label}"
        if attn == "fp8":
            check_fp8attn(out, ref, case, window, tag)
        else:
            check(out, ref, o, case, tag)
    b16 = gpu_prefill(g, case, torch.bfloat16, split=True)
    assert torch.equal(gpu_prefill(g, case, split=True).to(torch.bfloat16), b16)


@pytest.mark.parametrize("parts", ["2", "7", "200"])
def test_prefill_forced_key_partitions(parts, tune):
    # any partition count, whole prompts included (partitions past a row's
    # position stay empty); 200 asks for more partitions than tiles, so every
    # partition is one tile and the merge takes two chunks
    tune("prefill_key_parts", int(parts))
    case = synth.prefill_case(188, 16, 4, 128, [3000, 700, 40], [40, 700, 40], shuffle=True,
                              spare_frac=0.2)
    for window in (0, 100):
        g = GpuLayer(case, window=window)
        o = OracleLayer(case, window=window)
        check(gpu_prefill(g, case, split=True), oracle_prefill(o, case), o, case,
              f"prefill parts={parts} window={window}")


@pytest.mark.parametrize("split", [False, True])
def test_prefill_rows_before_position_zero_are_zero(split, tune):
    # a chunk longer than the context: its first rows sit at negative
    # positions and give zeros; the others attend [0, pos]
    if split:
        tune("prefill_key_parts", 2)
    case = synth.prefill_case(189, 16, 4, 128, [64, 100], [64, 30], shuffle=True)
    g = GpuLayer(case)
    o = OracleLayer(case)
    lens = np.array([40, 100], np.int32)
    out = host(gpu_prefill(g, case, split=split, context_lens=lens)).astype(np.float64)
    ref = oracle_prefill(o, case, lens=lens)
    assert np.all(out[:24] == 0.0) and np.all(ref[:24] == 0.0)
    assert np.all(np.isfinite(out))
    d = float(np.abs(out - ref).max())
    assert d <= 2.0 ** -8 * vmax(None, case) + 1e-5, d
