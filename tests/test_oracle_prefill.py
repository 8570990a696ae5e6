"""Pins of the oracle's chunked-prefill attention (no GPU).

Prefill is the phase that attends every input token to its own prefix ("State
of FP8 KV cache and attention quantization in vLLM", section "Single-request
benchmark": self-attention over the input, cost quadratic in its length).
With chunked prefill a sequence's new rows are its last positions, so row j of
a chunk of n rows over L written positions sits at position L - n + j and
attends causally to [lo, pos] (lo = pos + 1 - W with a window W). The pins
below come from closed forms and from the decode oracle, not from the
prefill code itself.
"""

import numpy as np
import pytest

import oracle
import synth
from test_oracle_attention import fill

FP8 = oracle.FP8


def prefill(case, kc, vc, ks, vs, window=0, q=None, rows=None, sm_scale=0.0):
    return oracle.prefill_attention(case.q if q is None else q, kc, vc, case.block_tables,
                                    case.query_start, case.lens, case.num_kv_heads, FP8, True,
                                    window, sm_scale, ks, vs, rows)


def decoded_v(case, vc, vs):
    """float64 V values of every written position, read back through the
    layout: [T][H][D] in the order of case.k_new."""
    dec = oracle.e4m3_decode_all()
    D = case.head_dim
    off = np.array([oracle.v_offset(r, d, 1) for r in range(16) for d in range(D)]).reshape(16, D)
    codes = vc[case.slots // 16][:, :, off][np.arange(case.slots.size), :, case.slots % 16]
    return dec[codes] * vs[None, :, None].astype(np.float64)


def positions(case):
    """(sequence, position) of every query row."""
    out = []
    for b, L in enumerate(case.lens):
        n = case.query_start[b + 1] - case.query_start[b]
        out += [(b, L - n + j) for j in range(n)]
    return out


@pytest.mark.parametrize("window", [0, 7, 40])
def test_zero_query_gives_the_mean_of_the_causal_window(window):
    # every logit is 0, so row at pos averages V over [lo, pos] exactly
    case = synth.prefill_case(130, 8, 2, 64, [100, 37, 16], [30, 37, 1], shuffle=True,
                              spare_frac=0.3)
    kc, vc, ks, vs = fill(case)
    zero = np.zeros_like(case.q)
    out = prefill(case, kc, vc, ks, vs, window, q=zero)
    v = decoded_v(case, vc, vs)
    start = np.concatenate([[0], np.cumsum(case.lens)])
    for r, (b, pos) in enumerate(positions(case)):
        lo = max(0, pos + 1 - window) if window else 0
        mean = v[start[b] + lo:start[b] + pos + 1].mean(axis=0)       # [H][D]
        for i in range(8):
            assert np.allclose(out[r, i], mean[i // 4], rtol=0, atol=1e-12), (r, i, window)


def test_first_position_returns_its_value():
    case = synth.prefill_case(131, 4, 1, 64, [40], [40])
    kc, vc, ks, vs = fill(case)
    out = prefill(case, kc, vc, ks, vs)
    v = decoded_v(case, vc, vs)
    assert np.array_equal(out[0, :, :], np.repeat(v[0:1, 0], 4, axis=0))


def test_last_row_is_the_decode_attention():
    case = synth.prefill_case(132, 16, 4, 128, [300, 77, 5], [64, 77, 2], shuffle=True)
    kc, vc, ks, vs = fill(case)
    for window in (0, 50):
        out = prefill(case, kc, vc, ks, vs, window)
        last = case.query_start[1:] - 1
        q_last = case.q[last]
        dec = oracle.attention(q_last, kc, vc, case.block_tables, case.lens, 4, FP8, True,
                               window, 0.0, ks, vs)
        assert np.array_equal(out[last], dec), window


def test_future_positions_do_not_matter():
    # perturbing the cache at position pos + 1 leaves row pos alone; at pos it
    # changes it
    case = synth.prefill_case(133, 4, 1, 64, [64], [64])
    kc, vc, ks, vs = fill(case)
    out = prefill(case, kc, vc, ks, vs)
    for pos in (0, 15, 16, 40):
        for target, same in ((pos + 1, True), (pos, False)):
            kc2, vc2 = kc.copy(), vc.copy()
            slot = case.slots[target]
            p, r = slot // 16, slot % 16
            for d in range(64):
                vc2[p, 0, oracle.v_offset(r, d, 1)] ^= 0x08     # a different finite code
            out2 = prefill(case, kc2, vc2, ks, vs)
            assert np.array_equal(out2[pos], out[pos]) == same, (pos, target)


def test_row_subset_matches_the_full_computation():
    case = synth.prefill_case(134, 8, 2, 64, [200, 90], [120, 90], shuffle=True)
    kc, vc, ks, vs = fill(case)
    full = prefill(case, kc, vc, ks, vs, 33)
    rows = np.array([0, 5, 119, 120, 209], np.int32)
    assert np.array_equal(prefill(case, kc, vc, ks, vs, 33, rows=rows), full[rows])


def test_fp8attn_last_row_is_the_decode_fp8attn():
    # the all-FP8 arithmetic row by row: each sequence's last row is the
    # (pinned) all-FP8 decode attention
    case = synth.prefill_case(135, 16, 4, 128, [300, 77, 5], [64, 77, 2], shuffle=True)
    kc, vc, ks, vs = fill(case)
    for window in (0, 50):
        out = oracle.prefill_attention(case.q, kc, vc, case.block_tables, case.query_start,
                                       case.lens, 4, FP8, True, window, 0.0, ks, vs,
                                       fp8attn=True)
        last = case.query_start[1:] - 1
        dec = oracle.attention_fp8attn(case.q[last], kc, vc, case.block_tables, case.lens, 4,
                                       FP8, True, window, 0.0, ks, vs)
        assert np.array_equal(out[last], dec), window


def test_fp8attn_zero_query_gives_the_window_mean():
    # q = 0: s_q = 1, every logit 0, every block's p = e4m3(1) = 1
    case = synth.prefill_case(136, 8, 2, 64, [100, 37], [30, 37], shuffle=True)
    kc, vc, ks, vs = fill(case)
    zero = np.zeros_like(case.q)
    out = oracle.prefill_attention(zero, kc, vc, case.block_tables, case.query_start, case.lens,
                                   2, FP8, True, 7, 0.0, ks, vs, fp8attn=True)
    ref = prefill(case, kc, vc, ks, vs, 7, q=zero)
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
