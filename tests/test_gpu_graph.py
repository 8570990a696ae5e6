"""The hot path under HIP graph capture: the decode step (write + split +
reduce), the two-call decode, the dynamic-scale decode step, the split
chunked prefill (prefill + merge) and the static scale calibration with a
prefill-sized cache write are captured once and replayed several times, with
eager work of the program between the replays; every replay must give the
eager result bit for bit. None of these launches records a memset
(workspaces are written before they are read; the calibration clears its
accumulator words with a kernel)."""

import os

import numpy as np
import pytest
import torch

import fp8_kv_cache_write_amd as kv
import synth
from _gpu import GpuLayer, bf16_dev, dev, host, i32_dev
from test_gpu_parity import newest_rows, say, split_newest

pytestmark = pytest.mark.gpu
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(kv.LIB_PATH):
        from fp8_kv_cache_write_amd import build
        build.build()
    yield


def bits(t):
    """Host copy for exact comparison (bf16 as its 16-bit patterns)."""
    return host(t.view(torch.int16)) if t.dtype == torch.bfloat16 else host(t)


def replay_and_compare(fn, outs, label, state=()):
    """fn() launches on the current stream and writes the tensors in outs
    (and in state, which it also reads: the caches of a decode step).
    Runs it eagerly, captures it, then replays it REPLAYS times with other
    eager work in between (an eager call of fn and unrelated torch kernels),
    comparing each replay's outputs (cleared to NaN first) and state with the
    eager ones."""
    outs = list(outs) + list(state)
    nclear = len(outs) - len(state)
    fn()
    torch.cuda.synchronize()
    want = [bits(o).copy() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                  # warm up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    junk = torch.randn(1 << 20, device=dev())
    for r in range(REPLAYS):
        for o in outs[:nclear]:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(bits(o), want[i], equal_nan=True), (label, r, i)
        say(f"[{label}] replay {r} matches")
        junk.mul_(1.0001).add_(0.5)           # unrelated eager work between replays
        fn()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(bits(o), want[i], equal_nan=True), (label, "eager", r, i)


@pytest.mark.parametrize("dyn", [None, "per_token_head"])
def test_decode_step_graph(dyn):
    case = synth.decode_case(200, 32, 8, 128, [3000, 77, 1], shuffle=True, spare_frac=0.2,
                             values="spread" if dyn else "normal")
    pre = split_newest(case)
    knew, vnew = newest_rows(case)
    full = GpuLayer(case, dyn=dyn)
    g = GpuLayer(pre, dyn=dyn, scales=None if dyn else full.scales_host())
    q = bf16_dev(case.q)
    kn, vn = bf16_dev(knew), bf16_dev(vnew)
    bt, lens = i32_dev(case.block_tables), i32_dev(case.lens)
    out = torch.empty((case.num_seqs, 32, 128), dtype=torch.float32, device=dev())
    ws = kv.alloc_workspace(g.desc, case.num_seqs, case.max_context_len)
    step = kv.decode_step_dynamic if dyn else kv.decode_step

    def fn():
        # the write is idempotent: every replay stores the same codes (and
        # scales) at the same slots before attending
        step(g.desc, kn, vn, g.k_cache, g.v_cache, out, q, bt, lens, case.max_context_len,
             g.k_scale, g.v_scale, ws)

    state = [g.k_cache, g.v_cache] + ([g.k_scale, g.v_scale] if dyn else [])
    replay_and_compare(fn, [out], f"decode step dyn={dyn}", state=state)
    assert np.array_equal(host(out), host(full.attend()))


def test_two_call_decode_graph():
    case = synth.decode_case(201, 64, 8, 128, [5000, 300], shuffle=True, spare_frac=0.2)
    g = GpuLayer(case)
    bt, lens = i32_dev(case.block_tables), i32_dev(case.lens)
    out = torch.empty((case.num_seqs, 64, 128), dtype=torch.bfloat16, device=dev())
    ws = kv.alloc_workspace(g.desc, case.num_seqs, case.max_context_len)

    def fn():
        kv.paged_decode_attention(g.desc, out, g.q, g.k_cache, g.v_cache, bt, lens,
                                  case.max_context_len, g.k_scale, g.v_scale, ws)

    replay_and_compare(fn, [out], "two-call decode (bf16 out)")


@pytest.mark.parametrize("attn", ["bf16", "fp8"])
def test_split_prefill_graph(attn):
    case = synth.prefill_case(202, 32, 8, 128, [6000, 900], [64, 20], shuffle=True,
                              spare_frac=0.2)
    g = GpuLayer(case, attn=attn)
    ws = kv.alloc_prefill_workspace(g.desc, case.num_seqs, case.max_query_len,
                                    case.block_tables.shape[1])
    assert ws is not None                     # the plan splits the keys
    qs = i32_dev(case.query_start)
    out = torch.empty((case.num_query_rows, 32, 128), dtype=torch.float32, device=dev())

    def fn():
        kv.paged_prefill_attention(g.desc, out, g.q, g.k_cache, g.v_cache, g.block_tables, qs,
                                   g.context_lens, case.max_query_len, g.k_scale, g.v_scale,
                                   workspace=ws)

    replay_and_compare(fn, [out], f"split prefill attn={attn}")


@pytest.mark.parametrize("per_head", [True, False])
def test_scale_calibration_and_prefill_write_graph(per_head):
    # The static scale calibration (clear, many-work-group atomic maximum,
    # finish: the caller's output words are the accumulator in between) and
    # a prefill-sized cache write with it, captured together: every replay
    # recomputes the scales from zero and rewrites the same bytes.
    case = synth.decode_case(203, 32, 8, 128, [5000, 1000], shuffle=True, spare_frac=0.2)
    desc = kv.layer_desc(32, 8, 128, scale_mode="per_kv_head" if per_head else "per_tensor")
    k, v = bf16_dev(case.k_new), bf16_dev(case.v_new)
    ks = torch.empty(8 if per_head else 1, dtype=torch.float32, device=dev())
    vs = torch.empty_like(ks)
    pc = synth.poisoned_cache(case.num_pages, 8, 128, True)
    kc, vc = torch.from_numpy(pc).to(dev()), torch.from_numpy(pc).to(dev())
    slots = torch.from_numpy(case.slots).to(dev())

    def fn():
        kv.kv_scale_from_amax(desc, k, ks)
        kv.kv_scale_from_amax(desc, v, vs)
        kv.kv_cache_write(desc, k, v, slots, kc, vc, ks, vs)

    replay_and_compare(fn, [ks, vs], f"calibration + write per_head={per_head}",
                       state=[kc, vc])
