"""kvq_paged_decode_attention_noalloc: the decode attention with the
library's own device scratch array as its split workspace, for callers that
cannot allocate. Checked against kvq_paged_decode_attention (caller-owned
workspace) on the same inputs: the same kernels, so the same bits. Two calls
in a row, the second smaller, so the second runs on the array the first left
behind; then the size limit."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_write_amd as kv
import synth
from _gpu import GpuLayer, OracleLayer, errors, GATE_MAX_ABS, GATE_MEAN_ABS

pytestmark = pytest.mark.gpu


def _both(layer):
    c = layer.case
    shape = (c.num_seqs, c.num_q_heads, c.head_dim)
    ref = layer.attend()
    assert kv.decode_workspace_bytes(layer.desc, c.num_seqs, c.max_context_len) > 0
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    kv.paged_decode_attention_noalloc(layer.desc, out, layer.q, layer.k_cache, layer.v_cache,
                                      layer.block_tables, layer.context_lens,
                                      c.max_context_len, layer.k_scale, layer.v_scale)
    torch.cuda.synchronize()
    return out, ref


@pytest.mark.parametrize("fmt", ["fp8_e4m3", "bf16"])
def test_noalloc_matches_the_workspace_entry_point(fmt):
    fp8 = fmt != "bf16"
    # first call: a ragged batch of the 8B layer shape with many partitions
    big = synth.decode_case(71, 32, 8, 128, [9000, 4100, 77, 0, 6001], shuffle=True,
                            spare_frac=0.2)
    print(f"noalloc first call: {fmt} lens={list(big.lens)}", flush=True)
    g1 = GpuLayer(big, fp8=fp8)
    out1, ref1 = _both(g1)
    assert torch.equal(out1, ref1), "first call differs from kvq_paged_decode_attention"
    mx, mn = errors(out1, OracleLayer(big, fp8=fp8).attend())
    assert mx <= GATE_MAX_ABS and mn <= GATE_MEAN_ABS, (mx, mn)
    # second call, smaller: fewer sequences, partitions and heads
    small = synth.decode_case(72, 8, 2, 64, [700, 1500], shuffle=True)
    print(f"noalloc second call: {fmt} lens={list(small.lens)}", flush=True)
    g2 = GpuLayer(small, fp8=fp8)
    out2, ref2 = _both(g2)
    assert torch.equal(out2, ref2), "second call differs from kvq_paged_decode_attention"
    mx, mn = errors(out2, OracleLayer(small, fp8=fp8).attend())
    assert mx <= GATE_MAX_ABS and mn <= GATE_MEAN_ABS, (mx, mn)


def test_noalloc_rejects_plans_beyond_its_array():
    d = kv.layer_desc(32, 8, 128)
    assert kv.decode_workspace_bytes(d, 64, 131072) > kv.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((64, 32, 128), dtype=torch.float32, device="cuda")
    kc = torch.zeros((1, 8, d.page_bytes), dtype=torch.uint8, device="cuda")
    bt = torch.zeros((64, 8192), dtype=torch.int32, device="cuda")
    lens = torch.ones(64, dtype=torch.int32, device="cuda")
    s = torch.ones(8, dtype=torch.float32, device="cuda")
    with pytest.raises(kv.Kvfp8Error) as e:
        kv.paged_decode_attention_noalloc(d, out, q, kc, kc, bt, lens, 131072, s, s)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0     # nothing ran
