"""Accumulation precision of the matrix instructions (tests/hw/
mfma_accumulation.hip, run as a child process). The bf16 MFMA that every
bf16-arithmetic path uses sums exact products like an FP32 accumulator. The
fp8 MFMA of the all-FP8 mode sums each instruction's 32 products to about
13 bits, but carries its accumulator at FP32: chaining it gives what adding
each instruction's result in FP32 gives, up to rounding order. So neither
has the long-contraction loss of Hopper's FP8 tensor cores ("vLLM FP8
KV-Cache and Attention Quantization Update", section "Two-Level Accumulation
for Accuracy"); the all-FP8 mode folds each 32-position block into FP32
because its P is quantised relative to the block's own maximum."""

import json
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "hw", "mfma_accumulation.bin")


def test_mfma_accumulation_precision():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "build() compiles tests/hw/mfma_accumulation.hip"
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    r = json.loads(res.stdout.strip().splitlines()[-1])
    print(r)
    # a sequential FP32 sum of 128 exact products errs by at most about
    # 127 * 2^-24 of the sum of their magnitudes
    assert r["fp32_sequential"] <= 127 * 2.0 ** -24
    # the bf16 MFMA: FP32-class summation (within 4x of the sequential sum's bound)
    assert r["bf16_16x16x32_chain"] <= 4 * 127 * 2.0 ** -24, r
    # the fp8 MFMA: a dot product, coarser than FP32 but well inside the
    # all-FP8 mode's parity bar (its P codes step by 1/16)
    assert r["fp8_16x16x32_chain"] <= 2.0 ** -10, r
    assert r["fp8_16x16x128"] <= 2.0 ** -10, r
    # the fp8 accumulator itself: chained = folded in FP32, up to a few
    # FP32 roundings of the running sum
    assert r["fp8_chain_minus_fp32_fold"] <= 4 * 2.0 ** -24, r
