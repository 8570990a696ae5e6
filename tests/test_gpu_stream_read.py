"""The streaming-read timing aid (kvq_stream_read) reads every byte once:
its per-work-group XOR checksums match the same XOR taken on the host over
the documented split of the buffer into contiguous shares."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_write_amd as kv

pytestmark = pytest.mark.gpu


def expected_sink(words, num_blocks):
    # work-group w reads the 16-byte chunks [w*per, min((w+1)*per, n16))
    n16 = words.size // 4
    per = -(-n16 // num_blocks)
    out = np.zeros(num_blocks, np.uint32)
    for w in range(num_blocks):
        a, b = min(w * per, n16), min((w + 1) * per, n16)
        if b > a:
            out[w] = np.bitwise_xor.reduce(words[4 * a:4 * b])
    return out


@pytest.mark.parametrize("n_bytes,num_blocks", [
    (16, 1), (4096, 3), (3 * (1 << 20) + 48, 7), (3 * (1 << 20) + 48, 256),
    (1 << 20, 1000), (160, 64),          # more work-groups than chunks: empty shares
])
def test_stream_read_checksums(n_bytes, num_blocks):
    rng = np.random.default_rng(n_bytes + num_blocks)
    words = rng.integers(0, 1 << 32, size=n_bytes // 4, dtype=np.uint32)
    src = torch.from_numpy(words.view(np.int32).copy()).cuda()
    sink = torch.full((num_blocks,), -1, dtype=torch.int32, device="cuda")
    kv.stream_read(src, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected_sink(words, num_blocks))
    assert np.bitwise_xor.reduce(got) == np.bitwise_xor.reduce(words)
