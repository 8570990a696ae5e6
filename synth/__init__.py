"""Seeded synthetic decode workloads, shared by the tests and the benchmark.

This module only draws inputs: bf16 query / key / value bits, sequence
lengths, page pools, block tables and slot mappings. It holds none of the
method's arithmetic (no quantisation, no scales, no attention); both the
oracle and the HIP path receive exactly the arrays made here.

Recipe (every stream comes from numpy PCG64 seeded with SeedSequence([2026,
workload id]) and spawned per purpose):
  * values: float32 standard normals rounded to bf16 (RNE, by torch);
  * "tiny": 2 fixed channels per KV head scaled x20 in K and in V (the
    fixed-channel outliers of "cooking-agi: FP8 and the KV cache", section
    "why K and V are grouped differently"), Q plain;
  * "drift": V[t,h,d] = beta[h,d] * t / L + N(0,1), beta ~ N(0,1), plus 64
    heavy-tail positions whose V rows are scaled x30;
  * batched: lengths uniform in [18000, 22000], a page pool of the needed
    pages plus 10% spare, randomly permuted;
  * unused pool pages and the tails of partial pages hold poison: 0x7F (the
    e4m3 NaN code) in fp8 caches and 0x7FC0 (a bf16 NaN) in bf16 caches.
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

PAGE = 16
POISON_FP8 = 0x7F
POISON_BF16 = 0x7FC0

_STREAMS = {"q": 0, "k": 1, "v": 2, "lens": 3, "perm": 4, "outlier": 5,
            "drift": 6, "heavy": 7, "new": 8, "extra": 9, "spread": 10}


def rng(workload: int, purpose: str) -> np.random.Generator:
    children = np.random.SeedSequence([2026, int(workload)]).spawn(len(_STREAMS))
    return np.random.Generator(np.random.PCG64(children[_STREAMS[purpose]]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def normal(workload: int, purpose: str, shape) -> np.ndarray:
    return rng(workload, purpose).standard_normal(size=shape, dtype=np.float32)


@dataclass
class DecodeCase:
    """One decode-attention input set for a layer.

    k_new / v_new hold every position of every sequence, concatenated in
    sequence order ([sum(lens)][Hkv][D] bf16 bits); slots gives each row's
    cache slot, so that writing all of them fills the caches."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    lens: np.ndarray            # int32 [B]
    q: np.ndarray               # uint16 [B][Hq][D]
    k_new: np.ndarray           # uint16 [T][Hkv][D]
    v_new: np.ndarray           # uint16 [T][Hkv][D]
    slots: np.ndarray           # int64 [T]
    block_tables: np.ndarray    # int32 [B][max_pages]
    num_pages: int
    seq_of_row: np.ndarray = field(default=None)  # int32 [T]
    pos_of_row: np.ndarray = field(default=None)  # int32 [T]

    @property
    def num_seqs(self):
        return int(self.lens.shape[0])

    @property
    def max_context_len(self):
        return int(self.lens.max()) if self.lens.size else 0


def make_pages(workload: int, lens, shuffle: bool, spare_frac: float = 0.0,
               max_pages_per_seq: Optional[int] = None):
    """Assign pages to sequences. Returns (block_tables, num_pages)."""
    lens = np.asarray(lens, dtype=np.int64)
    need = [(int(L) + PAGE - 1) // PAGE for L in lens]
    total = int(sum(need))
    num_pages = max(1, total + int(np.ceil(total * spare_frac)))
    ids = np.arange(num_pages, dtype=np.int32)
    if shuffle:
        ids = rng(workload, "perm").permutation(ids).astype(np.int32)
    mp = max_pages_per_seq or max(1, max(need) if need else 1)
    bt = np.zeros((len(lens), mp), dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        bt[b, :n] = ids[at:at + n]
        at += n
    return bt, num_pages


def slots_for(block_tables: np.ndarray, lens) -> tuple:
    """Slot of every position of every sequence, in sequence order."""
    rows_seq, rows_pos, slots = [], [], []
    for b, L in enumerate(np.asarray(lens, dtype=np.int64)):
        pos = np.arange(int(L), dtype=np.int64)
        slots.append(block_tables[b, pos // PAGE].astype(np.int64) * PAGE + pos % PAGE)
        rows_seq.append(np.full(int(L), b, dtype=np.int32))
        rows_pos.append(pos.astype(np.int32))
    if not slots:
        z = np.zeros(0, dtype=np.int64)
        return z, z.astype(np.int32), z.astype(np.int32)
    return (np.concatenate(slots), np.concatenate(rows_seq),
            np.concatenate(rows_pos))


def decode_case(workload: int, num_q_heads: int, num_kv_heads: int,
                head_dim: int, lens, shuffle: bool = False,
                spare_frac: float = 0.0, values: str = "normal",
                max_pages_per_seq: Optional[int] = None) -> DecodeCase:
    """values: "normal" (all N(0,1)), "tiny" (2 outlier channels x20 per KV
    head in K and V), "drift" (slow V mean drift and 64 heavy-tail rows) or
    "spread" (every (token, KV head) row of K and of V scaled by 2^u, u an
    integer drawn uniformly from -6..6: tokens of very different magnitude)."""
    lens = np.asarray(lens, dtype=np.int32)
    B, Hq, Hkv, D = len(lens), num_q_heads, num_kv_heads, head_dim
    T = int(lens.astype(np.int64).sum())
    bt, num_pages = make_pages(workload, lens, shuffle, spare_frac, max_pages_per_seq)
    slots, seq_of_row, pos_of_row = slots_for(bt, lens)
    q = normal(workload, "q", (B, Hq, D))
    k = normal(workload, "k", (T, Hkv, D))
    v = normal(workload, "v", (T, Hkv, D))
    if values == "tiny":
        r = rng(workload, "outlier")
        for h in range(Hkv):
            ch = r.choice(D, size=2, replace=False)
            k[:, h, ch] *= 20.0
            v[:, h, ch] *= 20.0
    elif values == "drift":
        beta = normal(workload, "drift", (Hkv, D))
        Lrow = lens[seq_of_row].astype(np.float32)
        frac = pos_of_row.astype(np.float32) / np.maximum(Lrow, 1.0)
        v += beta[None, :, :] * frac[:, None, None]
        r = rng(workload, "heavy")
        heavy = r.choice(T, size=min(64, T), replace=False)
        v[heavy] *= 30.0
    elif values == "spread":
        r = rng(workload, "spread")
        k *= np.exp2(r.integers(-6, 7, size=(T, Hkv, 1))).astype(np.float32)
        v *= np.exp2(r.integers(-6, 7, size=(T, Hkv, 1))).astype(np.float32)
    elif values != "normal":
        raise ValueError(values)
    return DecodeCase(Hq, Hkv, D, lens, bf16_bits(q), bf16_bits(k), bf16_bits(v),
                      slots, bt, num_pages, seq_of_row, pos_of_row)


def poisoned_cache(num_pages: int, num_kv_heads: int, head_dim: int,
                   fp8: bool) -> np.ndarray:
    """uint8 [P][Hkv][PB] filled with poison."""
    pb = PAGE * head_dim * (1 if fp8 else 2)
    c = np.empty((num_pages, num_kv_heads, pb), dtype=np.uint8)
    if fp8:
        c.fill(POISON_FP8)
    else:
        c.view(np.uint16).fill(POISON_BF16)
    return c


# Workload ids used across the tests and the benchmark.
TINY, LLAMA8B, BATCHED, LLAMA70B, HD256, GPTOSS = 1, 2, 3, 4, 5, 6

WORKLOADS = {
    TINY: dict(num_q_heads=4, num_kv_heads=2, head_dim=64, lens=[256],
               values="tiny"),
    LLAMA8B: dict(num_q_heads=32, num_kv_heads=8, head_dim=128),
    BATCHED: dict(num_q_heads=32, num_kv_heads=8, head_dim=128),
    LLAMA70B: dict(num_q_heads=64, num_kv_heads=8, head_dim=128,
                   values="drift"),
    HD256: dict(num_q_heads=8, num_kv_heads=2, head_dim=256),
    GPTOSS: dict(num_q_heads=64, num_kv_heads=8, head_dim=64),
}


def batched_lens(workload: int = BATCHED, num_seqs: int = 8, lo: int = 18000,
                 hi: int = 22000) -> np.ndarray:
    return rng(workload, "lens").integers(lo, hi + 1, size=num_seqs).astype(np.int32)


@dataclass
class PrefillCase(DecodeCase):
    """A chunked-prefill input: every position of every sequence is in
    k_new / v_new (written to the caches before the attention), and sequence
    b's last n_b positions are queries: q is [sum n_b][Hq][D], sequence b's
    rows are query_start[b] .. query_start[b+1]-1."""
    query_start: np.ndarray = field(default=None)   # int32 [B+1]

    @property
    def num_query_rows(self):
        return int(self.query_start[-1])

    @property
    def max_query_len(self):
        return int(np.diff(self.query_start).max()) if self.num_seqs else 0


def prefill_case(workload: int, num_q_heads: int, num_kv_heads: int, head_dim: int, lens,
                 chunk_lens, shuffle: bool = False, spare_frac: float = 0.0,
                 values: str = "normal") -> PrefillCase:
    """Sequences of lens[b] positions whose last chunk_lens[b] are the new
    (query) rows; K/V and block tables as decode_case draws them."""
    base = decode_case(workload, num_q_heads, num_kv_heads, head_dim, lens, shuffle,
                       spare_frac, values)
    n = np.asarray(chunk_lens, dtype=np.int32)
    assert n.shape == base.lens.shape and np.all(n <= base.lens) and np.all(n >= 0)
    qs = np.zeros(n.size + 1, dtype=np.int32)
    qs[1:] = np.cumsum(n)
    q = normal(workload, "extra", (int(qs[-1]), num_q_heads, head_dim))
    return PrefillCase(base.num_q_heads, base.num_kv_heads, base.head_dim, base.lens,
                       bf16_bits(q), base.k_new, base.v_new, base.slots, base.block_tables,
                       base.num_pages, base.seq_of_row, base.pos_of_row, qs)
