#!/usr/bin/env python3
"""Decode-step benchmark of the FP8 e4m3 paged KV cache on one MI355X.

A step is one decode step of a layer stack: for every layer, write the new
token's K/V into the paged cache (kv_cache_write) and run GQA decode attention
over the cache (split + reduce kernels). Inputs are synthetic, seeded and
resident in HBM before timing; the layer stack is large enough (>= 1 GiB of
cache) that the 256 MB Infinity Cache cannot serve it.

Default run (about a minute of GPU time):
  * headline: Llama-3.1-8B-shaped layer (32 q / 8 KV heads, head_dim 128),
    batch 1, context 131072, fp8 e4m3 cache with per-KV-head scales, 32
    layers per step -> value = KV GB/s of the whole step;
  * sweep over contexts 16..128k for the fp8 and the bf16 cache with a linear
    fit us/layer = slope * context + intercept over 8k..128k (the ITL fit of
    "State of FP8 KV cache and attention quantization in vLLM", section
    "Single-request benchmark"), the fp8/bf16 slope ratio and the break-even
    context, beside the cost of one dependent launch in a captured graph (the
    floor under the intercept);
  * the fp8 step at 262144, 524288 and 1048576 positions (long_contexts);
  * roofline of the split kernel from HIP events around its launches;
  * the float64 CPU oracle timed on the host as a reported baseline.

Prints one JSON line (rank 0, N = 1).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
GIB = 1 << 30

WORKLOADS = {
    # name: (B, Hq, Hkv, D, default context, layers of the model)
    "llama8b": dict(B=1, Hq=32, Hkv=8, D=128, ctx=131072, layers=32,
                    desc="Llama-3.1-8B-shaped decode layer (32 q / 8 KV heads, head_dim 128), batch 1"),
    "batched": dict(B=8, Hq=32, Hkv=8, D=128, ctx=None, layers=32,
                    desc="8 sequences of 18k-22k positions, 8B layer shape, shuffled page pool"),
    "llama70b": dict(B=1, Hq=64, Hkv=8, D=128, ctx=131072, layers=80,
                     desc="Llama-3.1-70B-shaped decode layer (64 q / 8 KV heads, head_dim 128), batch 1"),
    "hd256": dict(B=1, Hq=8, Hkv=2, D=256, ctx=65536, layers=32,
                  desc="head_dim 256 layer (8 q / 2 KV heads), batch 1"),
    "gptoss": dict(B=1, Hq=64, Hkv=8, D=64, ctx=32768, layers=24,
                   desc="gpt-oss-20b-like hybrid: full fp8 layers and sliding-window-128 bf16 layers"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class LayerStack:
    """NL layers of one shape, each with its own caches, filled with seeded
    synthetic K/V up to position L-1; a step writes position L-1 and attends
    over L positions."""

    def __init__(self, kv, torch, B, Hq, Hkv, D, lens, NL, cache_dtype="fp8_e4m3",
                 window=0, shuffle=False, spare_frac=0.0, seed=0, dtypes=None, path="fused",
                 attn="bf16", scales="per_kv_head"):
        self.kv, self.torch = kv, torch
        self.path = path
        dev = torch.device("cuda:0")
        self.dev = dev
        self.B, self.Hq, self.Hkv, self.D = B, Hq, Hkv, D
        self.lens = [int(x) for x in lens]
        self.NL = NL
        self.max_len = max(self.lens)
        dtypes = dtypes or [cache_dtype] * NL
        windows = window if isinstance(window, list) else [window] * NL
        self.descs = [kv.layer_desc(Hq, Hkv, D, dtypes[i], scales, windows[i],
                                    attn=attn if dtypes[i] != "bf16" else "bf16")
                      for i in range(NL)]
        import numpy as np
        need = [(L + 15) // 16 for L in self.lens]
        total = sum(need)
        num_pages = total + int(math.ceil(total * spare_frac))
        ids = np.arange(num_pages, dtype=np.int32)
        if shuffle:
            ids = np.random.default_rng(seed + 99).permutation(ids).astype(np.int32)
        mp = max(need)
        bt = np.zeros((B, mp), dtype=np.int32)
        at = 0
        for b, n in enumerate(need):
            bt[b, :n] = ids[at:at + n]
            at += n
        self.num_pages = num_pages
        self.block_tables = torch.from_numpy(bt).to(dev)
        self.context_lens = torch.tensor(self.lens, dtype=torch.int32, device=dev)
        # slots of every position (all sequences), and of the newest ones
        slots, newest = [], []
        for b, L in enumerate(self.lens):
            pos = np.arange(L, dtype=np.int64)
            s = bt[b, pos // 16].astype(np.int64) * 16 + pos % 16
            slots.append(s[:-1])
            newest.append(s[-1])
        self.fill_slots = torch.from_numpy(np.concatenate(slots)).to(dev)
        self.new_slots = torch.tensor(newest, dtype=torch.int64, device=dev)
        gen = torch.Generator(device=dev)
        self.layers = []
        T = int(self.fill_slots.numel())
        for li in range(NL):
            d = self.descs[li]
            gen.manual_seed(seed * 1000 + li)
            kc = torch.empty(kv.cache_shape(d, num_pages), dtype=torch.uint8, device=dev)
            vc = torch.empty_like(kc)
            k_all = torch.randn((T + B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
            v_all = torch.randn((T + B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
            if d.dynamic:
                # dynamic per-token scales: pools beside the pages, set by the write
                ks = torch.zeros(kv.scale_pool_shape(d, num_pages), dtype=torch.float32,
                                 device=dev)
                vs = torch.zeros_like(ks)
                kv.kv_cache_write_dynamic(d, k_all[:T], v_all[:T], self.fill_slots, kc, vc, ks,
                                          vs)
            else:
                if d.fp8:
                    ks = torch.empty(Hkv, dtype=torch.float32, device=dev)
                    vs = torch.empty(Hkv, dtype=torch.float32, device=dev)
                    kv.kv_scale_from_amax(d, k_all, ks)
                    kv.kv_scale_from_amax(d, v_all, vs)
                else:
                    ks = vs = None
                kv.kv_cache_write(d, k_all[:T], v_all[:T], self.fill_slots, kc, vc, ks, vs)
            k_new = k_all[T:].contiguous()
            v_new = v_all[T:].contiguous()
            q = torch.randn((B, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
            ws = kv.alloc_workspace(d, B, self.max_len)
            self.layers.append(dict(desc=d, kc=kc, vc=vc, ks=ks, vs=vs, k_new=k_new,
                                    v_new=v_new, q=q, out=out, ws=ws))
            del k_all, v_all
        torch.cuda.synchronize()

    def step(self):
        """One decode step of every layer: the new token's cache write, then
        the attention. path "fused": one kvq_decode_step call per layer (the
        split kernel does the write); "separate": kvq_kv_cache_write then
        kvq_paged_decode_attention."""
        kv = self.kv
        for ly in self.layers:
            d = ly["desc"]
            if self.path == "fused":
                step = kv.decode_step_dynamic if d.dynamic else kv.decode_step
                step(d, ly["k_new"], ly["v_new"], ly["kc"], ly["vc"], ly["out"], ly["q"],
                     self.block_tables, self.context_lens, self.max_len, ly["ks"], ly["vs"],
                     ly["ws"])
            else:
                write = kv.kv_cache_write_dynamic if d.dynamic else kv.kv_cache_write
                write(d, ly["k_new"], ly["v_new"], self.new_slots, ly["kc"], ly["vc"], ly["ks"],
                      ly["vs"])
                kv.paged_decode_attention(d, ly["out"], ly["q"], ly["kc"], ly["vc"],
                                          self.block_tables, self.context_lens, self.max_len,
                                          ly["ks"], ly["vs"], ly["ws"])

    # ---- algorithmic byte model (per layer) -------------------------------
    def attended(self, desc):
        W = desc.sliding_window
        return [min(L, W) if W > 0 else L for L in self.lens]

    def kv_bytes(self, desc):
        return sum(self.attended(desc)) * self.Hkv * self.D * 2 * desc.elem_bytes

    def split_bytes(self, desc):
        """Bytes the split kernel must read: K/V rows, q, block-table
        entries, scales."""
        n = self.attended(desc)
        bt = sum((x + 15) // 16 + 1 for x in n) * 4
        if desc.dynamic:      # a K and a V scale per attended position and KV head
            sc = sum(n) * self.Hkv * 2 * 4
        else:
            sc = 2 * self.Hkv * 4 if desc.fp8 else 0
        return self.kv_bytes(desc) + self.B * self.Hq * self.D * 2 + bt + sc

    def write_bytes(self, desc):
        """The cache write of the new tokens: bf16 K/V in, cache rows out."""
        sc = self.B * self.Hkv * 2 * 4 if desc.dynamic else 0    # the new rows' scales
        return self.B * self.Hkv * self.D * 2 * (2 + desc.elem_bytes) + sc

    def step_bytes(self, desc):
        """Whole layer step: attention (K/V, q, out, block table, scales) plus
        the cache write of the new tokens."""
        return self.split_bytes(desc) + self.B * self.Hq * self.D * 4 + self.write_bytes(desc)

    def total_step_bytes(self):
        return sum(self.step_bytes(ly["desc"]) for ly in self.layers)

    def total_kv_bytes(self):
        return sum(self.kv_bytes(ly["desc"]) for ly in self.layers)


SCALE_TEXT = {"per_kv_head": "per-KV-head scales", "per_tensor": "per-tensor scales",
              "per_token": "dynamic per-token scales",
              "per_token_head": "dynamic per-token, per-KV-head scales"}


_SLEEP_HZ = []


def gpu_head_start(torch, launches):
    """Occupy the GPU (torch's spin kernel) for about 0.06 ms per launch that
    follows, at least 20 ms: the host then enqueues those launches while the
    GPU waits, and kernel-event timestamps bracket GPU work only. A launch
    with an event pair costs the host more time (about 40 us per layer step)
    than the split kernel takes below about 64k positions, so without a head
    start the pairs would time the host's launch rate."""
    if not _SLEEP_HZ:
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(10_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_HZ.append(1e7 / (e0.elapsed_time(e1) * 1e-3))
    ms = min(400.0, max(20.0, 0.06 * launches))
    torch.cuda._sleep(int(ms * 1e-3 * _SLEEP_HZ[0]))


def time_steps(torch, kv, stack, steps, warmup, profile=True):
    """Eager steps: mean ms per step (no profiling events: the host's launch
    rate included, as a caller that does not capture a graph sees it) and,
    with profile, the split kernel's mean duration from the library's
    kernel-timestamped HIP events over a second pass of the same steps that
    starts behind a GPU head start (gpu_head_start)."""
    for _ in range(warmup):
        stack.step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        stack.step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    if not profile:
        return ms, None, 0
    kv.profile_begin(steps * stack.NL)
    gpu_head_start(torch, steps * stack.NL)
    for _ in range(steps):
        stack.step()
    split_ms, n = kv.profile_end()
    return ms, (split_ms / n if n else None), n


def same_size_read_us(torch, kv, nbytes, min_total=2 * GIB, reps=10):
    """Graph-timed plain streaming read (kvq_stream_read) of nbytes per
    launch, over enough distinct buffers that the Infinity Cache cannot
    serve them: the mean launch time, best of 1024 and 4096 work-groups.
    What a read-only kernel with no attention work takes for one layer's
    bytes."""
    nbytes = nbytes // 16 * 16
    n = max(8, min(256, math.ceil(min_total / nbytes)))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1) for _ in range(n)]
    best = None
    for blocks in (1024, 4096):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        kv.stream_read(bufs[0], sink)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for b in bufs:
                kv.stream_read(b, sink)
        for _ in range(3):
            g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * n)
        best = us if best is None else min(best, us)
        del g
    del bufs
    torch.cuda.empty_cache()
    return best


def same_size_read_kernel_us(torch, kv, nbytes, min_total=2 * GIB, reps=4):
    """The plain streaming read of nbytes per launch timed like the split
    kernel: kernel-timestamped HIP event pairs (kvq_profile_begin/end) around
    eager launches over distinct buffers, behind a GPU head start; the mean
    kernel time, best of 1024 and 4096 work-groups."""
    nbytes = nbytes // 16 * 16
    n = max(8, min(256, math.ceil(min_total / nbytes)))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1) for _ in range(n)]
    best = None
    for blocks in (1024, 4096):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        for b in bufs[:2]:
            kv.stream_read(b, sink)
        torch.cuda.synchronize()
        kv.profile_begin(reps * n)
        gpu_head_start(torch, reps * n)
        for _ in range(reps):
            for b in bufs:
                kv.stream_read(b, sink)
        ms, cnt = kv.profile_end()
        us = ms * 1e3 / cnt if cnt else None
        if us is not None:
            best = us if best is None else min(best, us)
    del bufs
    torch.cuda.empty_cache()
    return best


def time_steps_graph(torch, stack, steps, warmup, per_step=False):
    """The step captured once as a HIP graph, replayed: mean ms per step
    (and, with per_step, the sorted ms of every replay of a second pass).
    The replayed outputs are checked against the eager step's."""
    stack.step()
    torch.cuda.synchronize()
    ref = [ly["out"].clone() for ly in stack.layers]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stack.step()
    for _ in range(max(warmup, 1)):
        g.replay()
    torch.cuda.synchronize()
    for ly, r in zip(stack.layers, ref):
        if not torch.equal(ly["out"], r):
            raise RuntimeError("graph replay differs from the eager step")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    if per_step:
        # a second pass with an event pair around every replay, for the spread
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        del g
        return ms, sorted(a.elapsed_time(b) for a, b in evs)
    del g
    return ms


def percentile(sorted_xs, q):
    """Linear-interpolated percentile of an ascending list."""
    if len(sorted_xs) == 1:
        return sorted_xs[0]
    pos = (len(sorted_xs) - 1) * q
    lo = int(math.floor(pos))
    hi = min(lo + 1, len(sorted_xs) - 1)
    return sorted_xs[lo] + (sorted_xs[hi] - sorted_xs[lo]) * (pos - lo)


def read_ceiling_gbs(torch, kv, reps=5):
    """Measured device ceilings on a 4 GiB buffer: the library's plain
    streaming read (kvq_stream_read: every byte once, 16-byte non-temporal
    loads, best over work-group counts) and torch's device copy (read +
    write bytes). GB/s each."""
    x = torch.ones(GIB, dtype=torch.float32, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    best = 0.0
    for blocks in (1024, 2048, 4096, 8192):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        kv.stream_read(x, sink)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            kv.stream_read(x, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 4 * GIB * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy = 2 * 4 * GIB * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return best, copy


KERNEL_SOURCES = ["fp8_kv_cache_write_amd/csrc/paged_decode.hpp",
                  "fp8_kv_cache_write_amd/csrc/paged_decode.hip",
                  "fp8_kv_cache_write_amd/csrc/paged_decode_d128.hip",
                  "fp8_kv_cache_write_amd/csrc/device_common.hpp",
                  "fp8_kv_cache_write_amd/csrc/launch.hpp",
                  "fp8_kv_cache_write_amd/csrc/api.cpp"]
TRAFFIC_PROFILE = "profiles/paged_decode_split_llama8b_128k_fp8_traffic.json"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload_key):
    """HBM bytes per split-kernel launch from the committed rocprofv3 PMC
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's readings), or
    None when it was taken on other kernel sources or another workload."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != kernel_source_hash() or t.get("workload") != workload_key:
        return None
    return t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]


def layers_for(bytes_per_layer, lo=8, hi=512, target=2 * GIB):
    return int(min(hi, max(lo, math.ceil(target / max(bytes_per_layer, 1)))))


def fit(xs, ys):
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    sxy = sum((x - mx) * (y - my) for x, y in zip(xs, ys))
    slope = sxy / sxx
    return slope, my - slope * mx


def graph_kernel_floor(torch, n=64, reps=20):
    """Mean cost of one launch in a captured graph of n dependent 1-element
    torch kernels: the per-kernel floor that every layer step's kernels pay."""
    x = torch.zeros(1, device="cuda")
    x.add_(1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            x.add_(1)
    for _ in range(3):
        g.replay()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n)


def gptoss_sweep(torch, kv, w, contexts, steps, warmup, window=128, per_type=12):
    """The gpt-oss-like hybrid by layer type: graph-timed per-layer cost of a
    full-attention layer and of a sliding-window layer, each with an fp8 and
    a bf16 cache, over contexts. From them, the per-step cost of three model
    configurations of per_type full + per_type windowed layers (all bf16,
    all fp8, and fp8 with the windowed layers kept bf16: the skip path) and
    a linear fit of each against context (the vLLM post's gpt-oss
    comparison, "Single-request benchmark")."""
    rows = []
    for ctx in contexts:
        t = {}
        for kind, win in (("full", 0), ("window", window)):
            for dt in ("fp8_e4m3", "bf16"):
                e = 1 if dt.startswith("fp8") else 2
                if win == 0:
                    NL = layers_for(ctx * w["Hkv"] * w["D"] * 2 * e, hi=64)
                else:
                    NL = 32   # a window reads 128 positions: launch-bound at any size
                st = LayerStack(kv, torch, 1, w["Hq"], w["Hkv"], w["D"], [ctx], NL, dt,
                                window=win, seed=ctx + 7)
                t[(kind, dt)] = time_steps_graph(torch, st, steps, warmup) * 1e3 / NL
                del st
                torch.cuda.empty_cache()
        row = dict(context=ctx, full_fp8_us=round(t[("full", "fp8_e4m3")], 3),
                   full_bf16_us=round(t[("full", "bf16")], 3),
                   window_fp8_us=round(t[("window", "fp8_e4m3")], 3),
                   window_bf16_us=round(t[("window", "bf16")], 3))
        row["step_us"] = {
            "all_bf16": round(per_type * (t[("full", "bf16")] + t[("window", "bf16")]), 2),
            "all_fp8": round(per_type * (t[("full", "fp8_e4m3")] + t[("window", "fp8_e4m3")]),
                             2),
            "fp8_skip_window": round(per_type * (t[("full", "fp8_e4m3")]
                                                 + t[("window", "bf16")]), 2)}
        log(f"gptoss ctx={ctx:6d} full fp8/bf16 {row['full_fp8_us']:.2f}/{row['full_bf16_us']:.2f}"
            f" us, window fp8/bf16 {row['window_fp8_us']:.2f}/{row['window_bf16_us']:.2f} us")
        rows.append(row)
    out = dict(points=rows, layers=f"{per_type} full + {per_type} window-{window}",
               window_note="windowed layers read 128 positions, so their caches stay in the "
                           "Infinity Cache across replays; they are launch-bound either way")
    fits = {}
    for cfg in ("all_bf16", "all_fp8", "fp8_skip_window"):
        s_, b_ = fit([r["context"] for r in rows], [r["step_us"][cfg] for r in rows])
        fits[cfg] = dict(slope_us_per_token=s_, intercept_us=b_)
    out["fits"] = fits
    bb = fits["all_bf16"]["slope_us_per_token"]
    out["slope_ratio_all_fp8_over_bf16"] = fits["all_fp8"]["slope_us_per_token"] / bb
    out["slope_ratio_skip_over_bf16"] = fits["fp8_skip_window"]["slope_us_per_token"] / bb
    return out


TRACE_POINTS = [
    ("llama8b_32768", ["--context", "32768"]),
    ("llama8b_65536", ["--context", "65536"]),
    ("llama8b_98304", ["--context", "98304"]),
    ("hd256_65536", ["--workload", "hd256", "--context", "65536"]),
    ("gptoss_full_32768", ["--workload", "gptoss", "--context", "32768"]),
]


def trace_point_kernel_times(args, timeout=150):
    """One trace point in a child `rocprofv3 --kernel-trace -- bench.py
    --trace-point ARGS` (graph-replayed decode steps, then plain reads of the
    split kernel's bytes per launch at 1024 and 4096 work-groups): the split
    kernel's and the read's mean dispatch times (the read: the better
    work-group count). None when the run fails or leaves no trace. Runs in
    the trace server, a process that never touches the GPU."""
    import glob
    import shutil
    import subprocess
    import tempfile
    exe = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    if not os.path.exists(exe):
        return None
    env = dict(os.environ, TMPDIR="/tmp")
    with tempfile.TemporaryDirectory(dir="/tmp") as d:
        cmd = [exe, "--kernel-trace", "-d", d, "-o", "tp", "--output-format", "csv", "--",
               sys.executable, os.path.abspath(__file__), "--trace-point", *args]
        # the profiler and the program under it in a process group of their
        # own, so that a run past its time limit is ended whole
        try:
            proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                                    text=True, env=env, cwd=ROOT, start_new_session=True)
        except OSError:
            return None
        try:
            stdout, _ = proc.communicate(timeout=timeout)
        except subprocess.TimeoutExpired:
            import signal
            try:
                os.killpg(proc.pid, signal.SIGKILL)
            except OSError:
                pass
            proc.communicate()
            return None
        # the profiler may end with a fault of its own after the program has
        # finished: the trace is used when the program's own line printed
        if not any(l.startswith("{") for l in stdout.splitlines()):
            return None
        return split_read_times(
            glob.glob(os.path.join(d, "**", "tp_kernel_trace.csv"), recursive=True))


def split_read_times(trace_csvs):
    """From rocprofv3 kernel-trace CSV files: the split kernel's mean
    dispatch time, the plain read's (the better of its work-group counts)
    and their ratio, or None when either kernel is missing."""
    import csv
    split, read = [], {}
    for f in trace_csvs:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                n = row["Kernel_Name"]
                dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
                if "paged_decode_split_kernel" in n:
                    split.append(dur)
                elif "stream_read_kernel" in n:
                    wg = int(row["Grid_Size_X"]) // int(row["Workgroup_Size_X"])
                    read.setdefault(wg, []).append(dur)
    if not split or not read:
        return None
    sp = sum(split) / len(split)
    rd = min(sum(v) / len(v) for v in read.values())
    return dict(split_us=round(sp, 3), read_us=round(rd, 3), ratio=round(sp / rd, 4),
                split_launches=len(split))


def trace_server():
    """`bench.py --trace-server`: one JSON request per stdin line ({"args":
    [...]}), one JSON reply per line (trace_point_kernel_times). The bench
    starts it before it initialises the GPU, so the profiler runs start from a
    process that never touched the GPU."""
    for line in sys.stdin:
        try:
            req = json.loads(line)
            res = trace_point_kernel_times(req["args"])
        except Exception:      # a malformed request or a failed run: no result
            res = None
        sys.stdout.write(json.dumps(res) + "\n")
        sys.stdout.flush()


def start_trace_server():
    """The trace server as a child process (before any GPU use), or None."""
    import subprocess
    try:
        return subprocess.Popen([sys.executable, os.path.abspath(__file__), "--trace-server"],
                                stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True, cwd=ROOT)
    except OSError:
        return None


def kernel_trace_ratios(server, points=TRACE_POINTS, timeout=200):
    """The split kernel against a plain read of the same bytes, both timed by
    the profiler's dispatch timestamps, per point ({point: {split_us, read_us,
    ratio, split_launches}}, None for a point without a result; None with no
    server). Kernel-event pairs cannot time the graph-replayed split kernel,
    and in eager launches it runs about 1.4 us longer than under graph
    replay."""
    import select
    if server is None or server.poll() is not None:
        return None
    out = {}
    for name, args in points:
        out[name] = None
        try:
            server.stdin.write(json.dumps({"args": args}) + "\n")
            server.stdin.flush()
            ready, _, _ = select.select([server.stdout], [], [], timeout)
            if not ready:
                log(f"kernel trace {name}: no reply in {timeout} s")
                server.kill()
                break
            res = json.loads(server.stdout.readline() or "null")
        except (OSError, ValueError):
            break
        out[name] = res
        if res:
            log(f"kernel trace {name}: split {res['split_us']:.2f} us, same-size read "
                f"{res['read_us']:.2f} us ({res['ratio']:.3f}x)")
        else:
            log(f"kernel trace {name}: no result")
    return out


def stop_trace_server(server):
    if server is None:
        return
    try:
        server.stdin.close()
        server.wait(timeout=10)
    except Exception:
        server.kill()


def long_contexts(torch, kv, w, contexts, steps, warmup):
    """The fp8 decode step past 131072 positions (per-KV-head scales, one
    sequence, graph-replayed): at least 2 GiB of cache per stack."""
    rows = []
    for ctx in contexts:
        per_layer = ctx * w["Hkv"] * w["D"] * 2
        NL = layers_for(per_layer, lo=4)
        st = LayerStack(kv, torch, 1, w["Hq"], w["Hkv"], w["D"], [ctx], NL, "fp8_e4m3", seed=ctx)
        ms = time_steps_graph(torch, st, steps, warmup)
        gbs = st.total_kv_bytes() / (ms * 1e-3) / 1e9
        del st
        torch.cuda.empty_cache()
        rows.append(dict(context=ctx, layers=NL, us_per_layer=round(ms * 1e3 / NL, 3),
                         kv_gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4)))
        log(f"long context {ctx:8d} layers={NL:2d} {ms * 1e3 / NL:9.2f} us/layer {gbs:7.1f} GB/s")
    return rows


def sweep(torch, kv, w, contexts, steps, warmup):
    rows = []
    for dt in ("fp8_e4m3", "bf16"):
        e = 1 if dt.startswith("fp8") else 2
        for ctx in contexts:
            per_layer = ctx * w["Hkv"] * w["D"] * 2 * e
            NL = layers_for(per_layer)
            st = LayerStack(kv, torch, 1, w["Hq"], w["Hkv"], w["D"], [ctx], NL, dt, seed=ctx)
            ms = time_steps_graph(torch, st, steps, warmup)
            # eager steps (no graph, no events), then the event-timed pass
            ms_eager, split_ms, _ = time_steps(torch, kv, st, 3, 1)
            us_layer = ms * 1e3 / NL
            gbs = st.total_kv_bytes() / (ms * 1e-3) / 1e9
            d0 = st.layers[0]["desc"]
            split_bytes = st.split_bytes(d0) + st.write_bytes(d0)
            del st
            torch.cuda.empty_cache()
            # (from 4096 positions: smaller reads would run from the Infinity Cache)
            read_us = same_size_read_us(torch, kv, split_bytes) if ctx >= 4096 else None
            read_k = same_size_read_kernel_us(torch, kv, split_bytes) if ctx >= 4096 else None
            split_us = split_ms * 1e3 if split_ms else None
            rows.append(dict(cache=dt, context=ctx, layers=NL, us_per_layer=round(us_layer, 3),
                             us_per_layer_eager=round(ms_eager * 1e3 / NL, 3),
                             kv_gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4),
                             split_us=round(split_us, 3) if split_us else None,
                             same_size_read_us=round(read_us, 3) if read_us else None,
                             step_over_same_size_read=round(us_layer / read_us, 3)
                             if read_us else None,
                             same_size_read_kernel_us=round(read_k, 3) if read_k else None,
                             split_over_same_size_read_kernel=round(split_us / read_k, 3)
                             if read_k and split_us else None))
            log(f"sweep {dt:8s} ctx={ctx:6d} layers={NL:3d} {us_layer:8.2f} us/layer "
                f"{gbs:7.1f} GB/s split={rows[-1]['split_us']} us read={read_us} us")
    fits = {}
    fits_eager = {}
    for dt in ("fp8_e4m3", "bf16"):
        for key, dst in (("us_per_layer", fits), ("us_per_layer_eager", fits_eager)):
            pts = [(r["context"], r[key]) for r in rows
                   if r["cache"] == dt and r["context"] >= 8192]
            if len(pts) >= 2:
                s, b = fit([p[0] for p in pts], [p[1] for p in pts])
                dst[dt] = dict(slope_us_per_token=s, intercept_us=b)
    out = dict(points=rows, fit_range="8192..%d" % max(contexts),
               graph_kernel_floor_us=round(graph_kernel_floor(torch), 3))
    if "fp8_e4m3" in fits and "bf16" in fits:
        f, bb = fits["fp8_e4m3"], fits["bf16"]
        out["fits"] = fits
        out["slope_ratio_fp8_over_bf16"] = f["slope_us_per_token"] / bb["slope_us_per_token"]
        ds = bb["slope_us_per_token"] - f["slope_us_per_token"]
        out["break_even_context"] = ((f["intercept_us"] - bb["intercept_us"]) / ds
                                     if ds > 0 else None)
    # the same fit over eager steps (each layer's calls launched from the
    # host, no graph): a second intercept beside the graph-replayed one
    if "fp8_e4m3" in fits_eager and "bf16" in fits_eager:
        out["fits_eager"] = fits_eager
        out["slope_ratio_fp8_over_bf16_eager"] = (fits_eager["fp8_e4m3"]["slope_us_per_token"] /
                                                  fits_eager["bf16"]["slope_us_per_token"])
    return out


PREFILL_LENGTHS = [1024, 2048, 4096, 8192, 16384, 32768]


CHUNKED_PREFILL = [(512, 8192), (512, 32768), (512, 131072), (2048, 131072)]


def chunked_prefill_bench(torch, kv, w, cases, steps, warmup, scales="per_kv_head", attn="bf16"):
    """Chunked prefill per layer: the last `chunk` rows of a context of
    `ctx` positions (already in the fp8 cache) attend causally to their
    prefix, once with the key split (a workspace from
    alloc_prefill_workspace) and once without. Flops: 4 D Hq per (row,
    attended key) pair."""
    dev = torch.device("cuda:0")
    Hq, Hkv, D = w["Hq"], w["Hkv"], w["D"]
    d = kv.layer_desc(Hq, Hkv, D, "fp8_e4m3", scales, attn=attn)
    rows = []
    for chunk, L in cases:
        gen = torch.Generator(device=dev)
        gen.manual_seed(chunk * 7 + L)
        pages = (L + 15) // 16
        kc = torch.empty(kv.cache_shape(d, pages), dtype=torch.uint8, device=dev)
        vc = torch.empty_like(kc)
        k = torch.randn((L, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((L, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
        q = torch.randn((chunk, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
        out = torch.empty((chunk, Hq, D), dtype=torch.bfloat16, device=dev)
        slots = torch.arange(L, dtype=torch.int64, device=dev)
        bt = torch.arange(pages, dtype=torch.int32, device=dev).view(1, pages)
        qs = torch.tensor([0, chunk], dtype=torch.int32, device=dev)
        lens = torch.tensor([L], dtype=torch.int32, device=dev)
        if d.dynamic:
            ks = torch.zeros(kv.scale_pool_shape(d, pages), dtype=torch.float32, device=dev)
            vs = torch.zeros_like(ks)
            kv.kv_cache_write_dynamic(d, k, v, slots, kc, vc, ks, vs)
        else:
            ks = torch.empty(Hkv, dtype=torch.float32, device=dev)
            vs = torch.empty(Hkv, dtype=torch.float32, device=dev)
            kv.kv_scale_from_amax(d, k, ks)
            kv.kv_scale_from_amax(d, v, vs)
            kv.kv_cache_write(d, k, v, slots, kc, vc, ks, vs)
        ws = kv.alloc_prefill_workspace(d, 1, chunk, pages)
        flops = 4.0 * D * Hq * (chunk * L - chunk * (chunk - 1) / 2)
        res = dict(chunk=chunk, context=L, workspace_bytes=0 if ws is None else ws.numel())
        for tag, wsp in (("split", ws), ("no_split", None)):
            def attend():
                kv.paged_prefill_attention(d, out, q, kc, vc, bt, qs, lens, chunk, ks, vs,
                                           workspace=wsp)
            for _ in range(warmup):
                attend()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                attend()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            res[tag + "_us"] = round(us, 2)
            res[tag + "_tflops"] = round(flops / (us * 1e-6) / 1e12, 1)
        rows.append(res)
        log(f"chunked prefill chunk={chunk:5d} ctx={L:6d}: split {res['split_us']:9.1f} us "
            f"({res['split_tflops']:6.1f} TFLOP/s), no split {res['no_split_us']:9.1f} us "
            f"({res['no_split_tflops']:6.1f} TFLOP/s)")
        del kc, vc, k, v, q, out, ws
        torch.cuda.empty_cache()
    return dict(points=rows, cache="fp8_e4m3", scales=scales, attention=attn)


def prefill_bench(torch, kv, w, lengths, steps, warmup, scales="per_kv_head", attn="bf16"):
    """Single-request prefill per layer (the TTFT share of one layer): the
    cache write of a whole prompt of L tokens, then chunked-prefill attention
    of all L rows over it, for fp8 and bf16 caches; fits TTFT_layer = a L^2 +
    b L + c (the post's single-request TTFT model) and reports the prefill
    kernel's MFMA roofline at the longest prompt."""
    import numpy as np
    dev = torch.device("cuda:0")
    B, Hq, Hkv, D = 1, w["Hq"], w["Hkv"], w["D"]
    rows = []
    for dt in ("fp8_e4m3", "bf16"):
        d = kv.layer_desc(Hq, Hkv, D, dt, scales if dt != "bf16" else "per_kv_head",
                          attn=attn if dt != "bf16" else "bf16")
        for L in lengths:
            gen = torch.Generator(device=dev)
            gen.manual_seed(L)
            pages = (L + 15) // 16
            kc = torch.empty(kv.cache_shape(d, pages), dtype=torch.uint8, device=dev)
            vc = torch.empty_like(kc)
            k = torch.randn((L, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
            v = torch.randn((L, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
            q = torch.randn((L, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
            out = torch.empty((L, Hq, D), dtype=torch.bfloat16, device=dev)
            slots = torch.arange(L, dtype=torch.int64, device=dev)
            bt = torch.arange(pages, dtype=torch.int32, device=dev).view(1, pages)
            qs = torch.tensor([0, L], dtype=torch.int32, device=dev)
            lens = torch.tensor([L], dtype=torch.int32, device=dev)
            ks = vs = None
            if d.dynamic:   # per-token scales: pools, set by the (timed) write
                ks = torch.zeros(kv.scale_pool_shape(d, pages), dtype=torch.float32, device=dev)
                vs = torch.zeros_like(ks)
            elif d.fp8:     # static calibration, untimed
                ks = torch.empty(Hkv, dtype=torch.float32, device=dev)
                vs = torch.empty(Hkv, dtype=torch.float32, device=dev)
                kv.kv_scale_from_amax(d, k, ks)
                kv.kv_scale_from_amax(d, v, vs)

            def write():
                if d.dynamic:
                    kv.kv_cache_write_dynamic(d, k, v, slots, kc, vc, ks, vs)
                else:
                    kv.kv_cache_write(d, k, v, slots, kc, vc, ks, vs)

            def attend():
                kv.paged_prefill_attention(d, out, q, kc, vc, bt, qs, lens, L, ks, vs)

            def timed(fn):
                for _ in range(warmup):
                    fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(steps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) / steps

            wms = timed(write)
            ams = timed(attend)
            flops = 4.0 * D * Hq * L * (L + 1) / 2          # q k^T and P v over the causal pairs
            tfs = flops / (ams * 1e-3) / 1e12
            rows.append(dict(cache=dt, prompt=L, write_us=round(wms * 1e3, 2),
                             attention_us=round(ams * 1e3, 2),
                             layer_us=round((wms + ams) * 1e3, 2), attention_tflops=round(tfs, 1),
                             frac_mfma_bf16=round(tfs / MFMA_BF16_PEAK_TFLOPS, 4)))
            log(f"prefill {dt:8s} L={L:6d} write {wms * 1e3:9.1f} us attention {ams * 1e3:10.1f} us "
                f"({tfs:6.1f} TFLOP/s)")
            del kc, vc, k, v, q, out
            torch.cuda.empty_cache()
    fits = {}
    for dt in ("fp8_e4m3", "bf16"):
        pts = [r for r in rows if r["cache"] == dt]
        x = np.array([r["prompt"] for r in pts], np.float64)
        y = np.array([r["layer_us"] for r in pts], np.float64)
        a, b_, c_ = np.polyfit(x, y, 2)
        fits[dt] = dict(a_us_per_token2=a, b_us_per_token=b_, c_us=c_)
    top = [r for r in rows if r["prompt"] == max(lengths)]
    fp8_top = [r for r in top if r["cache"] == "fp8_e4m3"][0]
    return dict(points=rows, fits=fits, scales=scales, attention=attn,
                quadratic_ratio_fp8_over_bf16=fits["fp8_e4m3"]["a_us_per_token2"] /
                fits["bf16"]["a_us_per_token2"],
                roofline={"bound": "mfma", "kernel": "paged_prefill_kernel (fp8 cache)",
                          "achieved": fp8_top["attention_tflops"],
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": fp8_top["frac_mfma_bf16"], "prompt": max(lengths),
                          "algorithmic_flops": 4 * D * Hq * max(lengths) * (max(lengths) + 1) // 2})


def stack_point(torch, kv, stack, steps, warmup):
    """One layer stack: graph-timed µs per layer step, the split kernel's
    mean launch time (kernel-timestamped events over eager steps), the same
    bytes read by a plain streaming read, and the ratios."""
    ms = time_steps_graph(torch, stack, steps, warmup)
    _, split_ms, _ = time_steps(torch, kv, stack, 3, 1)
    NL = stack.NL
    d0 = stack.layers[0]["desc"]
    split_bytes = stack.split_bytes(d0) + stack.write_bytes(d0)
    us = ms * 1e3 / NL
    step_gbs = stack.total_step_bytes() / (ms * 1e-3) / 1e9
    split_us = split_ms * 1e3 if split_ms else None
    return dict(layers=NL, us_per_layer_step=round(us, 3), step_gbs=round(step_gbs, 1),
                step_frac_hbm=round(step_gbs / HBM_PEAK_GBS, 4),
                split_us=round(split_us, 3) if split_us else None,
                split_gbs=round(split_bytes / (split_us * 1e-6) / 1e9, 1) if split_us else None,
                split_frac_hbm=round(split_bytes / (split_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                if split_us else None,
                split_bytes=split_bytes), split_bytes


def other_workloads(torch, kv, steps, warmup):
    """The other decode workloads, each as a graph-timed layer stack of at
    least 2 GiB of cache: the batched step (8 sequences of 18k-22k positions,
    shuffled pool, each step writing 8 new tokens), the 70B layer at 131072
    positions, the head_dim 256 layer at 65536, and the gpt-oss-like layer
    types at 32768 (full-attention fp8 layers; window-128 bf16 skip
    layers). Each point carries the split kernel's time against a plain
    read of the same bytes (same_size_read_us)."""
    import synth
    out = {}
    W = WORKLOADS
    cfgs = [
        ("batched_8x18k-22k", W["batched"], [int(x) for x in synth.batched_lens()],
         dict(shuffle=True, spare_frac=0.1)),
        ("llama70b_131072", W["llama70b"], [131072], {}),
        ("hd256_65536", W["hd256"], [65536], {}),
        ("gptoss_full_fp8_32768", W["gptoss"], [32768], {}),
    ]
    for name, w, lens, kw in cfgs:
        per_layer = sum(lens) * w["Hkv"] * w["D"] * 2
        NL = layers_for(per_layer, hi=64)
        st = LayerStack(kv, torch, len(lens), w["Hq"], w["Hkv"], w["D"], lens, NL, seed=11,
                        **kw)
        pt, sb = stack_point(torch, kv, st, steps, warmup)
        del st
        torch.cuda.empty_cache()
        rd = same_size_read_us(torch, kv, sb)
        rk = same_size_read_kernel_us(torch, kv, sb)
        pt["same_size_read_us"] = round(rd, 3)
        pt["step_over_same_size_read"] = round(pt["us_per_layer_step"] / rd, 4)
        pt["same_size_read_kernel_us"] = round(rk, 3) if rk else None
        pt["split_over_same_size_read_kernel"] = (round(pt["split_us"] / rk, 4)
                                                  if pt["split_us"] and rk else None)
        pt["shape"] = dict(batch=len(lens), q_heads=w["Hq"], kv_heads=w["Hkv"], head_dim=w["D"],
                           contexts=f"{min(lens)}..{max(lens)}" if len(lens) > 1 else lens[0])
        log(f"workload {name}: {pt['us_per_layer_step']:.2f} us/layer step "
            f"({pt['step_frac_hbm'] * 100:.1f} % of peak), split {pt['split_us']} us, "
            f"read {rd:.2f} us (graph) {rk} us (kernel events)")
        out[name] = pt
    # the gpt-oss window layers: window 128, bf16 cache (the skip path)
    w = W["gptoss"]
    st = LayerStack(kv, torch, 1, w["Hq"], w["Hkv"], w["D"], [32768], 32, "bf16", window=128,
                    seed=12)
    ms = time_steps_graph(torch, st, steps, warmup)
    out["gptoss_window128_bf16_32768"] = dict(
        layers=32, us_per_layer_step=round(ms * 1e3 / 32, 3),
        note="reads the last 128 positions: launch-bound (its caches stay in the Infinity Cache)")
    del st
    torch.cuda.empty_cache()
    return out


def quantisation_error(torch, kv):
    """Error of fp8 attention (per-KV-head scales, amax/448) against
    unquantised bf16 attention on the same inputs: the 8B layer (normal
    values) and the 70B layer (drifting V with heavy-tail rows) at 131072
    positions, drawn by synth. The unquantised reference is the library's
    bf16-cache path on the same bf16 K/V and q, which the full-size parity
    tests hold within 3e-6 of the float64 oracle."""
    import numpy as np
    import synth
    dev = torch.device("cuda:0")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
            torch.bfloat16)

    res = {}
    for name, wl, Hq, values in (("llama8b_131072", synth.LLAMA8B, 32, "normal"),
                                 ("llama70b_131072", synth.LLAMA70B, 64, "drift")):
        case = synth.decode_case(wl, Hq, 8, 128, [131072], values=values)
        k, v, q = bf16(case.k_new), bf16(case.v_new), bf16(case.q)
        slots = torch.from_numpy(case.slots).to(dev)
        bt = torch.from_numpy(case.block_tables).to(dev)
        lens = torch.from_numpy(case.lens).to(dev)
        outs = {}
        for dt in ("fp8_e4m3", "bf16"):
            d = kv.layer_desc(Hq, 8, 128, dt, "per_kv_head")
            kc = torch.empty(kv.cache_shape(d, case.num_pages), dtype=torch.uint8, device=dev)
            vc = torch.empty_like(kc)
            ks = vs = None
            if d.fp8:
                ks = torch.empty(8, dtype=torch.float32, device=dev)
                vs = torch.empty(8, dtype=torch.float32, device=dev)
                kv.kv_scale_from_amax(d, k, ks)
                kv.kv_scale_from_amax(d, v, vs)
            kv.kv_cache_write(d, k, v, slots, kc, vc, ks, vs)
            o = torch.empty((1, Hq, 128), dtype=torch.float32, device=dev)
            kv.paged_decode_attention(d, o, q, kc, vc, bt, lens, 131072, ks, vs,
                                      kv.alloc_workspace(d, 1, 131072))
            torch.cuda.synchronize()
            outs[dt] = o.double()
            del kc, vc
        diff = (outs["fp8_e4m3"] - outs["bf16"]).abs()
        res[name] = dict(max_abs=float(diff.max()), mean_abs=float(diff.mean()),
                         output_max_abs=float(outs["bf16"].abs().max()))
        log(f"quantisation error {name}: max {res[name]['max_abs']:.3e} "
            f"mean {res[name]['mean_abs']:.3e}")
        del k, v, q, outs
        torch.cuda.empty_cache()
    res["how"] = ("fp8 e4m3 cache with per-KV-head scales amax/448 against the bf16 cache on "
                  "the same inputs (synth workloads llama8b and llama70b-drift); reported, "
                  "not gated")
    return res


def cpu_baseline(w, ctx, min_seconds=10.0):
    """The float64 oracle on the headline layer (all heads, full context),
    repeated until at least min_seconds of wall time."""
    import numpy as np
    import oracle
    import synth
    threads = min(16, os.cpu_count() or 1)
    os.environ["ORACLE_THREADS"] = str(threads)
    case = synth.decode_case(synth.LLAMA8B, w["Hq"], w["Hkv"], w["D"], [ctx])
    kc = synth.poisoned_cache(case.num_pages, w["Hkv"], w["D"], True)
    vc = kc.copy()
    ks = oracle.scale_from_amax(case.k_new, True)
    vs = oracle.scale_from_amax(case.v_new, True)
    oracle.kv_cache_write(kc, vc, case.k_new, case.v_new, case.slots, oracle.FP8, True, ks, vs)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(case.q, kc, vc, case.block_tables, case.lens, w["Hkv"], oracle.FP8,
                         True, 0, 0.0, ks, vs)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 50:
            break
    kv_bytes = ctx * w["Hkv"] * w["D"] * 2
    gbs = kv_bytes * reps / el / 1e9
    host = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            host = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return dict(value=round(gbs, 4), unit="GB/s", cores=threads, kind="oracle",
                host_cpu=f"{host}, {os.cpu_count()} logical CPUs visible",
                sample=f"{w['desc']}, context {ctx}, fp8 per-KV-head, all {w['Hq']} query "
                       f"heads, attention only, {reps} repetitions in {el:.1f} s "
                       f"({el / reps * 1e3:.0f} ms per layer step)")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b", choices=sorted(WORKLOADS))
    ap.add_argument("--context", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--cache", default="fp8_e4m3", choices=["fp8_e4m3", "fp8_e5m2", "bf16"])
    ap.add_argument("--attn", default="bf16", choices=["bf16", "fp8"],
                    help="attention arithmetic: bf16 MFMA on exact cache codes, or the "
                         "all-FP8 mode (e4m3 q and P, fp8 MFMA)")
    ap.add_argument("--scales", default="per_kv_head",
                    choices=["per_kv_head", "per_tensor", "per_token", "per_token_head"],
                    help="static scales (per KV head, per tensor) or dynamic per-token scales "
                         "(stored per slot beside the pages)")
    ap.add_argument("--path", default="fused", choices=["fused", "separate"],
                    help="fused: kvq_decode_step per layer; separate: write + attention calls")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the single-request prefill (TTFT) sweep")
    ap.add_argument("--prefill-only", action="store_true",
                    help="print the prefill sweep only (no decode headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other decode workloads (batched, 70B, head_dim 256, "
                         "gpt-oss layer types) and the quantisation-error report")
    ap.add_argument("--sweep-steps", type=int, default=10)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (for scaling PMC byte counters)")
    ap.add_argument("--trace-server", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-kernel-trace", action="store_true",
                    help="skip the rocprofv3 kernel-trace comparison of the split kernel with a "
                         "plain read (child processes, about a minute)")
    ap.add_argument("--trace-point", action="store_true",
                    help="for a kernel trace: 20 graph-replayed decode steps of --workload at "
                         "--context (all layers of the workload's cache type), then plain "
                         "streaming reads of the split kernel's bytes per launch (1024 and "
                         "4096 work-groups, no events), so the profiler times both kernels "
                         "the same way")
    args = ap.parse_args()

    if args.trace_server:
        trace_server()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each sequence and KV head is independent; sharding is the caller's). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    # the profiler's child processes start from a process that has not
    # touched the GPU: the trace server, started first
    tracer = None
    if (args.workload == "llama8b" and not args.no_sweep and not args.no_kernel_trace
            and not args.prefill_only and not args.trace_point and not args.copy_calibration):
        tracer = start_trace_server()

    import torch
    import fp8_kv_cache_write_amd as kv
    if not os.path.exists(kv.LIB_PATH):
        from fp8_kv_cache_write_amd import build
        build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        src = torch.empty(GIB, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(copy_bytes=GIB, launches=3)))
        return

    w = WORKLOADS[args.workload]
    if args.trace_point:
        ctx = args.context or w["ctx"]
        if not ctx:
            print("--trace-point needs --context for this workload", file=sys.stderr)
            sys.exit(2)
        NL = args.layers or layers_for(ctx * w["Hkv"] * w["D"] * 2, hi=64)
        stack = LayerStack(kv, torch, 1, w["Hq"], w["Hkv"], w["D"], [ctx], NL, args.cache,
                           seed=ctx, attn=args.attn, scales=args.scales)
        ms = time_steps_graph(torch, stack, 20, 3)
        nb = stack.split_bytes(stack.descs[0]) // 16 * 16
        del stack
        torch.cuda.empty_cache()
        n = max(8, min(256, math.ceil(2 * GIB / nb)))
        bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1) for _ in range(n)]
        for blocks in (1024, 4096):
            sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
            for _ in range(4):
                for b in bufs:
                    kv.stream_read(b, sink)
        torch.cuda.synchronize()
        print(json.dumps(dict(workload=args.workload, context=ctx, layers=NL,
                              us_per_layer_step_graph=round(ms * 1e3 / NL, 3),
                              read_bytes_per_launch=nb, read_buffers=n)))
        return
    if args.prefill_only:
        # the 8B layer by default; --workload picks another layer shape
        # (hd256: the head_dim-256 prefill the vLLM post finds slower in fp8)
        res = prefill_bench(torch, kv, w, PREFILL_LENGTHS, 5, 2, scales=args.scales,
                            attn=args.attn)
        res["workload"] = args.workload
        res["chunked"] = chunked_prefill_bench(torch, kv, w, CHUNKED_PREFILL, 5, 2,
                                               scales=args.scales, attn=args.attn)
        print(json.dumps(res))
        return
    ctx = args.context or w["ctx"]
    NL = args.layers or w["layers"]
    torch.manual_seed(0)

    # ---- headline --------------------------------------------------------
    if args.workload == "batched":
        import synth
        lens = [int(x) for x in synth.batched_lens()]
        stack = LayerStack(kv, torch, w["B"], w["Hq"], w["Hkv"], w["D"], lens, NL, args.cache,
                           shuffle=True, spare_frac=0.1, seed=3, path=args.path, attn=args.attn,
                           scales=args.scales)
        ctx_desc = f"lengths {min(lens)}..{max(lens)} (sum {sum(lens)})"
    elif args.workload == "gptoss":
        dts = ["fp8_e4m3" if i % 2 == 0 else "bf16" for i in range(NL)]
        wins = [0 if i % 2 == 0 else 128 for i in range(NL)]
        stack = LayerStack(kv, torch, 1, w["Hq"], w["Hkv"], w["D"], [ctx], NL, seed=5,
                           dtypes=dts, window=wins, path=args.path, attn=args.attn,
                           scales=args.scales)
        ctx_desc = f"context {ctx}; {NL // 2} full fp8 layers + {NL - NL // 2} SW-128 bf16 layers"
    else:
        stack = LayerStack(kv, torch, w["B"], w["Hq"], w["Hkv"], w["D"], [ctx], NL, args.cache,
                           seed=1, path=args.path, attn=args.attn, scales=args.scales)
        ctx_desc = f"context {ctx}"
    log(f"headline: {w['desc']}, {ctx_desc}, {NL} layers, cache {args.cache}, attention "
        f"{args.attn}, scales {args.scales}")
    # the timed region: K steps, each one replay of the captured decode step
    ms, per_step = time_steps_graph(torch, stack, args.steps, args.warmup, per_step=True)
    # eager steps with the split kernel's launches timed by the library
    ms_eager, split_ms, nsplit = time_steps(torch, kv, stack, args.steps, args.warmup)
    roof_kernel = "paged_decode_split_kernel"
    if args.workload == "gptoss":
        # the hybrid's split launches mix full and windowed layers: the
        # roofline is that of the full-attention fp8 layers, timed alone
        full = LayerStack(kv, torch, 1, w["Hq"], w["Hkv"], w["D"], [ctx], max(NL // 2, 1),
                          seed=5, path=args.path, attn=args.attn, scales=args.scales)
        _, split_ms, nsplit = time_steps(torch, kv, full, args.steps, args.warmup)
        del full
        torch.cuda.empty_cache()
        roof_kernel = "paged_decode_split_kernel (the full-attention fp8 layers, timed alone)"
    # the other path, for comparison (graph-replayed too)
    other = "separate" if args.path == "fused" else "fused"
    stack.path = other
    ms_other = time_steps_graph(torch, stack, args.steps, args.warmup)
    stack.path = args.path
    step_bytes = stack.total_step_bytes()
    value = step_bytes / (ms * 1e-3) / 1e9
    kv_gbs = stack.total_kv_bytes() / (ms * 1e-3) / 1e9
    d0 = stack.layers[0]["desc"]
    split_bytes = stack.split_bytes(d0) + (stack.write_bytes(d0) if args.path == "fused" else 0)
    achieved = split_bytes / (split_ms * 1e-3) / 1e9 if split_ms else None
    log(f"headline ({args.path}): {ms:.3f} ms/step (graph; eager {ms_eager:.3f}; {other} path "
        f"{ms_other:.3f}), {ms * 1e3 / NL:.2f} us/layer, {value:.1f} GB/s "
        f"(KV {kv_gbs:.1f} GB/s), split kernel {split_ms * 1e3 if split_ms else 0:.2f} us "
        f"-> {achieved or 0:.1f} GB/s")

    result = {
        "metric": "decode-attn µs/step & KV GB/s (% HBM peak) vs context; fp8/bf16 slope",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ((f"{args.cache} cache, e4m3 q and P on fp8 MFMA, fp32 accumulation"
                   if args.attn == "fp8" else
                   f"{args.cache} cache, bf16 MFMA on exact {args.cache[4:]} values, "
                   "fp32 accumulation") if args.cache.startswith("fp8")
                  else "bf16 cache, fp32 accumulation"),
        "data": "synthetic (seeded normal K/V/q)",
        "config": {
            "workload": f"{w['desc']}, {ctx_desc}, {args.cache} cache with "
                        f"{SCALE_TEXT[args.scales]}, "
                        f"{NL} layers per step (per layer: the new token's cache write + paged "
                        f"decode attention, " + ("one kvq_decode_step call" if args.path == "fused"
                        else "kvq_kv_cache_write + kvq_paged_decode_attention") + ")",
            "path": args.path,
            "attention": args.attn,
            "scales": args.scales,
            "batch": w["B"], "q_heads": w["Hq"], "kv_heads": w["Hkv"], "head_dim": w["D"],
            "page_size": 16, "layers_per_step": NL, "parallelism": "single GPU",
        },
        "timing": "each step is one replay of the decode step captured as a HIP graph",
        "ms_per_step_eager": round(ms_eager, 5),
        f"ms_per_step_{other}_path": round(ms_other, 5),
        "us_per_layer_step": round(ms * 1e3 / NL, 3),
        "us_per_layer_step_p10_p50_p90": [round(percentile(per_step, q) * 1e3 / NL, 3)
                                          for q in (0.1, 0.5, 0.9)],
        "kv_gbs": round(kv_gbs, 2),
        "kv_frac_of_hbm_peak": round(kv_gbs / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": roof_kernel,
            "achieved": round(achieved, 1) if achieved else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
            "traffic": measured_traffic(f"{args.workload}:{ctx}:{args.cache}:{NL}:{args.path}")
            if args.workload == "llama8b" and args.attn == "bf16" and args.scales == "per_kv_head"
            else None,
            "launch_us": round(split_ms * 1e3, 3) if split_ms else None,
            "launches_timed": nsplit,
            "timed_with": "kernel-timestamped HIP event pairs around every split-kernel launch "
                          "of a pass of eager steps enqueued behind a GPU head start "
                          "(kvq_profile_begin/end)",
            "algorithmic_bytes_per_launch": split_bytes,
        },
    }
    del stack
    torch.cuda.empty_cache()
    ceiling, copy_gbs = read_ceiling_gbs(torch, kv)
    result["measured_ceilings"] = {
        "read_gbs": round(ceiling, 1),
        "read_how": "kvq_stream_read over 4 GiB: every byte once, 16-byte non-temporal loads, "
                    "best of 1024-8192 work-groups",
        "copy_gbs": round(copy_gbs, 1), "copy_how": "torch copy_ of 4 GiB, read + write bytes",
        "split_kernel_frac_of_read": round(achieved / ceiling, 4) if achieved else None,
        "step_frac_of_read": round(value / ceiling, 4),
        "step_frac_of_copy": round(value / copy_gbs, 4)}
    # the same read, one launch per layer's split bytes, graph-replayed: the
    # time a kernel with no attention work needs for this layer's bytes
    rd_us = same_size_read_us(torch, kv, split_bytes)
    rk_us = same_size_read_kernel_us(torch, kv, split_bytes)
    result["measured_ceilings"]["same_size_read_us"] = round(rd_us, 3)
    result["measured_ceilings"]["step_over_same_size_read"] = round(ms * 1e3 / NL / rd_us, 4)
    result["measured_ceilings"]["same_size_read_kernel_us"] = round(rk_us, 3) if rk_us else None
    result["measured_ceilings"]["split_kernel_over_same_size_read_kernel"] = (
        round(split_ms * 1e3 / rk_us, 4) if split_ms and rk_us else None)
    result["measured_ceilings"]["same_size_read_how"] = (
        "kvq_stream_read of the split kernel's bytes per launch over distinct buffers: "
        "same_size_read_us is the graph-replayed time per launch (compare with the step), "
        "same_size_read_kernel_us the kernel-event time (timed as the split kernel is)")

    if not args.no_sweep and args.workload == "llama8b":
        contexts = [16, 256, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 98304, 131072]
        result["sweep"] = sweep(torch, kv, w, contexts, args.sweep_steps, 2)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["long_contexts"] = long_contexts(torch, kv, w, [262144, 524288, 1048576],
                                                args.sweep_steps, 2)
        result["split_vs_read_kernel_trace"] = kernel_trace_ratios(tracer)
    stop_trace_server(tracer)
    if not args.no_workloads and args.workload == "llama8b":
        result["workloads"] = other_workloads(torch, kv, args.sweep_steps, 2)
        result["quantisation_error_vs_bf16"] = quantisation_error(torch, kv)
    if not args.no_sweep and args.workload == "gptoss":
        result["gptoss_sweep"] = gptoss_sweep(torch, kv, w, [8192, 32768, 65536, 131072],
                                              args.sweep_steps, 2)
    if not args.no_prefill and args.workload == "llama8b":
        result["prefill"] = prefill_bench(torch, kv, w, PREFILL_LENGTHS, 5, 2)
        result["chunked_prefill"] = chunked_prefill_bench(torch, kv, w, CHUNKED_PREFILL, 5, 2)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)...")
        result["cpu_baseline"] = cpu_baseline(WORKLOADS["llama8b"], 131072)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
