"""Helpers shared by the GPU parity tests: run one decode layer through the
HIP library (C ABI via the Python binding) and through the oracle on the same
seeded inputs."""

import numpy as np
import torch

import fp8_kv_cache_write_amd as kv
import oracle
import synth

FP8, BF16, E5M2 = oracle.FP8, oracle.BF16, oracle.E5M2
_ORACLE_FMT = {"fp8_e4m3": FP8, "fp8_e5m2": E5M2, "bf16": BF16}


def cache_fmt(fp8, fmt):
    """The cache dtype name: fmt if given, else e4m3 (fp8) or bf16."""
    return fmt if fmt is not None else ("fp8_e4m3" if fp8 else "bf16")
GATE_MAX_ABS = 1e-2      # attention gate (max-abs, unit-scale inputs)
GATE_MEAN_ABS = 1e-3     # attention gate (mean-abs)
# All-FP8 arithmetic: one flip (a probability rounded to the neighbouring
# e4m3 code) moves only its own (row, q head) pair, by up to an eighth of
# |v_j - o| there. With few pairs over few positions one flip alone can lift
# the mean above the gate (8 pairs over 8-9 positions: one step of a
# probability near 0.53 moved its pair by up to 0.058, the case's mean to 1.24
# of the gate); from this many pairs on, one such flip (that pair's mean
# error was 0.017) adds under a third of the gate, and the mean gate applies.
FLIP_DILUTION_PAIRS = 64


def dev():
    return torch.device("cuda:0")


def bf16_dev(bits):
    """uint16 bf16 bit patterns -> bf16 device tensor (same bits)."""
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).to(dev()).view(torch.bfloat16)


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def i64_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(dev())


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def host(t):
    return t.detach().cpu().numpy()


# ---- guard bands ------------------------------------------------------------
# Every device buffer the library writes in these helpers (caches, scale
# pools, outputs, workspaces) sits inside a larger allocation whose first and
# last GUARD bytes hold a fixed pattern; check_guards() after each call
# confirms that no kernel wrote outside its buffer.
GUARD = 4096
GUARD_BYTE = 0xA5


def guarded(shape, dtype, fill=None, registry=None):
    """A device tensor of shape/dtype inside a guarded allocation (the
    buffer itself 256-byte aligned, as the workspaces need); fill: a value,
    a host numpy array of the same bytes, or None (left uninitialised). The
    allocation and the buffer's size go into registry (a list) for
    check_guards."""
    elem = torch.empty((), dtype=dtype).element_size()
    n = 1
    for x in shape:
        n *= int(x)
    nbytes = n * elem
    big = torch.full((GUARD + nbytes + GUARD,), GUARD_BYTE, dtype=torch.uint8, device=dev())
    inner = big[GUARD:GUARD + nbytes].view(dtype).view(*shape)
    if isinstance(fill, np.ndarray):
        inner.view(torch.uint8).view(-1).copy_(
            torch.from_numpy(np.ascontiguousarray(fill).view(np.uint8).reshape(-1)).to(dev()))
    elif fill is not None:
        inner.fill_(fill)
    if registry is not None:
        registry.append((big, nbytes))
    return inner


def check_guards(registry, label=""):
    """Every guard band of the registered allocations still holds its
    pattern."""
    torch.cuda.synchronize()
    for big, nbytes in registry:
        ok = bool((big[:GUARD] == GUARD_BYTE).all()) and \
            bool((big[GUARD + nbytes:] == GUARD_BYTE).all())
        assert ok, f"{label}: a kernel wrote outside a buffer of {nbytes} bytes"


class GpuLayer:
    """One layer on the GPU: poisoned caches, scales calibrated by the
    library, every position of the case written by the library. dyn:
    "per_token" / "per_token_head" for dynamic scales (pools start as NaN,
    so a read of an unwritten slot's scale would show)."""

    def __init__(self, case, fp8=True, per_head=True, window=0, sm_scale=0.0,
                 scales=None, fmt=None, attn="bf16", dyn=None):
        self.case = case
        fmt = cache_fmt(fp8, fmt)
        self.fp8 = fp8 = fmt != "bf16"
        mode = dyn if dyn else ("per_kv_head" if per_head else "per_tensor")
        self.desc = kv.layer_desc(case.num_q_heads, case.num_kv_heads, case.head_dim, fmt,
                                  mode, window, sm_scale, attn)
        self.dyn = bool(dyn) and fp8
        self.k_new = bf16_dev(case.k_new)
        self.v_new = bf16_dev(case.v_new)
        self.slots = i64_dev(case.slots)
        pc = synth.poisoned_cache(case.num_pages, case.num_kv_heads, case.head_dim, fp8)
        self.guards = []                       # the caches' and scales' guard bands
        self.k_cache = guarded(pc.shape, torch.uint8, pc, self.guards)
        self.v_cache = guarded(pc.shape, torch.uint8, pc, self.guards)
        n = case.num_kv_heads if per_head else 1
        if self.dyn:
            shape = kv.scale_pool_shape(self.desc, case.num_pages)
            self.k_scale = guarded(shape, torch.float32, float("nan"), self.guards)
            self.v_scale = guarded(shape, torch.float32, float("nan"), self.guards)
        elif fp8:
            if scales is None:
                self.k_scale = guarded((n,), torch.float32, None, self.guards)
                self.v_scale = guarded((n,), torch.float32, None, self.guards)
                kv.kv_scale_from_amax(self.desc, self.k_new, self.k_scale)
                kv.kv_scale_from_amax(self.desc, self.v_new, self.v_scale)
            else:
                self.k_scale = torch.tensor(scales[0], dtype=torch.float32, device=dev())
                self.v_scale = torch.tensor(scales[1], dtype=torch.float32, device=dev())
        else:
            self.k_scale = self.v_scale = None
        if self.dyn:
            kv.kv_cache_write_dynamic(self.desc, self.k_new, self.v_new, self.slots,
                                      self.k_cache, self.v_cache, self.k_scale, self.v_scale)
        else:
            kv.kv_cache_write(self.desc, self.k_new, self.v_new, self.slots, self.k_cache,
                              self.v_cache, self.k_scale, self.v_scale)
        check_guards(self.guards, "cache write")
        self.q = bf16_dev(case.q)
        self.block_tables = i32_dev(case.block_tables)
        self.context_lens = i32_dev(case.lens)

    def attend(self, out_dtype=torch.float32, block_tables=None, q=None):
        c = self.case
        reg = list(self.guards)
        out = guarded((c.num_seqs, c.num_q_heads, c.head_dim), out_dtype, None, reg)
        n = kv.decode_workspace_bytes(self.desc, c.num_seqs, c.max_context_len)
        ws = guarded((n,), torch.uint8, None, reg) if n else None
        kv.paged_decode_attention(self.desc, out, self.q if q is None else q,
                                  self.k_cache, self.v_cache,
                                  self.block_tables if block_tables is None else block_tables,
                                  self.context_lens, c.max_context_len, self.k_scale,
                                  self.v_scale, ws)
        check_guards(reg, "decode attention")
        return out

    def scales_host(self):
        if not self.fp8:
            return None, None
        return host(self.k_scale), host(self.v_scale)


class OracleLayer:
    """The same layer through the oracle (its own scales, its own caches)."""

    def __init__(self, case, fp8=True, per_head=True, window=0, sm_scale=0.0,
                 scales=None, fmt=None, attn="bf16", dyn=None):
        fmt = cache_fmt(fp8, fmt)
        self.fmt = _ORACLE_FMT[fmt]
        self.attn = attn
        fp8 = fmt != "bf16"
        self.dyn = bool(dyn) and fp8
        if self.dyn:
            per_head = {"per_token": oracle.PER_TOKEN,
                        "per_token_head": oracle.PER_TOKEN_HEAD}[dyn]
        self.case, self.fp8, self.per_head = case, fp8, per_head
        self.window, self.sm_scale = window, sm_scale
        self.k_cache = synth.poisoned_cache(case.num_pages, case.num_kv_heads,
                                            case.head_dim, fp8)
        self.v_cache = self.k_cache.copy()
        if self.dyn:
            self.ks, self.vs = oracle.scale_pools(case.num_pages, case.num_kv_heads)
            self.ks[:] = np.nan
            self.vs[:] = np.nan
            oracle.kv_cache_write_dyn(self.k_cache, self.v_cache, case.k_new, case.v_new,
                                      case.slots, self.fmt, per_head, self.ks, self.vs)
            return
        if fp8:
            if scales is None:
                self.ks = oracle.scale_from_amax(case.k_new, per_head, fmt=self.fmt)
                self.vs = oracle.scale_from_amax(case.v_new, per_head, fmt=self.fmt)
            else:
                self.ks = np.asarray(scales[0], np.float32)
                self.vs = np.asarray(scales[1], np.float32)
        else:
            self.ks = self.vs = None
        oracle.kv_cache_write(self.k_cache, self.v_cache, case.k_new, case.v_new,
                              case.slots, self.fmt, per_head, self.ks, self.vs)

    def attend(self):
        c = self.case
        fn = oracle.attention_fp8attn if self.attn == "fp8" else oracle.attention
        return fn(c.q, self.k_cache, self.v_cache, c.block_tables, c.lens, c.num_kv_heads,
                  self.fmt, self.per_head, self.window, self.sm_scale, self.ks, self.vs)


def errors(gpu_out, ref):
    g = host(gpu_out.float()).astype(np.float64)
    d = np.abs(g - ref)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def unquantised_reference(case, window=0, sm_scale=0.0):
    """Attention over the bf16 inputs themselves (no quantisation): the
    reference for reporting the quantisation error."""
    o = OracleLayer(case, fp8=False, window=window, sm_scale=sm_scale)
    return o.attend()
