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
        self.k_cache = u8_dev(pc)
        self.v_cache = u8_dev(pc)
        n = case.num_kv_heads if per_head else 1
        if self.dyn:
            shape = kv.scale_pool_shape(self.desc, case.num_pages)
            self.k_scale = torch.full(shape, float("nan"), dtype=torch.float32, device=dev())
            self.v_scale = torch.full(shape, float("nan"), dtype=torch.float32, device=dev())
        elif fp8:
            if scales is None:
                self.k_scale = torch.empty(n, dtype=torch.float32, device=dev())
                self.v_scale = torch.empty(n, dtype=torch.float32, device=dev())
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
        self.q = bf16_dev(case.q)
        self.block_tables = i32_dev(case.block_tables)
        self.context_lens = i32_dev(case.lens)

    def attend(self, out_dtype=torch.float32, block_tables=None, q=None):
        c = self.case
        out = torch.empty((c.num_seqs, c.num_q_heads, c.head_dim), dtype=out_dtype,
                          device=dev())
        ws = kv.alloc_workspace(self.desc, c.num_seqs, c.max_context_len)
        kv.paged_decode_attention(self.desc, out, self.q if q is None else q,
                                  self.k_cache, self.v_cache,
                                  self.block_tables if block_tables is None else block_tables,
                                  self.context_lens, c.max_context_len, self.k_scale,
                                  self.v_scale, ws)
        torch.cuda.synchronize()
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
