"""Python binding of libkvfp8 (include/kvfp8.h): FP8 e4m3 paged KV-cache write
and GQA paged decode attention on MI355X (gfx950).

Argument marshalling only: every function checks that the tensors are what
the C ABI expects (device, dtype, contiguity, shape), passes their device
pointers and the current HIP stream, and raises Kvfp8Error on a non-zero
status. All computation runs in the library's HIP kernels; there is no
fallback. The library must have been built (``python -m
fp8_kv_cache_write_amd.build`` or ``__graft_entry__.build()``).
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvfp8.so")

# enums of kvfp8.h
BF16, FP8_E4M3, FP8_E5M2 = 0, 1, 2
PER_TENSOR, PER_KV_HEAD, PER_TOKEN, PER_TOKEN_HEAD = 0, 1, 2, 3
ATTN_BF16, ATTN_FP8 = 0, 1
OUT_F32, OUT_BF16 = 0, 1
PAGE_SIZE = 16

_DTYPES = {"bf16": BF16, "auto": BF16, "fp8": FP8_E4M3, "fp8_e4m3": FP8_E4M3,
           "fp8_e5m2": FP8_E5M2}
_SCALES = {"per_tensor": PER_TENSOR, "per_kv_head": PER_KV_HEAD, "per_token": PER_TOKEN,
           "per_token_head": PER_TOKEN_HEAD}
_ATTN = {"bf16": ATTN_BF16, "fp8": ATTN_FP8}


class Kvfp8Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} ({status})")


class LayerDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("cache_dtype", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
                ("sliding_window", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("attn_dtype", ctypes.c_int32)]

    @property
    def fp8(self):
        return self.cache_dtype in (FP8_E4M3, FP8_E5M2)

    @property
    def dynamic(self):
        """fp8 layer with per-token scales (pools written by the write)."""
        return self.fp8 and self.scale_mode in (PER_TOKEN, PER_TOKEN_HEAD)

    @property
    def elem_bytes(self):
        return 1 if self.fp8 else 2

    @property
    def page_bytes(self):
        """Bytes of one (page, kv head) block."""
        return PAGE_SIZE * self.head_dim * self.elem_bytes


def layer_desc(num_q_heads, num_kv_heads, head_dim, cache_dtype="fp8_e4m3",
               scale_mode="per_kv_head", sliding_window=0, sm_scale=0.0, attn="bf16"):
    """Descriptor of one attention layer. cache_dtype: "fp8_e4m3"/"fp8",
    "fp8_e5m2" or "bf16"/"auto"; scale_mode: "per_tensor", "per_kv_head"
    (static) or "per_token", "per_token_head" (dynamic, see scale_pool_shape);
    attn: "bf16" (exact cache codes, bf16 MFMA) or "fp8" (e4m3 q and P, fp8
    MFMA)."""
    return LayerDesc(int(num_q_heads), int(num_kv_heads), int(head_dim), PAGE_SIZE,
                     _DTYPES[cache_dtype] if isinstance(cache_dtype, str) else int(cache_dtype),
                     _SCALES[scale_mode] if isinstance(scale_mode, str) else int(scale_mode),
                     int(sliding_window), float(sm_scale),
                     _ATTN[attn] if isinstance(attn, str) else int(attn))


_lib = None


def lib():
    """The loaded libkvfp8.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m "
                "fp8_kv_cache_write_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        dp = ctypes.POINTER(LayerDesc)
        L.kvq_kv_cache_write.argtypes = [dp, vp, vp, vp, i64, vp, vp, i64, vp, vp, vp]
        L.kvq_decode_workspace_bytes.argtypes = [dp, i32, i32, ctypes.POINTER(sz)]
        L.kvq_paged_decode_attention.argtypes = [dp, vp, i32, vp, vp, vp, i64, vp, i32, vp,
                                                 i32, i32, vp, vp, vp, sz, vp]
        L.kvq_decode_step.argtypes = [dp, vp, vp, vp, vp, i64, vp, i32, vp, vp, i32, vp, i32,
                                      i32, vp, vp, vp, sz, vp]
        L.kvq_kv_cache_write_dynamic.argtypes = [dp, vp, vp, vp, i64, vp, vp, i64, vp, vp, vp]
        L.kvq_decode_step_dynamic.argtypes = [dp, vp, vp, vp, vp, i64, vp, i32, vp, vp, i32, vp,
                                              i32, i32, vp, vp, vp, sz, vp]
        L.kvq_paged_prefill_attention.argtypes = [dp, vp, i32, vp, vp, vp, i64, vp, i32, vp,
                                                  vp, i32, i32, vp, vp, vp, sz, vp]
        L.kvq_prefill_workspace_bytes.argtypes = [dp, i32, i32, i32, ctypes.POINTER(sz)]
        L.kvq_kv_scale_from_amax.argtypes = [dp, vp, i64, vp, vp]
        L.kvq_e4m3_quantize.argtypes = [vp, i64, vp, vp, vp]
        L.kvq_e5m2_quantize.argtypes = [vp, i64, vp, vp, vp]
        L.kvq_status_string.argtypes = [i32]
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_profile_begin.argtypes = [i32]
        L.kvq_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
        L.kvq_stream_read.argtypes = [vp, i64, vp, i32, vp]
        L.kvq_set_tuning.argtypes = [i32, i32]
        L.kvq_paged_decode_attention_noalloc.argtypes = [dp, vp, i32, vp, vp, vp, i64, vp, i32,
                                                         vp, i32, i32, vp, vp, vp]
        for f in ("kvq_kv_cache_write", "kvq_decode_workspace_bytes", "kvq_decode_step",
                  "kvq_paged_decode_attention", "kvq_kv_scale_from_amax",
                  "kvq_e4m3_quantize", "kvq_e5m2_quantize", "kvq_profile_begin",
                  "kvq_profile_end", "kvq_kv_cache_write_dynamic",
                  "kvq_decode_step_dynamic", "kvq_paged_prefill_attention",
                  "kvq_prefill_workspace_bytes", "kvq_stream_read", "kvq_set_tuning",
                  "kvq_paged_decode_attention_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status):
    return lib().kvq_status_string(int(status)).decode()


def _check(fn, status):
    if status != 0:
        raise Kvfp8Error(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype=None, device=True):
    import torch
    if t is None:
        return
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def cache_shape(desc, num_pages):
    """Shape of one K or V cache tensor (uint8): [num_pages, Hkv, page_bytes]."""
    return (int(num_pages), desc.num_kv_heads, desc.page_bytes)


def kv_cache_write(desc, k, v, slot_mapping, k_cache, v_cache, k_scale=None,
                   v_scale=None, stream=None):
    """Quantise (fp8) or copy (bf16) T new tokens into the paged caches.
    k, v: bf16 [T, Hkv, D]; slot_mapping: int64 [T]; caches: uint8
    [P, Hkv, page_bytes]; scales: float32 [1] or [Hkv] (fp8 layers)."""
    import torch
    _need(k, "k", torch.bfloat16)
    _need(v, "v", torch.bfloat16)
    _need(slot_mapping, "slot_mapping", torch.int64)
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache")
    _need(k_scale, "k_scale", torch.float32)
    _need(v_scale, "v_scale", torch.float32)
    T = k.shape[0]
    if tuple(k.shape) != (T, desc.num_kv_heads, desc.head_dim) or v.shape != k.shape:
        raise ValueError("k, v must be [T, Hkv, D]")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have T entries")
    num_pages = k_cache.numel() // (desc.num_kv_heads * desc.page_bytes) if k_cache.numel() else 0
    if k_cache.numel() * k_cache.element_size() != num_pages * desc.num_kv_heads * desc.page_bytes \
            or v_cache.numel() * v_cache.element_size() != k_cache.numel() * k_cache.element_size():
        raise ValueError("caches must be [P, Hkv, page_bytes] bytes")
    _check("kvq_kv_cache_write", lib().kvq_kv_cache_write(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache),
        _ptr(v_cache), num_pages, _ptr(k_scale), _ptr(v_scale), _stream(stream)))


def scale_pool_shape(desc, num_pages):
    """Shape of one K or V scale pool (float32) of a layer with dynamic
    scales: [num_pages, Hkv, 16], one scale per slot and KV head."""
    return (int(num_pages), desc.num_kv_heads, PAGE_SIZE)


def _check_pools(desc, k_cache, k_scales, v_scales):
    import torch
    _need(k_scales, "k_scales", torch.float32)
    _need(v_scales, "v_scales", torch.float32)
    if desc.dynamic:
        num_pages = k_cache.numel() * k_cache.element_size() // (desc.num_kv_heads *
                                                                 desc.page_bytes)
        for t in (k_scales, v_scales):
            if t is None or tuple(t.shape) != scale_pool_shape(desc, num_pages):
                raise ValueError("scale pools must be float32 [P, Hkv, 16]")


def kv_cache_write_dynamic(desc, k, v, slot_mapping, k_cache, v_cache, k_scales, v_scales,
                           stream=None):
    """kv_cache_write for a layer with dynamic per-token scales: each token's
    scales are computed from its values and stored into the pools
    (float32 [P, Hkv, 16]) at its slot."""
    import torch
    _need(k, "k", torch.bfloat16)
    _need(v, "v", torch.bfloat16)
    _need(slot_mapping, "slot_mapping", torch.int64)
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache")
    _check_pools(desc, k_cache, k_scales, v_scales)
    T = k.shape[0]
    if tuple(k.shape) != (T, desc.num_kv_heads, desc.head_dim) or v.shape != k.shape:
        raise ValueError("k, v must be [T, Hkv, D]")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have T entries")
    num_pages = k_cache.numel() * k_cache.element_size() // (desc.num_kv_heads * desc.page_bytes)
    _check("kvq_kv_cache_write_dynamic", lib().kvq_kv_cache_write_dynamic(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache),
        _ptr(v_cache), num_pages, _ptr(k_scales), _ptr(v_scales), _stream(stream)))


def decode_workspace_bytes(desc, num_seqs, max_context_len):
    n = ctypes.c_size_t(0)
    _check("kvq_decode_workspace_bytes", lib().kvq_decode_workspace_bytes(
        ctypes.byref(desc), int(num_seqs), int(max_context_len), ctypes.byref(n)))
    return int(n.value)


def alloc_workspace(desc, num_seqs, max_context_len, device="cuda"):
    """A uint8 device tensor big enough for one decode call (None if 0)."""
    import torch
    n = decode_workspace_bytes(desc, num_seqs, max_context_len)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def prefill_workspace_bytes(desc, num_seqs, max_query_len, max_pages_per_seq):
    n = ctypes.c_size_t(0)
    _check("kvq_prefill_workspace_bytes", lib().kvq_prefill_workspace_bytes(
        ctypes.byref(desc), int(num_seqs), int(max_query_len), int(max_pages_per_seq),
        ctypes.byref(n)))
    return int(n.value)


def alloc_prefill_workspace(desc, num_seqs, max_query_len, max_pages_per_seq, device="cuda"):
    """A uint8 device tensor for the key split of one prefill call (None when
    the plan has no split)."""
    import torch
    n = prefill_workspace_bytes(desc, num_seqs, max_query_len, max_pages_per_seq)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _decode_checks(desc, out, q, k_cache, v_cache, block_tables, context_lens, k_scale,
                   v_scale, workspace):
    import torch
    _need(out, "out")
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache")
    _need(block_tables, "block_tables", torch.int32)
    _need(context_lens, "context_lens", torch.int32)
    _need(k_scale, "k_scale", torch.float32)
    _need(v_scale, "v_scale", torch.float32)
    _need(workspace, "workspace")
    if out.dtype == torch.float32:
        out_dtype = OUT_F32
    elif out.dtype == torch.bfloat16:
        out_dtype = OUT_BF16
    else:
        raise ValueError("out must be float32 or bfloat16")
    B = q.shape[0]
    if tuple(q.shape) != (B, desc.num_q_heads, desc.head_dim) or out.shape != q.shape:
        raise ValueError("q, out must be [B, Hq, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables must be [B, max_pages], context_lens [B]")
    num_pages = k_cache.numel() * k_cache.element_size() // (desc.num_kv_heads * desc.page_bytes)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return out_dtype, num_pages, ws_bytes


def paged_decode_attention(desc, out, q, k_cache, v_cache, block_tables,
                           context_lens, max_context_len, k_scale=None,
                           v_scale=None, workspace=None, stream=None):
    """out: float32 or bf16 [B, Hq, D]; q: bf16 [B, Hq, D]; block_tables:
    int32 [B, max_pages]; context_lens: int32 [B]; max_context_len: host int
    bound of context_lens (sizes the split plan)."""
    out_dtype, num_pages, ws_bytes = _decode_checks(desc, out, q, k_cache, v_cache, block_tables,
                                                    context_lens, k_scale, v_scale, workspace)
    _check("kvq_paged_decode_attention", lib().kvq_paged_decode_attention(
        ctypes.byref(desc), _ptr(out), out_dtype, _ptr(q), _ptr(k_cache), _ptr(v_cache),
        num_pages, _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), q.shape[0],
        int(max_context_len), _ptr(k_scale), _ptr(v_scale), _ptr(workspace), ws_bytes,
        _stream(stream)))


# kvq_paged_decode_attention_noalloc's workspace (KVQ_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20


def paged_decode_attention_noalloc(desc, out, q, k_cache, v_cache, block_tables,
                                   context_lens, max_context_len, k_scale=None,
                                   v_scale=None, stream=None):
    """paged_decode_attention with the library's own device scratch array
    as the split workspace (no allocation; calls on one device must be
    ordered). Raises Kvfp8Error (workspace too small) when the plan needs
    more than NOALLOC_SCRATCH_BYTES."""
    out_dtype, num_pages, _ = _decode_checks(desc, out, q, k_cache, v_cache, block_tables,
                                             context_lens, k_scale, v_scale, None)
    _check("kvq_paged_decode_attention_noalloc", lib().kvq_paged_decode_attention_noalloc(
        ctypes.byref(desc), _ptr(out), out_dtype, _ptr(q), _ptr(k_cache), _ptr(v_cache),
        num_pages, _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), q.shape[0],
        int(max_context_len), _ptr(k_scale), _ptr(v_scale), _stream(stream)))


def decode_step(desc, k_new, v_new, k_cache, v_cache, out, q, block_tables,
                context_lens, max_context_len, k_scale=None, v_scale=None,
                workspace=None, stream=None):
    """Write every sequence's newest token (k_new, v_new: bf16 [B, Hkv, D],
    position context_lens[b] - 1) and attend, in one call: the same results
    as kv_cache_write followed by paged_decode_attention."""
    import torch
    _need(k_new, "k_new", torch.bfloat16)
    _need(v_new, "v_new", torch.bfloat16)
    B = q.shape[0]
    if tuple(k_new.shape) != (B, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new, v_new must be [B, Hkv, D]")
    out_dtype, num_pages, ws_bytes = _decode_checks(desc, out, q, k_cache, v_cache, block_tables,
                                                    context_lens, k_scale, v_scale, workspace)
    _check("kvq_decode_step", lib().kvq_decode_step(
        ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), num_pages,
        _ptr(out), out_dtype, _ptr(q), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, int(max_context_len), _ptr(k_scale), _ptr(v_scale),
        _ptr(workspace), ws_bytes, _stream(stream)))


def decode_step_dynamic(desc, k_new, v_new, k_cache, v_cache, out, q, block_tables,
                        context_lens, max_context_len, k_scales, v_scales, workspace=None,
                        stream=None):
    """decode_step for a layer with dynamic per-token scales: the new token's
    scales go into the pools (float32 [P, Hkv, 16]), then every position is
    attended with its own scales."""
    import torch
    _need(k_new, "k_new", torch.bfloat16)
    _need(v_new, "v_new", torch.bfloat16)
    B = q.shape[0]
    if tuple(k_new.shape) != (B, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new, v_new must be [B, Hkv, D]")
    _check_pools(desc, k_cache, k_scales, v_scales)
    out_dtype, num_pages, ws_bytes = _decode_checks(desc, out, q, k_cache, v_cache, block_tables,
                                                    context_lens, k_scales, v_scales, workspace)
    _check("kvq_decode_step_dynamic", lib().kvq_decode_step_dynamic(
        ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), num_pages,
        _ptr(out), out_dtype, _ptr(q), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, int(max_context_len), _ptr(k_scales), _ptr(v_scales),
        _ptr(workspace), ws_bytes, _stream(stream)))


def paged_prefill_attention(desc, out, q, k_cache, v_cache, block_tables, query_start,
                            context_lens, max_query_len, k_scale=None, v_scale=None,
                            workspace=None, stream=None):
    """Chunked-prefill attention: q, out [T, Hq, D] (bf16 / float32 or bf16)
    hold every sequence's new rows (sequence b's rows query_start[b] ..
    query_start[b+1]-1, int32 [B+1], are its last positions; context_lens
    int32 [B] counts the written positions, the chunk included); each row
    attends causally to its prefix. max_query_len: host bound of the rows per
    sequence. workspace: from alloc_prefill_workspace (lets a short chunk over
    a long context split its keys), or None (no split)."""
    import torch
    _need(out, "out")
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache")
    _need(block_tables, "block_tables", torch.int32)
    _need(query_start, "query_start", torch.int32)
    _need(context_lens, "context_lens", torch.int32)
    _need(k_scale, "k_scale", torch.float32)
    _need(v_scale, "v_scale", torch.float32)
    _need(workspace, "workspace")
    if out.dtype == torch.float32:
        out_dtype = OUT_F32
    elif out.dtype == torch.bfloat16:
        out_dtype = OUT_BF16
    else:
        raise ValueError("out must be float32 or bfloat16")
    T = q.shape[0]
    if tuple(q.shape) != (T, desc.num_q_heads, desc.head_dim) or out.shape != q.shape:
        raise ValueError("q, out must be [T, Hq, D]")
    B = context_lens.numel()
    if query_start.numel() != B + 1 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("query_start must be [B+1], block_tables [B, max_pages]")
    num_pages = k_cache.numel() * k_cache.element_size() // (desc.num_kv_heads * desc.page_bytes)
    _check("kvq_paged_prefill_attention", lib().kvq_paged_prefill_attention(
        ctypes.byref(desc), _ptr(out), out_dtype, _ptr(q), _ptr(k_cache), _ptr(v_cache),
        num_pages, _ptr(block_tables), block_tables.shape[1], _ptr(query_start),
        _ptr(context_lens), B, int(max_query_len), _ptr(k_scale), _ptr(v_scale),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))


def kv_scale_from_amax(desc, x, scale_out, stream=None):
    """scale_out[h] = amax(|x[:, h, :]|) / 448 (57344 for an e5m2 layer), or
    one scale over all heads for per-tensor layers. x: bf16 [T, Hkv, D];
    scale_out: float32."""
    import torch
    _need(x, "x", torch.bfloat16)
    _need(scale_out, "scale_out", torch.float32)
    if x.dim() != 3 or x.shape[1] != desc.num_kv_heads or x.shape[2] != desc.head_dim:
        raise ValueError("x must be [T, Hkv, D]")
    want = desc.num_kv_heads if desc.scale_mode == PER_KV_HEAD else 1
    if scale_out.numel() != want:
        raise ValueError(f"scale_out must have {want} entries")
    _check("kvq_kv_scale_from_amax", lib().kvq_kv_scale_from_amax(
        ctypes.byref(desc), _ptr(x), x.shape[0], _ptr(scale_out), _stream(stream)))


def _quantize(fn, x, scale, out, stream):
    import torch
    _need(x, "x", torch.float32)
    _need(scale, "scale", torch.float32)
    _need(out, "out", torch.uint8)
    if out.numel() != x.numel():
        raise ValueError("out must have as many elements as x")
    _check(fn, getattr(lib(), fn)(_ptr(x), x.numel(), _ptr(scale), _ptr(out), _stream(stream)))


def e4m3_quantize(x, scale, out, stream=None):
    """out[i] = e4m3_sat_rne(x[i] / scale[0]); x float32, out uint8."""
    _quantize("kvq_e4m3_quantize", x, scale, out, stream)


def e5m2_quantize(x, scale, out, stream=None):
    """out[i] = e5m2_sat_rne(x[i] / scale[0]); x float32, out uint8."""
    _quantize("kvq_e5m2_quantize", x, scale, out, stream)


# kvq_set_tuning knobs (include/kvfp8.h, enum kvq_tuning_knob)
TUNING_KNOBS = {"pages_per_wave": 0, "partition_rotate": 1, "split_shape": 2,
                "prefill_column_groups": 3, "prefill_key_parts": 4}


def set_tuning(knob, value):
    """Override one launch-plan choice for every later call (sweeps and
    tests; see kvq_set_tuning). knob: a TUNING_KNOBS name; value None (or
    -1) gives the choice back to the plan. split_shape takes "TPxRING" or
    "TPxRINGsSLOTS" (e.g. "2x1s1") or the header's integer code."""
    if value is None:
        value = -1
    elif knob == "split_shape" and isinstance(value, str):
        tp, rest = value.split("x")
        ring, _, slots = rest.partition("s")
        value = 100 * int(tp) + 10 * int(ring) + int(slots or 0)
    _check("kvq_set_tuning", lib().kvq_set_tuning(TUNING_KNOBS[knob], int(value)))


def reset_tuning():
    """Every knob back to the plan's choice."""
    for k in TUNING_KNOBS:
        set_tuning(k, None)


def profile_begin(max_launches):
    _check("kvq_profile_begin", lib().kvq_profile_begin(int(max_launches)))


def stream_read(src, sink, stream=None):
    """Timing aid: read every byte of the contiguous device tensor src once
    (16-byte non-temporal loads); sink (int32, one word per work-group,
    sink.numel() work-groups) receives per-work-group XOR checksums."""
    import torch
    if not src.is_contiguous() or src.numel() * src.element_size() % 16:
        raise ValueError("src must be contiguous with a size that is a multiple of 16 bytes")
    if sink.dtype != torch.int32 or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous int32 tensor")
    _check("kvq_stream_read",
           lib().kvq_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                 sink.numel(), _stream(stream)))


def profile_end():
    """(summed split-kernel milliseconds, launches recorded)."""
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    _check("kvq_profile_end", lib().kvq_profile_end(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, int(n.value)
