"""CPU oracle for the FP8 (e4m3, e5m2) paged KV cache and GQA paged decode
attention.

TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__ and the
CPU-baseline leg of bench.py import this package. The product path (the HIP
library and its binding) never does, and shares no code with it: liboracle.so
is built from oracle.c alone, in float64, from the definitions cited there.

Every function takes and returns numpy arrays; bf16 data travels as its raw
uint16 bits so that both sides see exactly the same inputs.
"""

import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_u64p = ctypes.POINTER(ctypes.c_uint64)

FP8 = 1          # e4m3
E5M2 = 2
BF16 = 0


def lib():
    """Load liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if _lib is None:
        # ORACLE_LIB names another build of oracle.c (the sanitizer test
        # loads liboracle_asan.so this way)
        path = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode_all.argtypes = [_f64p]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode_scan.restype = ctypes.c_uint8
        L.orc_e4m3_encode_scan.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode_bits.restype = ctypes.c_uint8
        L.orc_e4m3_encode_bits.argtypes = [ctypes.c_uint32]
        L.orc_e5m2_decode.restype = ctypes.c_double
        L.orc_e5m2_decode.argtypes = [ctypes.c_uint8]
        L.orc_e5m2_decode_all.argtypes = [_f64p]
        L.orc_e5m2_encode.restype = ctypes.c_uint8
        L.orc_e5m2_encode.argtypes = [ctypes.c_float]
        L.orc_e5m2_encode_scan.restype = ctypes.c_uint8
        L.orc_e5m2_encode_scan.argtypes = [ctypes.c_float]
        L.orc_e5m2_encode_bits.restype = ctypes.c_uint8
        L.orc_e5m2_encode_bits.argtypes = [ctypes.c_uint32]
        L.orc_sweep_encoders_e5m2.restype = ctypes.c_uint64
        L.orc_sweep_encoders_e5m2.argtypes = [ctypes.c_uint64, ctypes.c_uint64,
                                              ctypes.c_int, _u64p]
        L.orc_quantize_fmt.restype = ctypes.c_uint8
        L.orc_quantize_fmt.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_float]
        L.orc_quantize_fmt_array_mt.argtypes = [ctypes.c_int, _f32p, ctypes.c_int64,
                                                ctypes.c_float, _u8p, ctypes.c_int]
        L.orc_scale_from_amax_fmt.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              _f32p]
        L.orc_sweep_encoders.restype = ctypes.c_uint64
        L.orc_sweep_encoders.argtypes = [ctypes.c_uint64, ctypes.c_uint64,
                                         ctypes.c_int, _u64p]
        L.orc_quantize_f32.restype = ctypes.c_uint8
        L.orc_quantize_f32.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_quantize_f32_array.argtypes = [_f32p, ctypes.c_int64,
                                             ctypes.c_float, _u8p]
        L.orc_quantize_f32_array_mt.argtypes = [_f32p, ctypes.c_int64,
                                                ctypes.c_float, _u8p,
                                                ctypes.c_int]
        L.orc_scale_from_amax.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, _f32p]
        L.orc_k_offset.restype = ctypes.c_int64
        L.orc_k_offset.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.orc_v_offset.restype = ctypes.c_int64
        L.orc_v_offset.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.orc_kv_cache_write.argtypes = [ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, _u16p,
                                         _u16p, _i64p, ctypes.c_int64, _u8p,
                                         _u8p, ctypes.c_int64, _f32p, _f32p]
        L.orc_kv_cache_write_mt.argtypes = [ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, _u16p,
                                            _u16p, _i64p, ctypes.c_int64, _u8p,
                                            _u8p, ctypes.c_int64, _f32p, _f32p,
                                            ctypes.c_int]
        L.orc_kv_cache_write_dyn_mt.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, _u16p, _u16p, _i64p,
                                                ctypes.c_int64, _u8p, _u8p, ctypes.c_int64,
                                                _f32p, _f32p, ctypes.c_int]
        L.orc_prefill_attention.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_double, _u16p, _u8p, _u8p,
                                            _i32p, ctypes.c_int, _i32p, _i32p, _f32p, _f32p,
                                            _i32p, ctypes.c_int64, _f64p, ctypes.c_int,
                                            ctypes.c_int]
        L.orc_softmax_weighted_sum.argtypes = [_f64p, _f64p, ctypes.c_int64,
                                               ctypes.c_int, _f64p]
        att = [ctypes.c_int] * 7 + [ctypes.c_double, _u16p, _u8p, _u8p, _i32p,
                                     ctypes.c_int, _i32p, _f32p, _f32p, _f64p]
        L.orc_attention.argtypes = att + [ctypes.c_int]
        L.orc_attention_split.argtypes = att + [ctypes.c_int, ctypes.c_int]
        L.orc_attention_lowprec.argtypes = att + [ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int]
        L.orc_attention_fp8attn.argtypes = att + [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _threads(n=None):
    return int(n or os.environ.get("ORACLE_THREADS", 0) or os.cpu_count() or 1)


# ---------------------------------------------------------------- codec ----
def e4m3_decode_all() -> np.ndarray:
    out = np.zeros(256, dtype=np.float64)
    lib().orc_e4m3_decode_all(_ptr(out, _f64p))
    return out


def e4m3_encode(y: float) -> int:
    return int(lib().orc_e4m3_encode(ctypes.c_float(y)))


def e4m3_encode_scan(y: float) -> int:
    return int(lib().orc_e4m3_encode_scan(ctypes.c_float(y)))


def e4m3_encode_bits(u: int) -> int:
    return int(lib().orc_e4m3_encode_bits(ctypes.c_uint32(u)))


def sweep_encoders(lo=0, hi=1 << 32, nthreads=None, fmt=FP8):
    """Compare the table encoder with the bit-field encoder of one format
    (FP8 = e4m3, E5M2) on every 32-bit pattern in [lo, hi). Returns
    (mismatches, first mismatching pattern)."""
    first = ctypes.c_uint64(0)
    fn = lib().orc_sweep_encoders_e5m2 if fmt == E5M2 else lib().orc_sweep_encoders
    bad = fn(lo, hi, _threads(nthreads), ctypes.byref(first))
    return int(bad), int(first.value)


def e5m2_decode_all() -> np.ndarray:
    out = np.zeros(256, dtype=np.float64)
    lib().orc_e5m2_decode_all(_ptr(out, _f64p))
    return out


def e5m2_encode(y: float) -> int:
    return int(lib().orc_e5m2_encode(ctypes.c_float(y)))


def e5m2_encode_scan(y: float) -> int:
    return int(lib().orc_e5m2_encode_scan(ctypes.c_float(y)))


def e5m2_encode_bits(u: int) -> int:
    return int(lib().orc_e5m2_encode_bits(ctypes.c_uint32(u)))


def quantize(x_f32: np.ndarray, scale: float, nthreads=None, fmt=FP8) -> np.ndarray:
    """FMT_sat_RNE(x / scale) element by element (fp32 division); fmt FP8 is
    e4m3, E5M2 is e5m2."""
    x = np.ascontiguousarray(x_f32, dtype=np.float32).ravel()
    out = np.empty(x.size, dtype=np.uint8)
    lib().orc_quantize_fmt_array_mt(int(fmt), _ptr(x, _f32p), x.size, ctypes.c_float(scale),
                                    _ptr(out, _u8p), _threads(nthreads))
    return out.reshape(np.shape(x_f32))


def quantize_one(x: float, scale: float, fmt=FP8) -> int:
    return int(lib().orc_quantize_fmt(int(fmt), ctypes.c_float(x), ctypes.c_float(scale)))


# ---------------------------------------------------------------- scales ---
def scale_from_amax(x_bf16: np.ndarray, per_head: bool, fmt=FP8) -> np.ndarray:
    """x_bf16: uint16 [T][H][D]. Returns float32 [H] or [1]: amax / 448 (e4m3)
    or amax / 57344 (e5m2)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T, H, D = x.shape
    out = np.zeros(H if per_head else 1, dtype=np.float32)
    lib().orc_scale_from_amax_fmt(_ptr(x, _u16p), T, H, D, int(per_head), int(fmt),
                                  _ptr(out, _f32p))
    return out


# ---------------------------------------------------------------- layout ---
def k_offset(r, d, elem_bytes):
    return int(lib().orc_k_offset(r, d, elem_bytes))


def v_offset(r, d, elem_bytes):
    return int(lib().orc_v_offset(r, d, elem_bytes))


def page_bytes(head_dim: int, dtype: int) -> int:
    return 16 * head_dim * (2 if dtype == BF16 else 1)


# ----------------------------------------------------------- cache write ---
def kv_cache_write(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray,
                   v: np.ndarray, slots: np.ndarray, dtype: int, per_head: bool,
                   k_scale=None, v_scale=None, nthreads=None):
    """In place on uint8 caches [P][H][PB]. k, v: uint16 bf16 bits [T][H][D]."""
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    T, H, D = k.shape
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.dtype == np.uint8 and v_cache.dtype == np.uint8
    num_pages = k_cache.shape[0]
    ks = np.ascontiguousarray(k_scale if k_scale is not None else [1.0], dtype=np.float32)
    vs = np.ascontiguousarray(v_scale if v_scale is not None else [1.0], dtype=np.float32)
    lib().orc_kv_cache_write_mt(H, D, dtype, int(per_head), _ptr(k, _u16p),
                                _ptr(v, _u16p), _ptr(slots, _i64p), T,
                                _ptr(k_cache, _u8p), _ptr(v_cache, _u8p),
                                num_pages, _ptr(ks, _f32p), _ptr(vs, _f32p),
                                _threads(nthreads))


PER_TENSOR, PER_KV_HEAD, PER_TOKEN, PER_TOKEN_HEAD = 0, 1, 2, 3


def scale_pools(num_pages: int, num_kv_heads: int):
    """Zeroed K and V scale pools, float32 [P][H][16] (one scale per slot)."""
    return (np.zeros((num_pages, num_kv_heads, 16), np.float32),
            np.zeros((num_pages, num_kv_heads, 16), np.float32))


def kv_cache_write_dyn(k_cache, v_cache, k, v, slots, dtype, mode, k_pool, v_pool,
                       nthreads=None):
    """Cache write with dynamic per-token scales (mode PER_TOKEN: one per
    token over all heads; PER_TOKEN_HEAD: one per token and KV head). In
    place on the uint8 caches [P][H][PB] and the float32 pools [P][H][16]."""
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    T, H, D = k.shape
    assert mode in (PER_TOKEN, PER_TOKEN_HEAD) and H <= 256
    for a in (k_cache, v_cache):
        assert a.flags.c_contiguous and a.dtype == np.uint8
    for a in (k_pool, v_pool):
        assert a.flags.c_contiguous and a.dtype == np.float32 and a.shape == (k_cache.shape[0], H, 16)
    lib().orc_kv_cache_write_dyn_mt(H, D, dtype, int(mode), _ptr(k, _u16p), _ptr(v, _u16p),
                                    _ptr(slots, _i64p), T, _ptr(k_cache, _u8p),
                                    _ptr(v_cache, _u8p), k_cache.shape[0],
                                    _ptr(k_pool, _f32p), _ptr(v_pool, _f32p),
                                    _threads(nthreads))


# -------------------------------------------------------------- attention --
def softmax_weighted_sum(z: np.ndarray, v: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    n, D = v.shape
    out = np.zeros(D, dtype=np.float64)
    lib().orc_softmax_weighted_sum(_ptr(z, _f64p), _ptr(v, _f64p), n, D,
                                   _ptr(out, _f64p))
    return out


def _att_common(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                dtype, per_head, window, sm_scale, k_scale, v_scale):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    B, Hq, D = q.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    ks = np.ascontiguousarray(k_scale if k_scale is not None else [1.0], dtype=np.float32)
    vs = np.ascontiguousarray(v_scale if v_scale is not None else [1.0], dtype=np.float32)
    kc = np.ascontiguousarray(k_cache, dtype=np.uint8)
    vc = np.ascontiguousarray(v_cache, dtype=np.uint8)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    args = [B, Hq, num_kv_heads, D, dtype, int(per_head), int(window),
            float(sm_scale or 0.0), _ptr(q, _u16p), _ptr(kc, _u8p),
            _ptr(vc, _u8p), _ptr(bt, _i32p), bt.shape[1], _ptr(lens, _i32p),
            _ptr(ks, _f32p), _ptr(vs, _f32p), _ptr(out, _f64p)]
    keep = (q, bt, lens, ks, vs, kc, vc)
    return args, out, keep


def attention(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
              dtype, per_head=True, window=0, sm_scale=0.0, k_scale=None,
              v_scale=None, nthreads=None) -> np.ndarray:
    """float64 [B][Hq][D] decode attention over the paged caches. per_head
    is the scale mode: False / PER_TENSOR, True / PER_KV_HEAD, or PER_TOKEN /
    PER_TOKEN_HEAD with k_scale, v_scale the float32 [P][H][16] pools."""
    args, out, _keep = _att_common(q, k_cache, v_cache, block_tables,
                                   context_lens, num_kv_heads, dtype, per_head,
                                   window, sm_scale, k_scale, v_scale)
    lib().orc_attention(*args, _threads(nthreads))
    return out


def attention_split(q, k_cache, v_cache, block_tables, context_lens,
                    num_kv_heads, dtype, part_tokens, per_head=True, window=0,
                    sm_scale=0.0, k_scale=None, v_scale=None, nthreads=None):
    args, out, _keep = _att_common(q, k_cache, v_cache, block_tables,
                                   context_lens, num_kv_heads, dtype, per_head,
                                   window, sm_scale, k_scale, v_scale)
    lib().orc_attention_split(*args, int(part_tokens), _threads(nthreads))
    return out


def attention_lowprec(q, k_cache, v_cache, block_tables, context_lens,
                      num_kv_heads, dtype, acc_bits, acc_tile=0, per_head=True,
                      window=0, sm_scale=0.0, k_scale=None, v_scale=None,
                      nthreads=None):
    args, out, _keep = _att_common(q, k_cache, v_cache, block_tables,
                                   context_lens, num_kv_heads, dtype, per_head,
                                   window, sm_scale, k_scale, v_scale)
    lib().orc_attention_lowprec(*args, int(acc_bits), int(acc_tile),
                                _threads(nthreads))
    return out


def attention_fp8attn(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                      dtype, per_head=True, window=0, sm_scale=0.0, k_scale=None,
                      v_scale=None, nthreads=None) -> np.ndarray:
    """All-FP8 attention: q quantised to e4m3 per row (s = amax / 448), the
    probabilities quantised to e4m3 per aligned 32-position block relative
    to the block's largest logit; float64 elsewhere. [B][Hq][D]."""
    args, out, _keep = _att_common(q, k_cache, v_cache, block_tables,
                                   context_lens, num_kv_heads, dtype, per_head,
                                   window, sm_scale, k_scale, v_scale)
    lib().orc_attention_fp8attn(*args, _threads(nthreads))
    return out


def prefill_attention(q, k_cache, v_cache, block_tables, query_start, context_lens,
                      num_kv_heads, dtype, per_head=True, window=0, sm_scale=0.0, k_scale=None,
                      v_scale=None, rows=None, nthreads=None, fp8attn=False) -> np.ndarray:
    """Chunked-prefill attention: q bf16 [T][Hq][D] holds every sequence's
    new rows (sequence b's rows are query_start[b] .. query_start[b+1]-1, its
    last positions); each row attends causally to its prefix (window-limited).
    rows: optional indices of the rows to compute. fp8attn: the all-FP8
    arithmetic of attention_fp8attn, row by row. float64 [n_rows][Hq][D]."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    T, Hq, D = q.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    B = lens.shape[0]
    assert qs.shape == (B + 1,) and qs[0] == 0 and qs[-1] == T
    ks = np.ascontiguousarray(k_scale if k_scale is not None else [1.0], dtype=np.float32)
    vs = np.ascontiguousarray(v_scale if v_scale is not None else [1.0], dtype=np.float32)
    kc = np.ascontiguousarray(k_cache, dtype=np.uint8)
    vc = np.ascontiguousarray(v_cache, dtype=np.uint8)
    rw = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n_rows = T if rw is None else rw.shape[0]
    out = np.zeros((n_rows, Hq, D), dtype=np.float64)
    lib().orc_prefill_attention(B, Hq, num_kv_heads, D, dtype, int(per_head), int(window),
                                float(sm_scale or 0.0), _ptr(q, _u16p), _ptr(kc, _u8p),
                                _ptr(vc, _u8p), _ptr(bt, _i32p), bt.shape[1], _ptr(qs, _i32p),
                                _ptr(lens, _i32p), _ptr(ks, _f32p), _ptr(vs, _f32p),
                                None if rw is None else _ptr(rw, _i32p), n_rows,
                                _ptr(out, _f64p), int(bool(fp8attn)), _threads(nthreads))
    return out
