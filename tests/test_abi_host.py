"""Host-side checks of the C ABI (no GPU): the library loads, exports every
entry point include/kvfp8.h declares, and rejects bad arguments with the
documented status before anything is launched."""

import ctypes
import os
import re

import pytest

import fp8_kv_cache_write_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvfp8.h")

OK, INVALID, UNSUPPORTED, WS_SMALL, HIP_ERR = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kv.LIB_PATH):
        from fp8_kv_cache_write_amd import build
        build.build()
    return kv.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("kvq_kv_cache_write", "kvq_paged_decode_attention",
              "kvq_decode_workspace_bytes", "kvq_kv_scale_from_amax",
              "kvq_e4m3_quantize", "kvq_status_string"):
        assert f in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    assert kv.status_string(OK) == "ok"
    assert "workspace" in kv.status_string(WS_SMALL)
    assert kv.status_string(12345) == "unknown status"


FAKE = ctypes.c_void_p(0x100000)        # aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x100004)    # 4-byte aligned only


def write(L, desc, k=FAKE, v=FAKE, slots=FAKE, T=4, kc=FAKE, vc=FAKE, P=8,
          ks=FAKE, vs=FAKE):
    return L.kvq_kv_cache_write(ctypes.byref(desc), k, v, slots, T, kc, vc, P, ks, vs,
                                None)


def attend(L, desc, out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, P=8, bt=FAKE, mp=8,
           lens=FAKE, B=1, maxlen=100, ks=FAKE, vs=FAKE, ws=FAKE, wsb=1 << 30,
           out_dtype=0):
    return L.kvq_paged_decode_attention(ctypes.byref(desc), out, out_dtype, q, kc, vc, P,
                                        bt, mp, lens, B, maxlen, ks, vs, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), UNSUPPORTED),
    (dict(head_dim=512), UNSUPPORTED),
    (dict(num_q_heads=30, num_kv_heads=8), UNSUPPORTED),
    (dict(num_q_heads=68, num_kv_heads=4), UNSUPPORTED),   # group 17 > 16
    (dict(num_q_heads=65536, num_kv_heads=65536), UNSUPPORTED),   # Hkv > 65535
    (dict(num_q_heads=0), INVALID),
    (dict(sliding_window=-1), INVALID),
    (dict(sm_scale=-1.0), INVALID),
])
def test_descriptor_checks(L, kw, status):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128)
    base.update(kw)
    d = kv.layer_desc(**base)
    assert write(L, d) == status
    assert attend(L, d) == status
    n = ctypes.c_size_t()
    assert L.kvq_decode_workspace_bytes(ctypes.byref(d), 1, 100, ctypes.byref(n)) == status


def test_page_size_must_be_16(L):
    d = kv.layer_desc(32, 8, 128)
    d.page_size = 32
    assert write(L, d) == UNSUPPORTED


def test_write_argument_checks(L):
    d = kv.layer_desc(32, 8, 128)
    assert write(L, d, k=None) == INVALID
    assert write(L, d, slots=None) == INVALID
    assert write(L, d, kc=FAKE_ODD) == INVALID
    assert write(L, d, ks=None) == INVALID           # fp8 layers need scales
    assert write(L, d, T=-1) == INVALID
    assert write(L, d, T=0, k=None) == OK            # nothing to do, nothing launched
    b = kv.layer_desc(32, 8, 128, cache_dtype="bf16")
    assert write(L, b, T=0, ks=None, vs=None) == OK


def test_stream_read_argument_checks(L):
    # every rejection happens on the host, before any launch
    sr = L.kvq_stream_read
    assert sr(FAKE, 17, FAKE, 4, None) == INVALID        # not a multiple of 16 bytes
    assert sr(FAKE, -16, FAKE, 4, None) == INVALID
    assert sr(FAKE, 1024, FAKE, 0, None) == INVALID      # no work-groups
    assert sr(None, 1024, FAKE, 4, None) == INVALID
    assert sr(FAKE_ODD, 1024, FAKE, 4, None) == INVALID  # src not 16-byte aligned
    assert sr(FAKE, 1024, None, 4, None) == INVALID
    assert sr(None, 0, None, 4, None) == OK              # nothing to read, no launch


def test_attention_argument_checks(L):
    d = kv.layer_desc(32, 8, 128)
    assert attend(L, d, q=None) == INVALID
    assert attend(L, d, out=FAKE_ODD) == INVALID
    assert attend(L, d, mp=6, maxlen=100) == INVALID     # 100 positions need 7 pages
    assert attend(L, d, out_dtype=7) == INVALID
    assert attend(L, d, ks=None) == INVALID
    assert attend(L, d, B=0) == OK


def test_workspace_checks(L):
    d = kv.layer_desc(32, 8, 128)
    need = kv.decode_workspace_bytes(d, 1, 131072)
    assert need > 0
    mp = 131072 // 16
    assert attend(L, d, maxlen=131072, mp=mp, wsb=need - 1) == WS_SMALL
    assert attend(L, d, maxlen=131072, mp=mp, ws=None, wsb=need) == INVALID


def test_workspace_plan():
    d = kv.layer_desc(32, 8, 128)
    # short contexts and sliding windows finish in the split kernel
    assert kv.decode_workspace_bytes(d, 1, 256) == 0
    sw = kv.layer_desc(64, 8, 64, cache_dtype="bf16", sliding_window=128)
    assert kv.decode_workspace_bytes(sw, 1, 32768) == 0
    # long contexts split: one (m, l, o[D]) float row per partition and head
    sizes = [kv.decode_workspace_bytes(d, 1, n) for n in (8192, 32768, 131072)]
    assert sizes[0] <= sizes[1] <= sizes[2]
    assert sizes[2] >= 32 * 2 * (128 + 2) * 4
    # partials stay a small fraction of the KV bytes they summarise
    assert sizes[2] < 0.02 * (2 * 131072 * 8 * 128)


def test_no_oracle_in_the_product():
    pkg = os.path.join(ROOT, "fp8_kv_cache_write_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "liboracle" not in text, f
                assert "orc_" not in text, f


def test_fp8_attention_mode_checks():
    # the all-FP8 mode reads fp8 caches only; both modes take groups up to 16
    with pytest.raises(kv.Kvfp8Error):
        kv.decode_workspace_bytes(kv.layer_desc(32, 8, 128, "bf16", attn="fp8"), 1, 1024)
    assert kv.decode_workspace_bytes(kv.layer_desc(64, 4, 128, attn="fp8"), 1, 4096) >= 0
    assert kv.decode_workspace_bytes(kv.layer_desc(64, 4, 128, "fp8_e5m2", attn="fp8"), 1,
                                     4096) >= 0
    assert kv.decode_workspace_bytes(kv.layer_desc(64, 4, 128, attn="bf16"), 1, 4096) >= 0
    with pytest.raises(kv.Kvfp8Error):
        kv.decode_workspace_bytes(kv.layer_desc(68, 4, 128, attn="bf16"), 1, 1024)
    with pytest.raises(kv.Kvfp8Error):
        kv.decode_workspace_bytes(kv.layer_desc(128, 4, 128, attn="fp8"), 1, 1024)
    bad = kv.layer_desc(32, 8, 128)
    bad.attn_dtype = 7
    with pytest.raises(kv.Kvfp8Error):
        kv.decode_workspace_bytes(bad, 1, 1024)


def write_dyn(L, desc, k=FAKE, v=FAKE, slots=FAKE, T=4, kc=FAKE, vc=FAKE, P=8, ks=FAKE,
              vs=FAKE):
    return L.kvq_kv_cache_write_dynamic(ctypes.byref(desc), k, v, slots, T, kc, vc, P, ks, vs,
                                        None)


def step_dyn(L, desc, ks=FAKE, vs=FAKE, out=FAKE):
    return L.kvq_decode_step_dynamic(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, 8, out, 0,
                                     FAKE, FAKE, 8, FAKE, 1, 100, ks, vs, FAKE, 1 << 30, None)


def test_dynamic_scale_mode_checks(L):
    dyn = kv.layer_desc(32, 8, 128, scale_mode="per_token")
    dynh = kv.layer_desc(32, 8, 128, "fp8_e5m2", scale_mode="per_token_head")
    static = kv.layer_desc(32, 8, 128)
    assert dyn.dynamic and dynh.dynamic and not static.dynamic
    # each write / decode-step entry point takes its own kind of scales
    assert write(L, dyn) == INVALID
    assert write_dyn(L, static) == INVALID
    assert step_dyn(L, static) == INVALID
    assert L.kvq_decode_step(ctypes.byref(dyn), FAKE, FAKE, FAKE, FAKE, 8, FAKE, 0, FAKE, FAKE,
                             8, FAKE, 1, 100, FAKE, FAKE, FAKE, 1 << 30, None) == INVALID
    # pools: present and 16-byte aligned
    assert write_dyn(L, dyn, ks=None) == INVALID
    assert write_dyn(L, dynh, vs=FAKE_ODD) == INVALID
    assert attend(L, dyn, ks=FAKE_ODD) == INVALID
    assert step_dyn(L, dyn, vs=None) == INVALID
    assert write_dyn(L, dyn, T=-1) == INVALID
    assert write_dyn(L, dyn, T=0) == OK
    # static calibration does not apply; FP8 arithmetic does not combine with it
    assert L.kvq_kv_scale_from_amax(ctypes.byref(dyn), FAKE, 4, FAKE, None) == INVALID
    assert attend(L, kv.layer_desc(32, 8, 128, scale_mode="per_token", attn="fp8")) == UNSUPPORTED
    assert write_dyn(L, kv.layer_desc(512, 512, 64, scale_mode="per_token")) == UNSUPPORTED
    # a bf16 layer ignores the scale mode and copies
    assert write_dyn(L, kv.layer_desc(32, 8, 128, "bf16", scale_mode="per_token"), ks=None,
                     vs=None, T=0) == OK
    bad = kv.layer_desc(32, 8, 128)
    bad.scale_mode = 4
    assert write(L, bad) == INVALID


def test_dynamic_plan_leaves_the_lds_ring_for_d256():
    # a staged fp8 D=256 tile with its scales would pass 64 KiB of ring: the
    # plan takes the register shape, so the same workspace size follows
    s = kv.decode_workspace_bytes(kv.layer_desc(8, 2, 256), 1, 65536)
    d = kv.decode_workspace_bytes(kv.layer_desc(8, 2, 256, scale_mode="per_token_head"), 1, 65536)
    assert s >= 0 and d >= 0


def test_prefill_argument_checks(L):
    def pf(desc, out=FAKE, q=FAKE, qs=FAKE, lens=FAKE, B=1, mq=16, ks=FAKE, vs=FAKE, P=8,
           mp=8, ws=None, wsb=0):
        return L.kvq_paged_prefill_attention(ctypes.byref(desc), out, 0, q, FAKE, FAKE, P, FAKE,
                                             mp, qs, lens, B, mq, ks, vs, ws, wsb, None)
    d = kv.layer_desc(32, 8, 128)
    assert pf(d, ws=None, wsb=256) == INVALID       # a size without a workspace
    assert pf(d, ws=FAKE_ODD, wsb=1 << 20) == INVALID   # not 256-byte aligned
    # a 16-row chunk over 131072 positions splits its keys: a workspace must hold them
    need = kv.prefill_workspace_bytes(d, 1, 16, 8192)
    assert need > 0
    assert pf(d, mp=8192, ws=FAKE, wsb=need - 256) == WS_SMALL
    assert pf(d, out=None) == INVALID
    assert pf(d, qs=None) == INVALID
    assert pf(d, out=FAKE_ODD) == INVALID
    assert pf(d, ks=None) == INVALID               # fp8 layers need scales
    assert pf(d, B=-1) == INVALID
    assert pf(d, B=0) == OK and pf(d, mq=0) == OK   # nothing to do
    assert pf(d, P=0) == INVALID
    assert pf(kv.layer_desc(32, 8, 128, "bf16", attn="fp8")) == UNSUPPORTED
    assert pf(kv.layer_desc(32, 8, 128, scale_mode="per_token"), ks=FAKE_ODD) == INVALID
    assert pf(kv.layer_desc(32, 8, 96)) == UNSUPPORTED
    # more work-groups than one launch takes (65535 sequences x 4096 KV heads
    # x 22 query blocks): refused on the host before any device call
    assert pf(kv.layer_desc(4096, 4096, 64), B=65535, mq=4096) == HIP_ERR


def test_prefill_workspace_plan(tune):
    d = kv.layer_desc(32, 8, 128)
    tune("prefill_key_parts", None)
    # a short chunk over a long context splits; the partials are
    # (m, l, o[D]) per (row, query head, partition), plus the merge's slack
    n = kv.prefill_workspace_bytes(d, 1, 512, 2048)
    assert n >= 512 * 32 * 2 * (128 + 2) * 4
    assert kv.prefill_workspace_bytes(d, 1, 512, 8192) >= n
    # whole prompts (keys shorter than twice the chunk) and short key ranges
    # keep one partition; so do batches with more rows than the merge grid holds
    assert kv.prefill_workspace_bytes(d, 1, 32768, 2048) == 0
    assert kv.prefill_workspace_bytes(d, 1, 512, 32) == 0
    assert kv.prefill_workspace_bytes(d, 8, 16384, 65536) == 0
    assert kv.prefill_workspace_bytes(d, 0, 512, 2048) == 0
    # enough query blocks to fill the device: no split
    assert kv.prefill_workspace_bytes(d, 64, 512, 2048) == 0
    # the override forces a split even where the plan would not
    tune("prefill_key_parts", 3)
    assert kv.prefill_workspace_bytes(d, 1, 64, 40) > 0
    tune("prefill_key_parts", 1)
    assert kv.prefill_workspace_bytes(d, 1, 512, 8192) == 0


def test_tuning_overrides_are_explicit(tune, monkeypatch):
    """The plan changes only through kvq_set_tuning: environment variables
    named like the old sweep switches do nothing, out-of-range values are
    rejected, and -1 gives a knob back to the plan."""
    d = kv.layer_desc(32, 8, 128)
    base = kv.decode_workspace_bytes(d, 1, 32768)
    assert base > 0
    for name in ("KVFP8_PAGES_PER_WAVE", "KVFP8_PARTITION_ROTATE", "KVFP8_SPLIT_VARIANT",
                 "KVFP8_PREFILL_COLUMN_GROUPS", "KVFP8_PREFILL_KEY_PARTS"):
        monkeypatch.setenv(name, "1")
    assert kv.decode_workspace_bytes(d, 1, 32768) == base
    # 2-page runs: 8x the partitions of the plan's 16-page runs
    tune("pages_per_wave", 2)
    assert kv.decode_workspace_bytes(d, 1, 32768) > 4 * base
    tune("pages_per_wave", None)
    assert kv.decode_workspace_bytes(d, 1, 32768) == base
    L = kv.lib()
    for knob, bad in ((0, 0), (0, 65), (1, 2), (2, 213), (2, 0), (3, 4), (4, 0), (5, 1),
                      (-1, 1)):
        assert L.kvq_set_tuning(knob, bad) == INVALID, (knob, bad)
    for knob, good in ((0, 64), (1, 0), (2, 211), (3, 3), (4, 7)):
        assert L.kvq_set_tuning(knob, good) == OK
        assert L.kvq_set_tuning(knob, -1) == OK


def test_noalloc_size_limit_is_checked_on_the_host(L):
    """The no-allocation decode entry point rejects a plan whose workspace
    exceeds its device array before touching any device."""
    d = kv.layer_desc(32, 8, 128)
    assert kv.decode_workspace_bytes(d, 64, 131072) > kv.NOALLOC_SCRATCH_BYTES
    st = L.kvq_paged_decode_attention_noalloc(ctypes.byref(d), FAKE, 0, FAKE, FAKE, FAKE, 16,
                                              FAKE, 8192, FAKE, 64, 131072, FAKE, FAKE, None)
    assert st == WS_SMALL
    assert L.kvq_paged_decode_attention_noalloc(None, FAKE, 0, FAKE, FAKE, FAKE, 16, FAKE, 8192,
                                                FAKE, 1, 16, FAKE, FAKE, None) == INVALID
