"""C-ABI checks that need no GPU: libkvq.so loads, exports every function
include/kvq.h declares, and every host-side validation path returns its
status before anything is enqueued (only such paths are exercised here)."""
import ctypes
import os
import re
from ctypes import byref, c_double, c_size_t, c_void_p

import pytest

import quantized_paged_kv_store_amd as K
from oracle import accounting as A
from quantized_paged_kv_store_amd.kvq import CacheDesc, Layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, ARG, UNSUP, SIZE = 0, -1, -2, -3
FAKE_DEV = 0x7f0000000000  # never dereferenced by the host code under test


def _lib():
    if not os.path.exists(K.kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")
    return K.library()


def _declared(header="kvq.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(kvq_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function():
    lib = _lib()
    names = _declared()
    assert set(names) >= {"kvq_alloc_pages", "kvq_store", "kvq_decode", "kvq_compute_scale",
                          "kvq_bytes_per_token", "kvq_status_string", "kvq_cache_layout",
                          "kvq_free_handle", "kvq_decode_workspace_bytes", "kvq_profile_enable",
                          "kvq_profile_read", "kvq_decode_append"}
    for n in names:
        assert hasattr(lib, n), n
    for header in sorted(os.listdir(os.path.join(ROOT, "include"))):
        for n in _declared(header):
            assert hasattr(lib, n), (header, n)


def test_status_strings():
    lib = _lib()
    for st in (OK, ARG, UNSUP, SIZE, -4, 12345):
        assert lib.kvq_status_string(st)


def _desc(dtype="e4m3", kind="gqa", hkv=8, d=128, dv=None, p=16, n=64):
    return K.make_desc(dtype, kind, hkv, d, d if dv is None else dv, p, n)


def test_bytes_per_token_matches_accounting():
    lib = _lib()
    out = c_double()
    for dtype in ("e4m3", "e5m2", "mx16"):
        assert lib.kvq_bytes_per_token(byref(_desc(dtype)), byref(out)) == OK
        assert out.value == A.kv_bytes_per_token(1, 8, 128, dtype)
    assert lib.kvq_bytes_per_token(byref(_desc("nvfp4", "mla", 1, 576, 512, 64)), byref(out)) == OK
    assert out.value == 324.0
    # 3.56x / 1.78x token capacity of FP4 block-16 vs BF16 / FP8
    fp8 = K.kvq_bytes_per_token(_desc("e4m3"))
    fp4 = K.kvq_bytes_per_token(_desc("mx16"))
    assert round(2 * fp8 / fp4, 2) == 3.56 and round(fp8 / fp4, 2) == 1.78


def test_alloc_query_bind_and_layout():
    lib = _lib()
    d = _desc("mx16", hkv=4, n=100)
    need = c_size_t()
    assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == OK
    h = c_void_p()
    assert lib.kvq_alloc_pages(byref(d), c_void_p(FAKE_DEV), need.value, byref(need), byref(h)) == OK
    lay = Layout()
    assert lib.kvq_cache_layout(h, byref(lay)) == OK
    assert lay.k_codes_bytes == lay.v_codes_bytes == 100 * 4 * 16 * 64
    assert lay.k_scales_bytes == lay.v_scales_bytes == 100 * 4 * 16 * 8
    assert lay.scratch_bytes >= 4096 and lay.total_bytes == need.value
    offs = [lay.k_codes_offset, lay.v_codes_offset, lay.k_scales_offset, lay.v_scales_offset, lay.scratch_offset]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    lib.kvq_free_handle(h)
    lib.kvq_free_handle(None)


@pytest.mark.parametrize("desc,status", [
    (dict(dtype="e4m3", d=96), UNSUP),
    (dict(dtype="mx16", d=64), UNSUP),
    (dict(dtype="nvfp4", kind="gqa"), UNSUP),
    (dict(dtype="e4m3", kind="mla", hkv=1, d=576, dv=512), UNSUP),
    (dict(dtype="nvfp4", kind="mla", hkv=2, d=576, dv=512), ARG),
    (dict(p=8), ARG),
    (dict(n=0), ARG),
    (dict(dv=64), ARG),
    (dict(d=100), ARG),
    (dict(p=65536 + 16), UNSUP),
    (dict(hkv=4097), UNSUP),
])
def test_alloc_rejects_bad_descriptors(desc, status):
    lib = _lib()
    need = c_size_t()
    assert lib.kvq_alloc_pages(byref(_desc(**desc)), None, 0, byref(need), None) == status


def test_alloc_size_and_alignment_errors():
    lib = _lib()
    d = _desc()
    need = c_size_t()
    h = c_void_p()
    assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == OK
    assert lib.kvq_alloc_pages(byref(d), c_void_p(FAKE_DEV), need.value - 1, byref(need), byref(h)) == SIZE
    assert lib.kvq_alloc_pages(byref(d), c_void_p(FAKE_DEV + 16), need.value, byref(need), byref(h)) == ARG
    assert lib.kvq_alloc_pages(byref(d), c_void_p(FAKE_DEV), need.value, byref(need), None) == ARG
    assert lib.kvq_alloc_pages(None, None, 0, byref(need), None) == ARG


@pytest.fixture
def handles():
    lib = _lib()
    out = {}
    for name, d in (("fp8", _desc("e4m3", hkv=2)), ("mx", _desc("mx16", hkv=2)),
                    ("mla", _desc("nvfp4", "mla", 1, 576, 512, 64))):
        need = c_size_t()
        h = c_void_p()
        assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == OK
        assert lib.kvq_alloc_pages(byref(d), c_void_p(FAKE_DEV), need.value, byref(need), byref(h)) == OK
        out[name] = h
    yield lib, out
    for h in out.values():
        lib.kvq_free_handle(h)


def test_store_argument_errors(handles):
    lib, h = handles
    P = c_void_p(FAKE_DEV)
    assert lib.kvq_store(h["fp8"], P, P, P, 0, None, None, None) == OK          # no-op
    assert lib.kvq_store(h["fp8"], None, P, P, 4, None, None, None) == ARG
    assert lib.kvq_store(h["fp8"], P, None, P, 4, None, None, None) == ARG
    assert lib.kvq_store(h["fp8"], P, P, None, 4, None, None, None) == ARG
    assert lib.kvq_store(h["fp8"], c_void_p(FAKE_DEV + 2), P, P, 4, None, None, None) == ARG
    assert lib.kvq_store(h["fp8"], P, P, P, -1, None, None, None) == ARG
    assert lib.kvq_store(h["mla"], P, P, P, 4, P, None, None) == ARG            # MLA has no V input
    assert lib.kvq_store(h["mla"], P, None, P, 4, None, None, None) == ARG      # NVFP4 needs g
    assert lib.kvq_store(None, P, P, P, 4, None, None, None) == ARG
    # one launch covers at most 2^32 work-items: 2 KV heads x 8 pieces of 16 per token
    assert lib.kvq_store(h["fp8"], P, P, P, 2**31 - 1, None, None, None) == UNSUP


def test_compute_scale_argument_errors(handles):
    lib, h = handles
    P = c_void_p(FAKE_DEV)
    assert lib.kvq_compute_scale(h["mx"], P, 10, None, 0, P, None) == UNSUP
    assert lib.kvq_compute_scale(h["fp8"], None, 10, None, 0, P, None) == ARG
    assert lib.kvq_compute_scale(h["fp8"], P, 10, None, 5, P, None) == ARG
    assert lib.kvq_compute_scale(h["fp8"], P, 10, None, 0, None, None) == ARG
    assert lib.kvq_compute_scale(h["fp8"], P, -1, None, 0, P, None) == ARG


def test_decode_argument_errors(handles):
    lib, h = handles
    P = c_void_p(FAKE_DEV)
    args = lambda hq, stride, max_len, ws, wsb, batch=4: (
        h["fp8"], P, batch, hq, P, stride, P, max_len, 0.1, None, None, P, None, ws, wsb, None)
    assert lib.kvq_decode(*args(8, 4, 64, None, 0, batch=0)) == OK               # empty batch
    assert lib.kvq_decode(*args(7, 4, 64, None, 0)) == ARG                        # Hq % Hkv
    assert lib.kvq_decode(*args(34, 4, 64, None, 0)) == UNSUP                     # G = 17 > 16
    assert lib.kvq_decode(*args(8, 3, 64, None, 0)) == ARG                        # stride < ceil(64/16)
    need = lib.kvq_decode_workspace_bytes(h["fp8"], 4, 8, 200000)
    assert need > 0                                                               # long context -> splits
    assert lib.kvq_decode(*args(8, 12500, 200000, None, 0)) == SIZE
    assert lib.kvq_decode(*args(8, 12500, 200000, P, need - 1)) == SIZE
    assert lib.kvq_decode(*args(8, 12500, 200000, c_void_p(FAKE_DEV + 16), need)) == SIZE
    bad = list(args(8, 4, 64, None, 0))
    bad[1] = None
    assert lib.kvq_decode(*bad) == ARG
    # lengths past the 2,097,152-token cap are refused before the page count
    # ceil(max_len / P) is formed (near INT32_MAX that sum would overflow)
    assert lib.kvq_decode(*args(8, 1, 2**31 - 1, None, 0)) == UNSUP
    assert lib.kvq_decode(*args(8, 1, 2**21 + 1, None, 0)) == UNSUP
    assert lib.kvq_decode(*args(8, 2**17, 2**21, None, 0)) != UNSUP


def test_profile_entry_points_without_gpu():
    lib = _lib()
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.kvq_profile_enable(1) == OK
    assert lib.kvq_profile_read(b"decode", byref(ms), byref(n)) == OK and n.value == 0
    assert lib.kvq_profile_read(b"bogus", byref(ms), byref(n)) == ARG
    assert lib.kvq_profile_read(b"merge", None, byref(n)) == ARG
    assert lib.kvq_profile_enable(0) == OK


def test_mla_decode_argument_errors(handles):
    lib, h = handles
    P = c_void_p(FAKE_DEV)
    mla = lambda hq, ks, batch=2: (h["mla"], P, batch, hq, P, 16, P, 1000, 0.04, ks, None, P, None, None, 0, None)
    assert lib.kvq_decode(*mla(129, P)) == UNSUP         # at most 128 heads (one workgroup per split)
    assert lib.kvq_decode(*mla(0, P)) == ARG
    assert lib.kvq_decode(*mla(128, None)) == ARG        # the NVFP4 global scale is required
    assert lib.kvq_decode_workspace_bytes(h["mla"], 2, 129, 1000) == 0
    assert lib.kvq_decode_workspace_bytes(h["mla"], 2, 16, 1000) > 0


def test_split_plan_cap(handles):
    """Aimed at far more workgroups than one sequence has tiles, the planners
    stop at 128 splits: GQA 40,000 tokens = 2,500 tiles -> 157 splits of 16
    tiles, capped to 128, re-tiled at 20 tiles = 125 splits; MLA 8,192 tokens
    = 512 tiles -> 256 two-tile splits, capped to 128 of 4 tiles. The
    workspace is splits x (Dv + 1) floats per (sequence, head), each part
    rounded up to 256 bytes."""
    lib, h = handles
    for name in ("fp8", "mla"):
        assert lib.kvq_testing_set_split_target(h[name], 100000) == OK
    up = lambda x: (x + 255) // 256 * 256
    assert lib.kvq_decode_workspace_bytes(h["fp8"], 1, 8, 40000) == up(8 * 125 * 128 * 4) + up(8 * 125 * 4)
    assert lib.kvq_decode_workspace_bytes(h["mla"], 1, 16, 8192) == up(16 * 128 * 512 * 4) + up(16 * 128 * 4)
    for name in ("fp8", "mla"):
        assert lib.kvq_testing_set_split_target(h[name], 1) == OK
    # one split per sequence when it fits (no workspace); 1,024 tiles per GQA split at most
    assert lib.kvq_decode_workspace_bytes(h["fp8"], 1, 8, 16384) == 0
    assert lib.kvq_decode_workspace_bytes(h["fp8"], 1, 8, 40000) == up(8 * 3 * 128 * 4) + up(8 * 3 * 4)


def test_noalloc_decode_limit_and_errors(handles):
    """kvq_decode_noalloc refuses, before any device call, a shape whose split
    partials exceed its 80 MiB static workspace (KVQ_ERR_WORKSPACE), and
    otherwise validates like kvq_decode."""
    lib, h = handles
    P = c_void_p(FAKE_DEV)
    f = lib.kvq_decode_noalloc
    # MLA, 2,048 sequences x 128 heads x 2 splits x 512 floats = 1 GiB
    assert lib.kvq_decode_workspace_bytes(h["mla"], 2048, 128, 65536) > 80 << 20
    assert f(h["mla"], P, 2048, 128, P, 1024, P, 65536, 0.04, P, None, P, None, None) == -5
    # the DeepSeek-R1 shape (64 x 128 heads x 4 splits) fits: 64 MiB + 128 KiB
    assert lib.kvq_decode_workspace_bytes(h["mla"], 64, 128, 65536) <= 80 << 20
    assert f(h["fp8"], P, 0, 8, P, 4, P, 64, 0.1, None, None, P, None, None) == OK     # empty batch
    assert f(h["fp8"], P, 4, 7, P, 4, P, 64, 0.1, None, None, P, None, None) == ARG    # Hq % Hkv
    assert f(h["mla"], P, 2, 128, P, 16, P, 1000, 0.04, None, None, P, None, None) == ARG  # g required
    assert f(None, P, 4, 8, P, 4, P, 64, 0.1, None, None, P, None, None) == ARG
    assert b"static workspace" in lib.kvq_status_string(-5)


def test_decode_append_argument_errors(handles):
    lib, h = handles
    P = c_void_p(FAKE_DEV)
    tail = (P, 4, 8, P, 4, P, 64, 0.1, None, None, P, None, None, 0, None)
    assert lib.kvq_decode_append(h["fp8"], None, P, *tail) == ARG                  # k_new required
    assert lib.kvq_decode_append(h["fp8"], P, None, *tail) == ARG                  # GQA needs v_new
    assert lib.kvq_decode_append(h["fp8"], c_void_p(FAKE_DEV + 2), P, *tail) == ARG  # 16-byte aligned rows
    mla = (P, 2, 128, P, 16, P, 1000, 0.04, P, None, P, None, None, 0, None)
    assert lib.kvq_decode_append(h["mla"], P, P, *mla) == ARG                      # MLA has no V rows
    assert lib.kvq_decode_append(h["mla"], P, None, P, 2, 129, P, 16, P, 1000, 0.04, P, None, P, None, None, 0,
                                 None) == UNSUP
    assert lib.kvq_decode_append(h["fp8"], P, P, P, 0, 8, P, 4, P, 64, 0.1, None, None, P, None, None, 0,
                                 None) == OK                                       # empty batch


def test_per_head_scale_descriptor_rules():
    lib = _lib()
    need = c_size_t()
    d = _desc("e4m3")
    d.scale_mode = 1
    assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == OK
    for dtype, kind, args in (("mx16", "gqa", ()), ("nvfp4", "mla", (1, 576, 512, 64))):
        d = _desc(dtype, kind, *args)
        d.scale_mode = 1
        assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == UNSUP
    d = _desc("e4m3")
    d.scale_mode = -1
    assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == ARG


def test_per_head_compute_scale_shape_errors():
    lib = _lib()
    d = _desc("e4m3", hkv=4)
    d.scale_mode = 1
    need = c_size_t()
    h = c_void_p()
    assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == OK
    assert lib.kvq_alloc_pages(byref(d), c_void_p(FAKE_DEV), need.value, byref(need), byref(h)) == OK
    P = c_void_p(FAKE_DEV)
    assert lib.kvq_compute_scale(h, P, 4 * 128 + 1, None, 0, P, None) == ARG          # not whole rows
    assert lib.kvq_compute_scale(h, c_void_p(FAKE_DEV + 2), 4 * 128, None, 0, P, None) == ARG  # unaligned
    lib.kvq_free_handle(h)


def test_dequantize_prev_kv_argument_errors(handles):
    lib, h = handles
    P = c_void_p(FAKE_DEV)
    f = lib.kvq_dequantize_prev_kv
    assert f(h["fp8"], P, 4, None, None, None, P, P, None) == UNSUP               # FP4 caches only
    assert f(h["mx"], P, 0, None, None, None, None, None, None) == OK              # no pages: no-op
    assert f(h["mx"], P, -1, None, None, None, P, P, None) == ARG
    assert f(h["mx"], None, 4, None, None, None, P, P, None) == ARG               # page list required
    assert f(h["mx"], P, 4, None, None, None, None, P, None) == ARG               # dq_k required
    assert f(h["mx"], P, 4, None, None, None, P, None, None) == ARG               # GQA needs dq_v
    assert f(h["mx"], P, 4, None, None, None, c_void_p(FAKE_DEV + 8), P, None) == ARG  # 16-byte aligned
    assert f(h["mla"], P, 4, None, None, None, P, None, None) == ARG              # NVFP4 needs g
    assert f(h["mla"], P, 4, P, None, None, P, P, None) == ARG                    # MLA has no dq_v
    assert f(h["mla"], P, 4, P, None, P, P, None, None) == ARG                    # nor a V output scale
    assert f(None, P, 4, None, None, None, P, P, None) == ARG


def test_kivi_descriptor_layout_and_accounting():
    """KIVI-style caches: FP8 GQA only; no K scale buffer, one fp32 V scale
    per (page, kv head, token); 4 bytes per token-head in the accounting;
    the scratch holds one running max per (kv head, channel)."""
    lib = _lib()
    need = c_size_t()
    for dtype, kind, args in (("mx16", "gqa", ()), ("nvfp4", "mla", (1, 576, 512, 64))):
        d = _desc(dtype, kind, *args)
        d.scale_mode = 2
        assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == UNSUP
    d = _desc("e4m3", hkv=4, d=128, p=32, n=10)
    d.scale_mode = 3
    assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == ARG
    d.scale_mode = 2
    assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == OK
    h = c_void_p()
    assert lib.kvq_alloc_pages(byref(d), c_void_p(FAKE_DEV), need.value, byref(need), byref(h)) == OK
    L = Layout()
    assert lib.kvq_cache_layout(h, byref(L)) == OK
    assert L.k_scales_bytes == 0 and L.v_scales_bytes == 10 * 4 * 32 * 4
    assert L.scratch_bytes >= 4 * 128 * 4
    bpt = ctypes.c_double()
    assert lib.kvq_bytes_per_token(byref(d), byref(bpt)) == OK and bpt.value == 2 * 4 * 128 + 4 * 4
    P = c_void_p(FAKE_DEV)
    # K channel scales are required (and 16-byte aligned) for store and decode
    assert lib.kvq_store(h, P, P, P, 4, None, None, None) == ARG
    assert lib.kvq_store(h, P, P, P, 4, c_void_p(FAKE_DEV + 4), None, None) == ARG
    dec = lambda ks: lib.kvq_decode(h, P, 2, 8, P, 4, P, 64, 0.1, ks, None, P, None, None, 0, None)
    assert dec(None) == ARG and dec(c_void_p(FAKE_DEV + 4)) == ARG
    assert lib.kvq_compute_scale(h, P, 4 * 128 + 8, None, 0, P, None) == ARG     # whole rows only
    lib.kvq_free_handle(h)


def test_extend_attention_argument_errors():
    lib = _lib()
    P = c_void_p(FAKE_DEV)
    f = lib.kvq_extend_attention

    def call(q=P, total_q=64, batch=2, hq=32, hkv=2, d=128, page=16, max_chunk=32, npg=10, dq=P, out=P):
        return f(q, P, P, P, total_q, P, dq, dq, P, npg, None, None, batch, hq, hkv, d, page, max_chunk, 0.1,
                 out, None, None)
    assert call(batch=0) == OK and call(total_q=0) == OK and call(max_chunk=0) == OK      # no-ops
    assert call(d=64) == UNSUP                                   # head_dim 128 only
    assert call(hq=48, hkv=2) == UNSUP                           # G = 24
    assert call(hq=6, hkv=2) == UNSUP                            # G = 3: 256 rows / G not whole tokens
    assert call(hq=33, hkv=2) == ARG                             # Hq % Hkv
    assert call(q=None) == ARG and call(out=None) == ARG
    assert call(q=c_void_p(FAKE_DEV + 2)) == ARG                 # 16-byte alignment
    assert call(dq=None) == ARG                                  # pages but no workspace
    assert call(batch=-1) == ARG and call(page=0) == ARG and call(max_chunk=-1) == ARG


def test_fp8q_decode_and_q_scale_argument_errors(handles):
    """FP8-domain decode: FP8 GQA caches with tensor or per-head scales and the
    NVFP4 MLA latent only; q_scale 4-byte aligned; kvq_compute_q_scale's
    argument checks."""
    lib, h = handles
    P = c_void_p(FAKE_DEV)

    def dec(cache, qs=None, batch=4, hq=8):
        return lib.kvq_decode_fp8q(cache, P, batch, hq, P, 4, P, 64, 0.1, qs, None, None, P, None, None, 0, None)
    assert dec(h["mx"]) == UNSUP                                                 # codes are not FP8
    assert dec(h["mla"], hq=128) == ARG                                          # MLA: g required
    assert dec(h["mla"], hq=129) == UNSUP
    assert dec(h["fp8"], qs=c_void_p(FAKE_DEV + 2)) == ARG                       # misaligned q_scale
    assert dec(h["fp8"], batch=0) == OK                                          # empty batch
    assert dec(h["fp8"], hq=7) == ARG                                            # as kvq_decode
    app = lambda cache, k, v: lib.kvq_decode_append_fp8q(cache, k, v, P, 4, 8, P, 4, P, 64, 0.1, None, None, None,
                                                         P, None, None, 0, None)
    assert app(h["fp8"], None, P) == ARG and app(h["fp8"], P, None) == ARG and app(h["mx"], P, P) == UNSUP
    q = lib.kvq_compute_q_scale
    assert q(h["mx"], P, 4, 8, P, None) == UNSUP
    assert q(h["mla"], c_void_p(FAKE_DEV + 2), 4, 8, P, None) == ARG             # MLA served: past UNSUP
    assert q(h["fp8"], P, 4, 8, None, None) == ARG                               # no output
    assert q(h["fp8"], P, -1, 8, P, None) == ARG
    assert q(h["fp8"], P, 4, 7, P, None) == ARG                                  # Hq % Hkv
    assert q(h["fp8"], None, 4, 8, P, None) == ARG and q(h["fp8"], c_void_p(FAKE_DEV + 2), 4, 8, P, None) == ARG
    # KIVI caches fold a channel scale into the query: not an FP8-domain case
    d = _desc("e4m3", hkv=2)
    d.scale_mode = 2
    need = c_size_t()
    hk = c_void_p()
    assert lib.kvq_alloc_pages(byref(d), None, 0, byref(need), None) == OK
    assert lib.kvq_alloc_pages(byref(d), c_void_p(FAKE_DEV), need.value, byref(need), byref(hk)) == OK
    assert dec(hk) == UNSUP and q(hk, P, 4, 8, P, None) == UNSUP
    lib.kvq_free_handle(hk)
