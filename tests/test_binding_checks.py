"""The Python binding refuses bad tensor arguments before anything reaches
the C ABI (which sees raw pointers only, so a tensor on the wrong device or
one too small would otherwise become a GPU memory fault). Runs without a GPU:
the cache is bound to host memory, every bad argument must raise ValueError
naming it, and a call whose arguments are all good still stops at the
GPU-memory check instead of launching anything."""
import pytest
import torch

import quantized_paged_kv_store_amd as K
from quantized_paged_kv_store_amd import kvq

B, HQ, HKV, D, P, NP = 2, 8, 2, 128, 16, 8


def _lib_or_skip():
    import os
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")


def _host_cache(dtype="e4m3", kind="gqa", hkv=HKV, d=D, dv=D, p=P, scale_mode=None):
    _lib_or_skip()
    desc = K.make_desc(dtype, kind, hkv, d, dv, p, NP, scale_mode=scale_mode)
    need = kvq.c_size_t()
    assert K.library().kvq_alloc_pages(kvq.byref(desc), None, 0, kvq.byref(need), None) == 0
    raw = torch.zeros(need.value + 256, dtype=torch.uint8)
    off = (-raw.data_ptr()) % 256
    return kvq.Cache(desc, raw[off:off + need.value])


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def _i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def _f32(*shape):
    return torch.ones(shape, dtype=torch.float32)


def _raises(what, fn, *args, **kw):
    with pytest.raises(ValueError, match=what):
        fn(*args, **kw)


def _decode_args(**over):
    a = dict(q=_bf(B, HQ, D), page_table=_i32(B, 4), seq_lens=_i32(B), max_seq_len=64, sm_scale=0.1)
    a.update(over)
    return a


def test_decode_arguments():
    c = _host_cache()
    dec = lambda **o: K.kvq_decode(c, **_decode_args(**o))
    _raises("q: head dim", dec, q=_bf(B, HQ, 64))
    _raises("q: dtype", dec, q=torch.zeros(B, HQ, D, dtype=torch.float16))
    _raises("q: 2 dimensions", dec, q=_bf(B, HQ * D))
    _raises("q: not contiguous", dec, q=_bf(B, D, HQ).transpose(1, 2))
    _raises("q: on meta", dec, q=torch.zeros(B, HQ, D, dtype=torch.bfloat16, device="meta"))
    _raises("page_table: 1 rows", dec, page_table=_i32(1, 4))
    _raises("page_table: dtype", dec, page_table=torch.zeros(B, 4, dtype=torch.int64))
    _raises("page_table: on meta", dec, page_table=torch.zeros(B, 4, dtype=torch.int32, device="meta"))
    _raises("seq_lens: 3 elements", dec, seq_lens=_i32(B + 1))
    _raises("seq_lens: on meta", dec, seq_lens=torch.zeros(B, dtype=torch.int32, device="meta"))
    _raises("out: shape", dec, out=torch.zeros(B, HQ, 64))
    _raises("out: dtype", dec, out=torch.zeros(B, HQ, D, dtype=torch.float16))
    _raises("lse: shape", dec, lse=torch.zeros(B, HQ + 1))
    _raises("max_seq_len", dec, max_seq_len=-1)
    _raises("scale: dtype", dec, k_scale=torch.ones(1, dtype=torch.float64))
    _raises("scale: on meta", dec, v_scale=torch.ones(1, device="meta"))
    # all arguments good: stopped at the GPU-memory check, not at a launch
    _raises("need GPU memory", dec)


def test_decode_workspace_arguments():
    c = _host_cache()
    long = dict(page_table=_i32(B, 12500), max_seq_len=200000)
    need = K.kvq_decode_workspace_bytes(c, B, HQ, 200000)
    assert need > 0
    dec = lambda **o: K.kvq_decode(c, **_decode_args(**long, **o))
    _raises("workspace: .* at least", dec, workspace=torch.zeros(need - 1, dtype=torch.uint8))
    _raises("workspace: dtype", dec, workspace=torch.zeros(need, dtype=torch.int8))
    _raises("workspace: on meta", dec, workspace=torch.zeros(need, dtype=torch.uint8, device="meta"))
    _raises("need GPU memory", dec, workspace=torch.zeros(need, dtype=torch.uint8))


def test_append_and_fp8q_arguments():
    c = _host_cache()
    app = lambda k_new, v_new, **o: K.kvq_decode_append(c, k_new, v_new, **_decode_args(**o))
    _raises("k_new: 2048 elements, expected 512", app, _bf(B, HKV, D * 4), _bf(B, HKV, D))
    _raises("v_new: expected a tensor", app, _bf(B, HKV, D), None)
    _raises("v_new: dtype", app, _bf(B, HKV, D), torch.zeros(B, HKV, D))
    _raises("need GPU memory", app, _bf(B, HKV, D), _bf(B, HKV, D))
    f8 = lambda **o: K.kvq_decode_fp8q(c, **_decode_args(**o))
    _raises("scale: 0 elements", f8, q_scale=torch.ones(0))
    _raises("need GPU memory", f8, q_scale=_f32(1))
    f8a = lambda **o: K.kvq_decode_append_fp8q(c, _bf(B, HKV, D), _bf(B, HKV, D - 1), **_decode_args(**o))
    _raises("v_new: 508 elements", f8a)


def test_mla_arguments():
    c = _host_cache("nvfp4", "mla", 1, 576, 512, 64)
    a = dict(q=_bf(B, 128, 576), page_table=_i32(B, 4), seq_lens=_i32(B), max_seq_len=200, sm_scale=0.04,
             k_scale=_f32(1))
    dec = lambda **o: K.kvq_decode(c, **{**a, **o})
    _raises("out: shape", dec, out=torch.zeros(B, 128, 576))
    _raises("q: head dim 512", dec, q=_bf(B, 128, 512))
    _raises("need GPU memory", dec)
    _raises("v_new: an MLA cache", K.kvq_decode_append, c, _bf(B, 576), _bf(B, 576), **a)
    _raises("k_new: 576 elements", K.kvq_decode_append, c, _bf(1, 576), None, **a)
    slots = torch.zeros(3, dtype=torch.int64)
    _raises("v: an MLA cache", K.kvq_store, c, _bf(3, 576), _bf(3, 576), slots, _f32(1))
    _raises("k: 1152 elements", K.kvq_store, c, _bf(2, 576), None, slots, _f32(1))


def test_store_and_scale_arguments():
    c = _host_cache()
    slots = torch.zeros(5, dtype=torch.int64)
    _raises("k: .* expected 1280", K.kvq_store, c, _bf(4, HKV, D), _bf(5, HKV, D), slots)
    _raises("v: expected a tensor", K.kvq_store, c, _bf(5, HKV, D), None, slots)
    _raises("slot_mapping: dtype", K.kvq_store, c, _bf(5, HKV, D), _bf(5, HKV, D), slots.int())
    _raises("slot_mapping: 2 dimensions", K.kvq_store, c, _bf(5, HKV, D), _bf(5, HKV, D), slots.view(5, 1))
    _raises("need GPU memory", K.kvq_store, c, _bf(5, HKV, D), _bf(5, HKV, D), slots, _f32(1), _f32(1))
    _raises("x0: dtype", K.kvq_compute_scale, c, torch.zeros(10))
    _raises("x1: on meta", K.kvq_compute_scale, c, _bf(10), torch.zeros(10, dtype=torch.bfloat16, device="meta"))
    _raises("out: 0 elements", K.kvq_compute_scale, c, _bf(10), out=torch.zeros(0))
    _raises("need GPU memory", K.kvq_compute_scale, c, _bf(10))
    h = _host_cache(scale_mode="head")
    _raises("out: 1 elements, at least 8", K.kvq_compute_q_scale, h, _bf(3, HQ, D), out=torch.zeros(1))
    _raises("q: head dim 64", K.kvq_compute_q_scale, h, _bf(3, HQ, 64))
    k = _host_cache(scale_mode="kivi")
    _raises("scale: 1 elements, at least 256", K.kvq_store, k, _bf(5, HKV, D), _bf(5, HKV, D), slots, _f32(1))


def test_dequant_prev_and_extend_arguments():
    c = _host_cache("mx16")
    pages = torch.zeros(3, dtype=torch.int32)
    _raises("pages: dtype", K.kvq_dequantize_prev_kv, c, pages.long())
    small = torch.zeros(3 * HKV * P * D - 1, dtype=torch.uint8)
    _raises("dq_k: .* at least", K.kvq_dequantize_prev_kv, c, pages, dq_k=small)
    _raises("dq_v: .* at least", K.kvq_dequantize_prev_kv, c, pages,
            dq_k=torch.zeros(3 * HKV * P * D, dtype=torch.uint8), dq_v=small)
    _raises("need GPU memory", K.kvq_dequantize_prev_kv, c, pages)
    m = _host_cache("nvfp4", "mla", 1, 576, 512, 64)
    _raises("dq_v: an MLA cache", K.kvq_dequantize_prev_kv, m, pages, g=_f32(1),
            dq_v=torch.zeros(10, dtype=torch.uint8))

    nq, nb, npg = 40, 2, 6
    ext = dict(q=_bf(nq, HQ, D), k_new=_bf(nq, HKV, D), v_new=_bf(nq, HKV, D), cu_q=_i32(nb + 1),
               prefix_len=_i32(nb), dq_k=torch.zeros(npg, HKV, P, D, dtype=torch.uint8),
               dq_v=torch.zeros(npg, HKV, P, D, dtype=torch.uint8), page_off=_i32(nb), s_k=None, s_v=None,
               max_chunk=20, sm_scale=0.1)
    f = lambda **o: K.kvq_extend_attention(**{**ext, **o})
    _raises("k_new: shape", f, k_new=_bf(nq - 1, HKV, D))
    _raises("v_new: shape", f, v_new=_bf(nq, HKV + 1, D))
    _raises("cu_q: 2 elements", f, cu_q=_i32(nb))
    _raises("page_off: 3 elements", f, page_off=_i32(nb + 1))
    _raises("dq_v: shape", f, dq_v=torch.zeros(npg, HKV, P, D - 16, dtype=torch.uint8))
    _raises("dq_k: 3 dimensions", f, dq_k=torch.zeros(npg, HKV, P * D, dtype=torch.uint8))
    _raises("out: shape", f, out=torch.zeros(nq, HQ, 64))
    _raises("lse: dtype", f, lse=torch.zeros(nq, HQ, dtype=torch.float64))
    _raises("need GPU memory", f)


def test_split_target_hook_is_per_handle():
    """The planner target lives in the handle: the workspace query follows it
    on that cache only, and 0 restores the default."""
    a, b = _host_cache(), _host_cache()
    base = K.kvq_decode_workspace_bytes(a, B, HQ, 200000)
    with K.split_target(a, 1):
        one = K.kvq_decode_workspace_bytes(a, B, HQ, 200000)
        assert K.kvq_decode_workspace_bytes(b, B, HQ, 200000) == base
    assert one != base and K.kvq_decode_workspace_bytes(a, B, HQ, 200000) == base
    lib = K.library()
    assert lib.kvq_testing_set_split_target(a.handle, -1) == -1
    assert lib.kvq_testing_set_split_target(a.handle, (1 << 20) + 1) == -1
    assert lib.kvq_testing_set_split_target(None, 4) == -1
