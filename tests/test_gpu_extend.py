"""GPU parity of kvq_extend_attention (extend attention over a quantized
prefix read through E4M3 workspaces; PR #21954 analysis page, "code
analysis") against oracle.attention.extend_attention: outputs within max-abs
4e-3 / rel-L2 1e-3 of the float64 oracle fed the same codes and BF16 values,
LSE within 1e-4. Also the whole chain on an FP4 cache: kvq_store ->
kvq_dequantize_prev_kv -> kvq_extend_attention against the oracle's store,
dequantize_prev_kv and extend attention."""
import numpy as np
import pytest
import torch

import quantized_paged_kv_store_amd as K
from oracle import quantize as Q
from oracle.attention import extend_attention
from oracle.paged import CacheSpec, OracleCache, dequantize_prev_kv
from quantized_paged_kv_store_amd import inputs as I
from tests.kvq_cases import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(inp, hkv, s_k, s_v, sm, max_chunk=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    bf = lambda a: t(a).view(torch.bfloat16)
    cl = np.diff(inp["cu_q"])
    out, lse = K.kvq_extend_attention(bf(inp["q"]), bf(inp["k_new"]), bf(inp["v_new"]), t(inp["cu_q"]),
                                      t(inp["prefix_len"]), t(inp["dq_k"]), t(inp["dq_v"]), t(inp["page_off"]),
                                      s_k, s_v, int(cl.max()) if max_chunk is None else max_chunk, sm)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _oracle(inp, s_k, s_v, sm, rows=None):
    f = lambda a: I.bf16_to_f32(a).astype(np.float64)
    return extend_attention(f(inp["q"]), f(inp["k_new"]), f(inp["v_new"]), inp["cu_q"], inp["prefix_len"],
                            inp["dq_k"], inp["dq_v"], inp["page_off"], s_k, s_v, sm, rows=rows)


@pytest.mark.parametrize("G,P,prefix,chunk", [
    (16, 16, [0, 1, 63, 64, 65, 300], [1, 7, 8, 9, 64, 130]),
    (8, 32, [100, 0, 257], [33, 16, 17]),
    (4, 16, [500, 31], [40, 3]),
    (1, 16, [70, 129], [129, 5]),
    (1, 32, [40, 0], [300, 513]),      # G = 1: 256 chunk tokens per tile, so these span 2 and 3 tiles
    (2, 64, [64, 640], [200, 1]),
    (4, 48, [100, 0, 257], [33, 16, 17]),   # workspace pages that are not a power of two in size
    (16, 80, [300, 65], [64, 9]),
])
def test_extend_matches_oracle(G, P, prefix, chunk):
    hkv, D = 2, 128
    inp = I.extend_inputs(len(prefix) * 10 + G, prefix, chunk, hkv, G, D, P)
    s_k, s_v, sm = np.float32(0.0625), np.float32(0.03125), 1.0 / np.sqrt(D)
    got, glse = _run(inp, hkv, s_k, s_v, sm)
    want, wlse = _oracle(inp, s_k, s_v, sm)
    assert_close(got, want, f"extend G{G} P{P}")
    assert np.allclose(glse, wlse, rtol=0, atol=1e-4)


def test_extend_scales_default_and_larger_bound():
    """NULL workspace scales mean 1.0; max_chunk larger than every chunk only
    adds empty tiles."""
    inp = I.extend_inputs(5, [90, 20], [50, 12], 1, 4, 128, 16, max_code=0x40)
    got, glse = _run(inp, 1, None, None, 0.05, max_chunk=300)
    want, wlse = _oracle(inp, None, None, 0.05)
    assert_close(got, want, "extend default scales")
    assert np.allclose(glse, wlse, rtol=0, atol=1e-4)


def test_extend_out_of_range_device_data_is_clamped():
    """Prefix pages beyond the workspace are dropped and chunk offsets past
    total_q are clamped, without touching memory outside the inputs."""
    inp = I.extend_inputs(6, [40, 30], [10, 6], 1, 8, 128, 16)
    n_pages = inp["dq_k"].shape[0]
    inp2 = dict(inp)
    inp2["page_off"] = inp["page_off"].copy()
    inp2["page_off"][1] = n_pages + 5                       # sequence 1's prefix is not in the workspace
    got, _ = _run(inp2, 1, 0.1, 0.1, 0.09)
    ref = dict(inp)
    ref["prefix_len"] = np.array([40, 0], np.int32)
    want, _ = _oracle(ref, 0.1, 0.1, 0.09)
    assert_close(got, want, "extend clamped page_off")


def test_extend_after_dequantize_prev_kv_on_an_fp4_cache():
    """The whole chain on an MX16 cache: the prefix is stored FP4, turned into
    E4M3 rows by kvq_dequantize_prev_kv, and the chunk attends to it."""
    w = I.Workload("extend-chain", "mx16", "gqa", 3, 32, 2, 128, 128, 16, 400, 0, 1, "qwen", seed=55)
    prefix = np.array([0, 100, 380], np.int32)
    chunk = np.array([20, 9, 20], np.int32)
    P, D, hkv, G = 16, 128, 2, 16
    npg = (prefix + P - 1) // P
    pages = np.arange(int(npg.sum()), dtype=np.int32)[::-1].copy()   # any physical page order
    page_off = np.concatenate([[0], np.cumsum(npg)[:-1]]).astype(np.int32)
    cache = K.kvq_alloc_pages("mx16", "gqa", hkv, D, D, P, int(npg.sum()) + 1, device=DEV, fill=0)
    oc = OracleCache(CacheSpec("mx16", "gqa", hkv, D, D, P, int(npg.sum()) + 1))
    kr, vr, slots = [], [], []
    for b in range(3):
        if prefix[b] == 0:
            continue
        k, v = I.kv_rows(w, b, 0, int(prefix[b]))
        t = np.arange(prefix[b])
        kr.append(k)
        vr.append(v)
        slots.append(pages[page_off[b] + t // P].astype(np.int64) * P + t % P)
    kb, vb, sl = np.concatenate(kr), np.concatenate(vr), np.concatenate(slots)
    K.kvq_store(cache, torch.from_numpy(kb).to(DEV).view(torch.bfloat16),
                torch.from_numpy(vb).to(DEV).view(torch.bfloat16), torch.from_numpy(sl).to(DEV))
    oc.store(I.bf16_to_f32(kb), I.bf16_to_f32(vb), sl)
    s_k, s_v = np.float32(0.02), np.float32(0.01)
    dk, dv = K.kvq_dequantize_prev_kv(cache, torch.from_numpy(pages).to(DEV), s_k, s_v)
    wk, wv = dequantize_prev_kv(oc, pages, s_k, s_v)
    assert np.array_equal(dk.cpu().numpy(), wk) and np.array_equal(dv.cpu().numpy(), wv)
    rng = np.random.default_rng(56)
    cu = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    nq = int(cu[-1])
    q = I.bf16_bits(rng.standard_normal((nq, hkv * G, D), dtype=np.float32))
    kn = I.bf16_bits(rng.standard_normal((nq, hkv, D), dtype=np.float32))
    vn = I.bf16_bits(rng.standard_normal((nq, hkv, D), dtype=np.float32))
    inp = dict(q=q, k_new=kn, v_new=vn, cu_q=cu, prefix_len=prefix, page_off=page_off, dq_k=wk, dq_v=wv)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out, lse = K.kvq_extend_attention(t(q).view(torch.bfloat16), t(kn).view(torch.bfloat16),
                                      t(vn).view(torch.bfloat16), t(cu), t(prefix), dk, dv, t(page_off), s_k, s_v,
                                      int(chunk.max()), 1 / np.sqrt(D))
    want, wlse = _oracle(inp, s_k, s_v, 1 / np.sqrt(D))
    assert_close(out.cpu().numpy(), want, "extend chain")
    assert np.allclose(lse.cpu().numpy(), wlse, rtol=0, atol=1e-4)
