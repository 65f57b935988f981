"""Full-size parity on the larger workloads, in the launch configuration the
benchmark uses: codes/scales of sampled sequences compared byte for byte,
decode outputs of sampled sequences within max-abs 4e-3 / rel-L2 1e-3 of the
float64 oracle. The quantization error against unquantized BF16 attention is
printed as information."""
import numpy as np
import pytest
import torch

import quantized_paged_kv_store_amd as K
from oracle.attention import extend_attention
from oracle.paged import dequantize_prev_kv
from quantized_paged_kv_store_amd import inputs as I
from tests.kvq_cases import Case, assert_close, rel_l2

pytestmark = pytest.mark.gpu


def _check_case(c, ids, what):
    oc, otable, pages, _ = c.oracle(ids)
    c.oracle_table = otable
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        want = getattr(oc, name)
        if want is not None:
            assert np.array_equal(c.gpu_pages(name, pages), want), f"{what}: {name} differ"
    want, wlse, _, _ = c.oracle_decode(ids)
    got = c.out.cpu().numpy()
    mab, r = assert_close(got[ids], want[ids], what)
    assert np.allclose(c.lse.cpu().numpy()[ids], wlse[ids], rtol=0, atol=1e-4), what
    q = rel_l2(got[ids[0]], c.unquantized(ids[0]))
    print(f"{what}: max-abs {mab:.2e} rel-L2 {r:.2e}; quantization error vs BF16 attention rel-L2 {q:.3e}")
    return oc, pages


def _check_dequant_prev(c, oc, pages, what, ks=0.02, vs=0.01, sample=96):
    """kvq_dequantize_prev_kv over every page of the pool (the benchmark's
    launch); a seeded sample of the oracle-covered pages compared byte for byte."""
    mla = c.w.kind == "mla"
    dk, dv = K.kvq_dequantize_prev_kv(c.cache, torch.arange(c.npages, dtype=torch.int32, device=c.dev), ks,
                                      None if mla else vs, g=c.k_scale if mla else None)
    pick = np.sort(np.random.default_rng(7).choice(len(pages), size=min(sample, len(pages)), replace=False))
    wk, wv = dequantize_prev_kv(oc, pick, ks, None if mla else vs, g=c.oracle_scales()[0] if mla else None)
    idx = torch.from_numpy(pages[pick]).to(c.dev)
    assert np.array_equal(dk.index_select(0, idx).cpu().numpy(), wk), f"{what}: dq_k differ"
    if not mla:
        assert np.array_equal(dv.index_select(0, idx).cpu().numpy(), wv), f"{what}: dq_v differ"


def test_llama3_70b_share_fp8_variants():
    """Batch 32, 64/8 heads, lengths U[16K, 32K]; E4M3 and E5M2, each with
    scale 1.0 and with the calibrated amax scale."""
    base = I.WORKLOADS["llama3_70b"]
    data = None
    lens = I.seq_lens(base)
    ids = [int(np.argmin(lens)), int(np.argmax(lens))]
    for dtype in ("e4m3", "e5m2"):
        for mode in ("amax", "one"):
            c = Case(base.with_(dtype=dtype, scale_mode=mode), data=data).run_gpu()
            data = c.data
            _check_case(c, ids, f"llama3_70b {dtype} scale={mode}")
            del c


def _check_extend_step(c, oc, ids, rows=(0, 1, 777, 2047), s=0.05):
    """The chunked-prefill step as the benchmark launches it: every
    sequence's prefix pages through kvq_dequantize_prev_kv (scales 0.05), then
    kvq_extend_attention of all 64 chunks over prefix + chunk. For sequences
    `ids`: their workspace pages byte for byte against the oracle's
    dequantize_prev_kv, and sampled chunk rows against the oracle's extend
    attention fed the oracle's own workspace."""
    w = c.w
    C, P = w.new_tokens, w.page_size
    prefix = (c.lens - C).astype(np.int32)
    npg = (prefix + P - 1) // P
    pages = np.concatenate([c.table[b, :npg[b]] for b in range(w.batch)]).astype(np.int32)
    page_off = np.concatenate([[0], np.cumsum(npg)[:-1]]).astype(np.int32)
    st = torch.tensor([s], dtype=torch.float32, device=c.dev)
    dk, dv = K.kvq_dequantize_prev_kv(c.cache, torch.from_numpy(pages).to(c.dev), st, st)
    kn_d, vn_d, _ = c.new_dev
    nq = w.batch * C
    gen = torch.Generator(device=c.dev)
    gen.manual_seed(w.seed)
    q = torch.randn((nq, w.q_heads, w.head_dim), generator=gen, device=c.dev).to(torch.bfloat16)
    cu = torch.arange(0, nq + 1, C, dtype=torch.int32, device=c.dev)
    out, lse = K.kvq_extend_attention(q, kn_d, vn_d, cu, torch.from_numpy(prefix).to(c.dev), dk, dv,
                                      torch.from_numpy(page_off).to(c.dev), st, st, C, I.sm_scale(w))
    torch.cuda.synchronize()
    # the oracle's workspace for the sampled sequences, from its own cache
    opages = np.concatenate([c.oracle_table[b, :npg[b]] for b in ids])
    wk, wv = dequantize_prev_kv(oc, opages, np.float32(s), np.float32(s))
    o_off = np.concatenate([[0], np.cumsum([npg[b] for b in ids])[:-1]]).astype(np.int64)
    for k, b in enumerate(ids):
        sl = slice(int(page_off[b]), int(page_off[b] + npg[b]))
        ol = slice(int(o_off[k]), int(o_off[k] + npg[b]))
        assert np.array_equal(dk[sl].cpu().numpy(), wk[ol]) and np.array_equal(dv[sl].cpu().numpy(), wv[ol]), b
    kn, vn, _ = c.data["new"]
    f = lambda a: I.bf16_to_f32(a).astype(np.float64)
    qs = np.concatenate([q[b * C:(b + 1) * C].float().cpu().numpy() for b in ids]).astype(np.float64)
    kns = np.concatenate([f(kn[b * C:(b + 1) * C]) for b in ids]).reshape(len(ids) * C, w.kv_heads, w.head_dim)
    vns = np.concatenate([f(vn[b * C:(b + 1) * C]) for b in ids]).reshape(len(ids) * C, w.kv_heads, w.head_dim)
    cu_s = np.arange(0, len(ids) * C + 1, C)
    sel = [k * C + r for k in range(len(ids)) for r in rows]
    want, wlse = extend_attention(qs, kns, vns, cu_s, prefix[ids], wk, wv, o_off, np.float32(s), np.float32(s),
                                  I.sm_scale(w), rows=sel)
    gsel = [b * C + r for b in ids for r in rows]
    assert_close(out[gsel].cpu().numpy(), want[sel], "qwen3_235b extend step")
    assert np.allclose(lse[gsel].cpu().numpy(), wlse[sel], rtol=0, atol=1e-4)


def test_qwen3_235b_fp4_chunk_store_and_decode():
    """Batch 64, 64/4 heads, context 32,768, FP4 block-16: the last 2,048
    tokens of every sequence go through the chunk store, then decode; then the
    same cache serves the chunked-prefill step (dequantize_prev_kv of the
    30,720-token prefixes + extend attention of the 2,048-token chunks)."""
    c = Case(I.WORKLOADS["qwen3_235b"]).run_gpu()
    oc, pages = _check_case(c, [0, 63], "qwen3_235b mx16")
    _check_dequant_prev(c, oc, pages, "qwen3_235b dequantize_prev_kv")
    _check_extend_step(c, oc, [0, 63])


def test_dsr1_mla_nvfp4_sampled():
    """Batch 64, 128 heads over one 576-element latent, context 65,536, page
    64, NVFP4 with a computed global scale; oracle on sequences 0 and 63."""
    c = Case(I.WORKLOADS["dsr1_mla"]).run_gpu()
    oc, pages = _check_case(c, [0, 63], "dsr1_mla nvfp4")
    _check_dequant_prev(c, oc, pages, "dsr1_mla dequantize_prev_kv")
