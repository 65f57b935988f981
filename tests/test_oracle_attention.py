"""Pins for oracle/attention.py: textbook special cases, a library
cross-check against torch's scaled_dot_product_attention (float64, CPU), page
permutation invariance, and scipy's logsumexp for the LSE."""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import quantize as Q
from oracle.attention import decode_attention, softmax_attention
from oracle.paged import CacheSpec, OracleCache
from quantized_paged_kv_store_amd import inputs as I


def _filled_cache(dtype, B, Hkv, D, P, L, seed, identity=False):
    w = I.Workload("t", dtype, "gqa", B, 4 * Hkv, Hkv, D, D, P, L, L, 1, "llama", seed=seed)
    lens = I.seq_lens(w)
    table, npages = I.page_table(w, lens, identity=identity)
    spec = CacheSpec(dtype, "gqa", Hkv, D, D, P, npages)
    cache = OracleCache(spec)
    ks, vs = [], []
    for b in range(B):
        k, v = I.kv_rows(w, b, 0, L)
        ks.append(I.bf16_to_f32(k)); vs.append(I.bf16_to_f32(v))
        cache.store(I.bf16_to_f32(k), I.bf16_to_f32(v), I.slots_for(table[b], np.arange(L), P),
                    k_scale=np.float32(0.05), v_scale=np.float32(0.03))
    q = I.bf16_to_f32(I.queries(w))
    return w, cache, table, lens, q


def test_single_token_returns_its_value_row():
    w, cache, table, lens, q = _filled_cache("e4m3", 1, 1, 64, 16, 1, 1)
    out, lse = decode_attention(cache, q, table, lens, 0.125, np.float32(0.05), np.float32(0.03))
    vhat = cache.dequant(table[0, 0], 0, 0, "v", np.float32(0.05), np.float32(0.03))[0]
    khat = cache.dequant(table[0, 0], 0, 0, "k", np.float32(0.05), np.float32(0.03))[0]
    assert np.allclose(out[0], vhat[None, :], rtol=0, atol=0)
    assert np.allclose(lse[0], 0.125 * q[0] @ khat, rtol=1e-14)


def test_zero_query_gives_mean_of_values():
    w, cache, table, lens, q = _filled_cache("e5m2", 1, 2, 128, 16, 77, 2)
    out, _ = decode_attention(cache, np.zeros_like(q), table, lens, 0.1, np.float32(0.05), np.float32(0.03))
    page, t = table[0][np.arange(77) // 16], np.arange(77) % 16
    for h in range(2):
        mean = cache.dequant(page, t, h, "v", np.float32(0.05), np.float32(0.03)).mean(axis=0)
        assert np.allclose(out[0, 4 * h:4 * h + 4], mean[None, :], rtol=1e-13, atol=1e-15)


def test_empty_sequence():
    out, lse = softmax_attention(np.ones((3, 8)), np.zeros((0, 8)), np.zeros((0, 8)), 1.0)
    assert np.all(out == 0) and np.all(lse == -np.inf)


@pytest.mark.parametrize("dtype", ["e4m3", "mx16"])
def test_matches_torch_sdpa_fp64(dtype):
    B, Hkv, D, P, L = 2, 2, 128, 16, 300
    w, cache, table, lens, q = _filled_cache(dtype, B, Hkv, D, P, L, 3)
    ksc, vsc = (np.float32(0.05), np.float32(0.03)) if dtype == "e4m3" else (None, None)
    out, lse = decode_attention(cache, q, table, lens, 0.0883883, ksc, vsc)
    G = w.group
    for b in range(B):
        page, t = table[b][np.arange(L) // P], np.arange(L) % P
        K = np.stack([cache.dequant(page, t, h, "k", ksc, vsc) for h in range(Hkv)])    # [Hkv, L, D]
        V = np.stack([cache.dequant(page, t, h, "v", ksc, vsc) for h in range(Hkv)])
        Kt = torch.from_numpy(K).repeat_interleave(G, 0)[None]
        Vt = torch.from_numpy(V).repeat_interleave(G, 0)[None]
        qt = torch.from_numpy(q[b].astype(np.float64))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=0.0883883)[0, :, 0].numpy()
        assert np.allclose(out[b], ref, rtol=1e-12, atol=1e-13)
        s = 0.0883883 * np.einsum("hd,hld->hl", q[b].astype(np.float64), np.repeat(K, G, 0))
        assert np.allclose(lse[b], logsumexp(s, axis=1), rtol=1e-13)


def test_page_permutation_invariance():
    a = _filled_cache("e4m3", 2, 1, 64, 16, 100, 4, identity=True)
    b = _filled_cache("e4m3", 2, 1, 64, 16, 100, 4, identity=False)
    assert not np.array_equal(a[2], b[2])
    oa, la = decode_attention(a[1], a[4], a[2], a[3], 0.125, np.float32(0.05), np.float32(0.03))
    ob, lb = decode_attention(b[1], b[4], b[2], b[3], 0.125, np.float32(0.05), np.float32(0.03))
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_mla_value_is_latent_prefix():
    rng = np.random.default_rng(5)
    spec = CacheSpec("nvfp4", "mla", 1, 576, 512, 64, 2)
    cache = OracleCache(spec)
    lat = rng.standard_normal((100, 576)).astype(np.float32).astype(np.float64)
    g = Q.nvfp4_global_scale(np.abs(lat).max())
    cache.store(lat, None, np.arange(100), k_scale=g)
    q = rng.standard_normal((1, 8, 576))
    out, _ = decode_attention(cache, q, np.array([[0, 1]]), np.array([100]), 1 / 24, g)
    khat = cache.dequant(np.arange(100) // 64, np.arange(100) % 64, 0, "k", g)
    ref, _ = softmax_attention(q[0], khat, khat[:, :512], 1 / 24)
    assert np.allclose(out[0], ref, rtol=1e-14, atol=0)
