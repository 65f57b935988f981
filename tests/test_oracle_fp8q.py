"""Pins for the FP8-domain decode oracle (oracle.attention.quantize_query_fp8,
decode_attention_fp8q) and the query-scale calibration
(oracle.quantize.fp8_query_scales): vLLM "Quantized KV Cache" page, overview
(the query quantized to FP8 like K and V) and "Supported schemes" (q_scale per
attention head or per tensor).

- query codes against torch's own float8_e4m3fn conversion (an independent
  implementation of the E4M3 rounding) wherever no saturation happens;
- saturation of out-of-range queries in closed form (the scale-reuse trap);
- the whole attention against torch's scaled_dot_product_attention (float64)
  fed the torch-rounded query;
- a query already on the E4M3 grid reduces to plain decode_attention;
- on the decode workloads' data, FP8-domain attention differs from BF16-query
  attention by far more than the GPU parity tolerance, so the parity tests can
  tell the two apart;
- calibration closed forms (amax = 448 * 2^k gives 2^k, zero heads give 1.0).
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import formats as F
from oracle import quantize as Q
from oracle.attention import decode_attention, decode_attention_fp8q, quantize_query_fp8
from oracle.paged import CacheSpec, OracleCache
from quantized_paged_kv_store_amd import inputs as I


def _torch_e4m3(x32, s32):
    """codes of fl32(x / s) by torch's float8_e4m3fn conversion"""
    t = torch.from_numpy(np.array(x32, np.float32)) / torch.from_numpy(np.array(s32, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("per_head", [False, True])
def test_query_codes_match_torch_float8(per_head):
    rng = np.random.default_rng(5)
    B, Hq, D = 3, 8, 64
    q = I.bf16_to_f32(I.bf16_bits((rng.standard_normal((B, Hq, D)) * 10.0 ** rng.uniform(-4, 2, (1, Hq, 1)))
                                  .astype(np.float32)))
    q[0, 0, :5] = [0.0, -0.0, 1e-30, -1e-30, 2.0 ** -133]                 # zeros and far-subnormal values
    amax = np.abs(q).max(axis=(0, 2)) if per_head else np.abs(q).max()
    s = (np.asarray(amax, np.float32) / np.float32(400.0)).astype(np.float32)   # headroom: no saturation
    codes, s_used = quantize_query_fp8(q, s if per_head else np.float32(s))
    want = _torch_e4m3(q, np.broadcast_to(s_used[None, :, None], q.shape))
    assert np.array_equal(codes, want)
    # the codes reach subnormals and both zero signs
    assert np.any(((codes & 0x78) == 0) & ((codes & 7) != 0)) and np.any(codes == 0x80) and np.any(codes == 0)


def test_saturation_with_a_stale_scale():
    """A scale calibrated on smaller queries clamps the larger ones to +-448 (E4M3 has no infinity)."""
    q = np.zeros((1, 2, 16))
    q[0, 0, :4] = [1000.0, -1000.0, 449.0 * 2, 3.0]
    q[0, 1, :2] = [7.0, -7.0]
    codes, s = quantize_query_fp8(q, [2.0, 0.015625])
    assert list(codes[0, 0, :4]) == [0x7E, 0xFE, 0x7E, 0x3C]             # 448, -448, 448, 1.5 = 3 / 2
    assert list(codes[0, 1, :2]) == [0x7E, 0xFE]                         # 7 / 2^-6 = 448 exactly
    assert np.array_equal(F.decode(codes[0, 0, :4].astype(np.int64), F.E4M3) * 2.0, [896.0, -896.0, 896.0, 3.0])


def _cache(dtype, B, Hkv, D, P, L, seed, G=4):
    w = I.Workload("t", dtype, "gqa", B, G * Hkv, Hkv, D, D, P, L, L, 1, "llama", seed=seed)
    lens = I.seq_lens(w)
    table, npages = I.page_table(w, lens)
    cache = OracleCache(CacheSpec(dtype, "gqa", Hkv, D, D, P, npages))
    for b in range(B):
        k, v = I.kv_rows(w, b, 0, L)
        cache.store(I.bf16_to_f32(k), I.bf16_to_f32(v), I.slots_for(table[b], np.arange(L), P),
                    k_scale=np.float32(0.05), v_scale=np.float32(0.03))
    return w, cache, table, lens, I.bf16_to_f32(I.queries(w))


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_fp8q_decode_matches_sdpa_on_torch_rounded_query(dtype):
    B, Hkv, D, P, L, G = 2, 2, 128, 16, 200, 4
    w, cache, table, lens, q = _cache(dtype, B, Hkv, D, P, L, 11, G)
    ks, vs = np.float32(0.05), np.float32(0.03)
    qs = Q.fp8_query_scales(q, per_head=True) * np.float32(1.5)
    sm = 0.0883883
    out, lse = decode_attention_fp8q(cache, q, table, lens, sm, qs, ks, vs)
    for b in range(B):
        page, t = table[b][np.arange(L) // P], np.arange(L) % P
        K = np.stack([cache.dequant(page, t, h, "k", ks, vs) for h in range(Hkv)])
        V = np.stack([cache.dequant(page, t, h, "v", ks, vs) for h in range(Hkv)])
        codes = _torch_e4m3(q[b], np.broadcast_to(qs[:, None], q[b].shape))
        qh = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * qs[:, None].astype(np.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qh)[None, :, None, :], torch.from_numpy(K).repeat_interleave(G, 0)[None],
            torch.from_numpy(V).repeat_interleave(G, 0)[None], scale=sm)[0, :, 0].numpy()
        assert np.allclose(out[b], ref, rtol=1e-12, atol=1e-13)
        s = sm * np.einsum("hd,hld->hl", qh, np.repeat(K, G, 0))
        assert np.allclose(lse[b], logsumexp(s, axis=1), rtol=1e-13)


def test_query_on_the_grid_equals_bf16_decode():
    """q = E4M3 value * 2^-3 everywhere and q_scale = 2^-3: the rounding is the identity."""
    B, Hkv, D, P, L = 2, 2, 64, 16, 90
    w, cache, table, lens, _ = _cache("e4m3", B, Hkv, D, P, L, 12)
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7F, (B, 4 * Hkv, D)) | (rng.integers(0, 2, (B, 4 * Hkv, D)) << 7)
    q = F.decode(codes, F.E4M3) * 0.125
    a = decode_attention_fp8q(cache, q, table, lens, 0.11, np.float32(0.125), np.float32(0.05), np.float32(0.03))
    b = decode_attention(cache, q, table, lens, 0.11, np.float32(0.05), np.float32(0.03))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fp8_domain_is_distinguishable_at_the_parity_tolerance():
    B, Hkv, D, P, L = 2, 2, 128, 16, 400
    w, cache, table, lens, q = _cache("e4m3", B, Hkv, D, P, L, 13)
    qs = Q.fp8_query_scales(q, per_head=False)
    a, _ = decode_attention_fp8q(cache, q, table, lens, 0.0883883, qs, np.float32(0.05), np.float32(0.03))
    b, _ = decode_attention(cache, q, table, lens, 0.0883883, np.float32(0.05), np.float32(0.03))
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel > 1e-2                     # ten times the 1e-3 rel-L2 parity bound


def test_query_scale_calibration_closed_forms():
    q = np.zeros((3, 4, 8))
    q[1, 0, 2] = -448.0 * 2.0 ** -5        # head 0: amax 448 * 2^-5 -> 2^-5 exactly
    q[2, 1, 7] = 448.0 * 3.0               # head 1: -> 3.0
    q[0, 3, 0] = 1.0                       # head 3: -> fl32(1 / 448); head 2 all zero -> 1.0
    s = Q.fp8_query_scales(q, per_head=True)
    assert s.dtype == np.float32 and list(s[:3]) == [2.0 ** -5, 3.0, 1.0]
    assert s[3] == np.float32(np.float32(1.0) / np.float32(448.0))
    assert list(Q.fp8_query_scales(q, per_head=False)) == [3.0]
    assert list(Q.fp8_query_scales(np.zeros((0, 4, 8)), per_head=False)) == [1.0]


# ---------------------------------------------------------------------------
# FP8-domain MLA (oracle.attention.decode_attention_mla_fp8q): keys are the
# E4M3 rounding of e2m1 * e4m3 / 8 (the NVFP4 -> E4M3 step of
# dequantize_prev_kv with the output scale 8g), values stay exact.
# ---------------------------------------------------------------------------
from oracle.attention import decode_attention_mla_fp8q, mla_fp8_keys  # noqa: E402
from oracle.paged import dequantize_prev_kv  # noqa: E402


def _mla_cache(rows, g, P=16):
    L = rows.shape[0]
    npg = (L + P - 1) // P
    oc = OracleCache(CacheSpec("nvfp4", "mla", 1, 576, 512, P, npg))
    oc.store(rows, None, np.arange(L), k_scale=np.float32(g))
    table = np.arange(npg, dtype=np.int32)[None, :]
    return oc, table


def test_mla_fp8_keys_are_torch_e4m3_of_nvfp4_over_8():
    """Every key code equals torch's float8_e4m3fn rounding of the exact NVFP4
    value divided by 8g (an independent encoder); blocks scaled far down reach
    E4M3 subnormals; nothing saturates: |value| <= 336 < 448."""
    rng = np.random.default_rng(21)
    L = 70
    x = rng.standard_normal((L, 576)).astype(np.float32)
    x[:, :16] *= 8.0
    x[5:9, 32:64] *= 2.0 ** -9                                   # blocks whose E4M3 scales are tiny
    x = I.bf16_to_f32(I.bf16_bits(x))
    g = Q.nvfp4_global_scale(np.abs(x).max())
    oc, table = _mla_cache(x, g)
    npg = table.shape[1]
    s8 = np.float32(8.0 * np.float64(g))
    k8, _ = dequantize_prev_kv(oc, np.arange(npg), s8, None, g=g)
    k8 = k8.reshape(-1, 576)[:L]
    rows, s8r = mla_fp8_keys(oc, table[0], L, g)                  # the rows the decode uses
    assert s8r == s8 and np.array_equal(rows, k8)
    exact = oc.dequant(np.arange(L) // 16, np.arange(L) % 16, 0, "k", g) / (8.0 * np.float64(g))
    assert np.array_equal(exact, exact.astype(np.float32).astype(np.float64))   # e2m1 * e4m3 / 8: exact in fp32
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(k8, want)
    mag = k8 & 0x7F
    assert mag.max() <= 0x7A and not np.any(mag == 0x7E)                         # 0x7A = 320, <= 336
    assert np.any((mag > 0) & (mag < 8))                                         # E4M3 subnormals occur
    assert np.mean(F.decode(k8.astype(np.int64), F.E4M3) != exact) > 0.2         # most keys are rounded


def test_mla_fp8_on_grid_equals_plain_decode():
    """Latent rows of the form e2m1 * 2^k * g with block maxima 6 * 2^k * g:
    the NVFP4 scales are powers of two, every key e2m1 * 2^k / 8 is an E4M3
    value, and a query on the E4M3 grid (q_scale 1) is kept as it is, so the
    FP8-domain result equals the plain MLA decode."""
    rng = np.random.default_rng(22)
    L, g = 45, np.float32(2.0 ** -6)
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    blocks = rng.choice(e2m1, size=(L, 36, 16)) * rng.choice([-1.0, 1.0], size=(L, 36, 16))
    blocks[:, :, 0] = 6.0                                                        # block max 6 * 2^k
    k = rng.integers(-2, 6, size=(L, 36, 1))
    x = (blocks * 2.0 ** k * np.float64(g)).reshape(L, 576)
    oc, table = _mla_cache(x, g)
    q = F.decode(rng.integers(0, 0x7E, size=(2, 8, 576)) | (rng.integers(0, 2, size=(2, 8, 576)) << 7), F.E4M3)
    q = np.where(np.abs(q) > 240, 0.0, q) * 2.0 ** -6
    lens = np.array([L, 30])
    tab = np.repeat(table, 2, axis=0)
    a, la = decode_attention_mla_fp8q(oc, q, tab, lens, 0.041, 2.0 ** -6, g)
    b, lb = decode_attention(oc, q, tab, lens, 0.041, g)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14) and np.allclose(la, lb, rtol=1e-12, atol=1e-12)


def test_mla_fp8_zero_query_is_mean_of_exact_values():
    """q = 0: every score is 0, so the output is the mean of the exact NVFP4
    value rows (not of their E4M3 roundings) and the LSE is log L."""
    rng = np.random.default_rng(23)
    L = 37
    x = I.bf16_to_f32(I.bf16_bits(rng.standard_normal((L, 576)).astype(np.float32)))
    g = Q.nvfp4_global_scale(np.abs(x).max())
    oc, table = _mla_cache(x, g)
    out, lse = decode_attention_mla_fp8q(oc, np.zeros((1, 4, 576)), table, [L], 0.04, None, g)
    v = oc.dequant(np.arange(L) // 16, np.arange(L) % 16, 0, "v", g)
    assert np.allclose(out[0], v.mean(axis=0)[None, :], rtol=1e-12, atol=1e-15)
    assert np.allclose(lse, np.log(L), rtol=0, atol=1e-12)


def test_mla_fp8_differs_from_plain_beyond_tolerance():
    """On the DeepSeek-R1-shaped data the FP8-domain result moves far more than
    the GPU parity tolerance away from the plain MLA decode (so the parity
    tests tell the paths apart), and stays a few percent from it."""
    w = I.WORKLOADS["dsr1_mla"].with_(batch=1, max_len=300, min_len=300)
    k, _ = I.kv_rows(w, 0, 0, 300)
    x = I.bf16_to_f32(k)
    g = Q.nvfp4_global_scale(np.abs(x).max())
    oc, table = _mla_cache(x, g, P=64)
    q = I.bf16_to_f32(I.queries(w))[:, :16]
    qs = Q.fp8_query_scales(q, per_head=False)
    a, _ = decode_attention_mla_fp8q(oc, q, table, [300], I.sm_scale(w), qs, g)
    b, _ = decode_attention(oc, q, table, [300], I.sm_scale(w), g)
    d = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert np.abs(a - b).max() > 4e-3 or d > 1e-3, d
    assert d < 0.2, d


def test_mla_fp8_keys_ignore_slots_past_the_length():
    """Never-written slots of a sequence's last page (here NaN scale bytes)
    are not read: the key rows and the decode depend on the first L rows only."""
    rng = np.random.default_rng(24)
    L, P = 21, 16
    x = I.bf16_to_f32(I.bf16_bits(rng.standard_normal((L, 576)).astype(np.float32)))
    g = Q.nvfp4_global_scale(np.abs(x).max())
    oc = OracleCache(CacheSpec("nvfp4", "mla", 1, 576, 512, P, 2), fill=0xFF)
    oc.store(x, None, np.arange(L), k_scale=np.float32(g))
    clean, table = _mla_cache(x, g, P)
    rows, _ = mla_fp8_keys(oc, table[0], L, g)
    assert np.array_equal(rows, mla_fp8_keys(clean, table[0], L, g)[0])
    q = rng.standard_normal((1, 3, 576))
    a = decode_attention_mla_fp8q(oc, q, table, [L], 0.05, None, g)
    b = decode_attention_mla_fp8q(clean, q, table, [L], 0.05, None, g)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
