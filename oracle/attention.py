"""Paged decode attention by its textbook definition, float64 (CPU oracle).

TEST INFRASTRUCTURE (see ``oracle/formats.py``).

What is computed, per sequence b and query head h (the pages do not spell
attention out; this is the standard single-query softmax attention over the
cached tokens, with the quantized K/V dequantized first, the pages' point
being only that dequantization must live inside the attention kernel: SGLang
"Quantized KV Cache" page, performance warning in its introduction):

  kv head      = h // G, G = Hq / Hkv (consecutive query heads share a KV head)
  tokens       t = 0 .. L_b - 1, token t sits at page page_table[b][t // P],
               offset t % P
  s_t          = sm_scale * sum_d q[b,h,d] * K^[t,d]
  out[b,h,:]   = sum_t softmax(s)_t * V^[t,:]
  lse[b,h]     = log sum_t exp(s_t)
  L_b = 0      -> out = 0, lse = -inf

MLA (a single latent row per token shared by every head): K^ = the whole
latent row (Dk elements), V^ = its first Dv elements.
"""
from __future__ import annotations

import numpy as np

from .paged import OracleCache


def _pages_of(page_table_row, length, page_size):
    t = np.arange(length, dtype=np.int64)
    page = np.asarray(page_table_row, dtype=np.int64)[t // page_size]
    return page, t % page_size


def softmax_attention(q, k_hat, v_hat, sm_scale):
    """q [H, Dk], k_hat [L, Dk], v_hat [L, Dv] (float64) -> out [H, Dv], lse [H]."""
    h = q.shape[0]
    if k_hat.shape[0] == 0:
        return np.zeros((h, v_hat.shape[1])), np.full(h, -np.inf)
    s = sm_scale * (q @ k_hat.T)                       # [H, L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    denom = p.sum(axis=1, keepdims=True)
    out = (p @ v_hat) / denom
    lse = (m + np.log(denom))[:, 0]
    return out, lse


def decode_attention(cache: OracleCache, q, page_table, seq_lens, sm_scale,
                     k_scale=None, v_scale=None, batch_ids=None):
    """q [B, Hq, Dk] float -> (out [B, Hq, Dv], lse [B, Hq]) float64.

    ``batch_ids`` restricts the work to some sequences (others left 0 / nan).
    For NVFP4, ``k_scale`` is the global scale g.
    """
    spec = cache.spec
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape
    hkv = spec.num_kv_heads
    assert Hq % hkv == 0
    G = Hq // hkv
    out = np.zeros((B, Hq, spec.v_dim))
    lse = np.full((B, Hq), np.nan)
    for b in (range(B) if batch_ids is None else batch_ids):
        L = int(seq_lens[b])
        page, t = _pages_of(page_table[b], L, spec.page_size)
        for kvh in range(hkv):
            k_hat = cache.dequant(page, t, kvh, "k", k_scale, v_scale) if L else np.zeros((0, spec.head_dim))
            v_hat = cache.dequant(page, t, kvh, "v", k_scale, v_scale) if L else np.zeros((0, spec.v_dim))
            hs = slice(kvh * G, (kvh + 1) * G)
            o, l = softmax_attention(q[b, hs], k_hat, v_hat, sm_scale)
            out[b, hs] = o
            lse[b, hs] = l
    return out, lse



# --------------------------------------------------------------------------
# FP8-domain decode (vLLM "Quantized KV Cache" page, overview: with an FP8 KV
# cache, the Flash Attention 3 backend computes attention itself in FP8, the
# query being quantized to FP8 like the keys and values; its "Supported
# schemes" give the query its own scale, q_scale = [num_heads] per attention
# head or [1] per tensor, defaulting like k/v_scale to 1.0). Reading adopted:
# every query element is encoded to E4M3 as the cache's elements are,
# codes = encode(fl32(q / q_scale)) with saturation, whatever the cache's FP8
# format; the scores are then the exact products of those codes' values with
# the cached codes' values, times q_scale * k_scale * sm_scale; the weights
# and the value side are those of decode_attention. Equivalently: the
# attention of decode_attention with q replaced by decode(codes) * q_scale.
# --------------------------------------------------------------------------
def quantize_query_fp8(q, q_scale=None):
    """q [B, Hq, D] (BF16 values) -> (codes uint8 [B, Hq, D], per-head scales
    float32 [Hq]); q_scale None (1.0), a scalar, or one value per query head."""
    from .formats import E4M3
    from .quantize import quantize_fp8
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[1]
    s = np.full(hq, 1.0, np.float32) if q_scale is None else np.asarray(q_scale, np.float32)
    s = np.broadcast_to(s.reshape(-1), (hq,)).astype(np.float32) if s.size == 1 else s.reshape(hq)
    return quantize_fp8(q, s[None, :, None], E4M3), s


def decode_attention_fp8q(cache: OracleCache, q, page_table, seq_lens, sm_scale, q_scale=None,
                          k_scale=None, v_scale=None, batch_ids=None):
    """decode_attention in the FP8 domain: Q rounded to E4M3 with q_scale
    first (see quantize_query_fp8). Same arguments and results as
    decode_attention, plus q_scale."""
    from .formats import E4M3, decode
    codes, s = quantize_query_fp8(q, q_scale)
    q_hat = decode(codes.astype(np.int64), E4M3) * s[None, :, None].astype(np.float64)
    return decode_attention(cache, q_hat, page_table, seq_lens, sm_scale, k_scale, v_scale, batch_ids)

# --------------------------------------------------------------------------
# FP8-domain MLA decode (vLLM "Quantized KV Cache" page, overview: attention
# computed in FP8, the query quantized to FP8 like the keys; "Supported
# schemes": q_scale per tensor). The MLA latent is NVFP4, whose values no FP8
# format holds exactly, so the keys take the NVFP4 -> E4M3 step that
# dequantize_prev_kv defines (PR #21954 analysis page, "code analysis"), with
# the output scale 8g. Reading adopted: that scale is fixed by g, not
# calibrated: an NVFP4 value is e2m1 * e4m3 * g, at most 6 * 448 * g, so
# after the division by 8g every value lies within +-336 and no code
# saturates, and the division is exact (e2m1 * e4m3 / 8 has at most six
# significant bits), so each key element is the E4M3 rounding (to nearest,
# ties to even) of e2m1 * e4m3 / 8. Scores are
#   sm_scale * sum_d q^_d * (decode(K8 code) * 8g)_d
# with q^ = decode(quantize_query_fp8(q, q_scale)); the weights then multiply
# the exact NVFP4 values V^ = latent[:Dv] (the value side stays exact, as in
# the FP8-domain GQA path).
# --------------------------------------------------------------------------
def mla_fp8_keys(cache: OracleCache, page_table_row, length, g):
    """E4M3 key rows of the first `length` tokens of one MLA sequence: the
    dequantize_prev_kv rule (exact NVFP4 value, rounded once to binary32,
    then code = encode_E4M3(fl32(x^ / s))) with s = fl32(8g), applied to the
    sequence's own rows only (slots past its length hold arbitrary bytes).
    Returns (codes uint8 [length, Dk], s)."""
    from .formats import E4M3
    from .quantize import fl32, quantize_fp8
    s8 = np.float32(fl32(8.0 * np.float64(np.float32(g))))
    page, t = _pages_of(page_table_row, length, cache.spec.page_size)
    x_hat = fl32(cache.dequant(page, t, 0, "k", g))
    return quantize_fp8(x_hat, s8, E4M3), s8


def decode_attention_mla_fp8q(cache: OracleCache, q, page_table, seq_lens, sm_scale, q_scale=None, g=None,
                              batch_ids=None):
    """q [B, Hq, Dk] float -> (out [B, Hq, Dv], lse [B, Hq]) float64; an MLA
    NVFP4 cache, g its global scale (binary32, required)."""
    from .formats import E4M3, decode
    spec = cache.spec
    assert spec.kind == "mla" and spec.dtype == "nvfp4" and g is not None
    codes, s = quantize_query_fp8(q, q_scale)
    q_hat = decode(codes.astype(np.int64), E4M3) * s[None, :, None].astype(np.float64)
    B, Hq, _ = q_hat.shape
    out = np.zeros((B, Hq, spec.v_dim))
    lse = np.full((B, Hq), np.nan)
    for b in (range(B) if batch_ids is None else batch_ids):
        L = int(seq_lens[b])
        if L == 0:
            out[b], lse[b] = 0.0, -np.inf
            continue
        k8, s8 = mla_fp8_keys(cache, page_table[b], L, g)                   # [L, Dk] E4M3 codes
        k8_hat = decode(k8.astype(np.int64), E4M3) * np.float64(s8)
        page, t = _pages_of(page_table[b], L, spec.page_size)
        v_hat = cache.dequant(page, t, 0, "v", g)
        out[b], lse[b] = softmax_attention(q_hat[b], k8_hat, v_hat, sm_scale)
    return out, lse


# --------------------------------------------------------------------------
# Extend (chunked prefill) attention over a quantized prefix. The PR #21954
# analysis page ("code analysis") has dequantize_prev_kv turn the FP4 prefix
# into FP8 E4M3 workspaces (dq_k_buffer / dq_v_buffer) because only FP8
# prefill kernels exist; reading adopted for the attention that reads them:
# the C_b new tokens of sequence b attend to its L0_b prefix tokens through
# those E4M3 rows (value = decode(code) * s_k or s_v, the workspace's
# per-tensor scales) and to the chunk's own BF16 K/V causally (chunk token i
# sees chunk tokens 0..i), all query heads of a KV head sharing it (GQA).
# Prefix token t of sequence b is row t % P of page page_off[b] + t // P of
# the [n_pages, Hkv, P, D] workspace.
# --------------------------------------------------------------------------
def extend_attention(q, k_new, v_new, cu_q, prefix_len, dq_k, dq_v, page_off, s_k, s_v, sm_scale,
                     rows=None):
    """q [Nq, Hq, D], k_new / v_new [Nq, Hkv, D] (float), cu_q [B+1] chunk
    offsets, prefix_len / page_off [B], dq_k / dq_v uint8 E4M3 [n_pages, Hkv,
    P, D], s_k / s_v binary32 (None = 1.0) -> (out [Nq, Hq, D], lse [Nq, Hq])
    float64; ``rows`` restricts the work to some chunk rows (others nan)."""
    from .formats import E4M3, decode
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    Nq, Hq, D = q.shape
    Hkv = k_new.shape[1]
    G = Hq // Hkv
    P = dq_k.shape[2]
    sk = 1.0 if s_k is None else float(np.float32(s_k))
    sv = 1.0 if s_v is None else float(np.float32(s_v))
    out = np.full((Nq, Hq, D), np.nan)
    lse = np.full((Nq, Hq), np.nan)
    want = None if rows is None else set(int(r) for r in rows)
    for b in range(len(prefix_len)):
        if want is not None and not any(int(cu_q[b]) <= r < int(cu_q[b + 1]) for r in want):
            continue
        L0 = int(prefix_len[b])
        t = np.arange(L0)
        pg = int(page_off[b]) + t // P
        for kvh in range(Hkv):
            kp = decode(dq_k[pg, kvh, t % P].astype(np.int64), E4M3) * sk
            vp = decode(dq_v[pg, kvh, t % P].astype(np.int64), E4M3) * sv
            hs = slice(kvh * G, (kvh + 1) * G)
            for r in range(int(cu_q[b]), int(cu_q[b + 1])):
                if want is not None and r not in want:
                    continue
                keys = np.concatenate([kp, k_new[int(cu_q[b]):r + 1, kvh]])
                vals = np.concatenate([vp, v_new[int(cu_q[b]):r + 1, kvh]])
                o, l = softmax_attention(q[r, hs], keys, vals, sm_scale)
                out[r, hs] = o
                lse[r, hs] = l
    return out, lse
