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
