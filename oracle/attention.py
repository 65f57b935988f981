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
