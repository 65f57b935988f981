"""KV-cache byte accounting (CPU oracle).

TEST INFRASTRUCTURE (see ``oracle/formats.py``).

* "KV cache quantization mechanism and traps" page, section on measured
  INT8/FP8/INT4 numbers: bytes per token = 2 (K and V) x layers x KV heads x
  head_dim x bytes per element, and cache size = bytes per token x context x
  batch, reported in units of 1024**3 bytes (the page's sizing snippet in
  "when to enable").
* SGLang "Quantized KV Cache" page, "Memory savings": token capacity ratios
  that include the per-block scale overhead.
"""
from __future__ import annotations

# storage bits per element, including per-block scale overhead
BITS_PER_ELEMENT = {
    "bf16": 16.0,
    "fp16": 16.0,
    "e4m3": 8.0,           # per-tensor scale: no per-element overhead
    "e5m2": 8.0,
    "int8": 8.0,
    "int4": 4.0,
    "mx16": 4.0 + 8.0 / 16,    # E2M1 + one 8-bit exponent per 16 elements
    "nvfp4": 4.0 + 8.0 / 16,   # E2M1 + one E4M3 scale per 16 (+ one fp32 per tensor)
}


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype: str) -> float:
    return 2 * layers * kv_heads * head_dim * BITS_PER_ELEMENT[dtype] / 8


def kv_cache_gib(layers, kv_heads, head_dim, dtype, context, batch) -> float:
    return kv_bytes_per_token(layers, kv_heads, head_dim, dtype) * context * batch / 1024 ** 3


def capacity_ratio(dtype_from: str, dtype_to: str) -> float:
    """How many more tokens fit when switching dtype_from -> dtype_to."""
    return BITS_PER_ELEMENT[dtype_from] / BITS_PER_ELEMENT[dtype_to]


def decode_kv_bytes(seq_lens, kv_heads, head_dim, dtype, kind="gqa") -> int:
    """Algorithmic KV bytes one decode step reads: codes + block scales of
    every cached token (K and V for GQA; one latent row for MLA)."""
    per_row = head_dim * BITS_PER_ELEMENT[dtype] / 8
    rows = 2 * kv_heads if kind == "gqa" else 1
    return int(round(sum(int(L) for L in seq_lens) * rows * per_row))
