"""Pins for oracle/paged.py: the byte layout is a bijection onto each page
block, store places exactly the quantizer's codes, and gather returns the
quantizer's dequantized values (so a transposed index or a swapped nibble in
the layout formulas fails here)."""
import numpy as np
import pytest

from oracle import formats as F
from oracle import quantize as Q
from oracle.paged import (CacheSpec, OracleCache, k_code_pos, k_scale_pos,
                          v_code_pos, v_scale_pos)

SPECS = [
    CacheSpec("e4m3", "gqa", 2, 64, 64, 16, 4),
    CacheSpec("e5m2", "gqa", 2, 128, 128, 32, 4),
    CacheSpec("mx16", "gqa", 2, 128, 128, 16, 4),
    CacheSpec("mx16", "gqa", 1, 256, 256, 32, 2),
    CacheSpec("nvfp4", "mla", 1, 576, 512, 64, 2),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"{s.dtype}-{s.head_dim}-P{s.page_size}")
def test_layout_is_bijection(spec):
    cb, sb = spec.block_bytes()
    t, d = np.meshgrid(np.arange(spec.page_size), np.arange(spec.head_dim), indexing="ij")
    fns = [k_code_pos] + ([v_code_pos] if spec.kind == "gqa" else [])
    for fn in fns:
        byte, nib = fn(spec, t, d)
        key = byte * 2 + nib if spec.dtype not in ("e4m3", "e5m2") else byte
        n_slots = cb * (2 if spec.dtype not in ("e4m3", "e5m2") else 1)
        assert key.min() == 0 and key.max() == n_slots - 1
        assert len(np.unique(key)) == key.size == n_slots
    if sb:
        tb, b = np.meshgrid(np.arange(spec.page_size), np.arange(spec.head_dim // 16), indexing="ij")
        for fn in [k_scale_pos] + ([v_scale_pos] if spec.kind == "gqa" else []):
            pos = fn(spec, tb, b)
            assert pos.min() == 0 and pos.max() == sb - 1 and len(np.unique(pos)) == pos.size


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"{s.dtype}-{s.head_dim}-P{s.page_size}")
def test_store_then_gather_equals_quantize_dequantize(spec):
    rng = np.random.default_rng(9)
    n_tok = spec.num_pages * spec.page_size
    slots = rng.permutation(n_tok)[: n_tok - 5]
    H = spec.num_kv_heads
    k = rng.standard_normal((len(slots), H, spec.head_dim)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((len(slots), H, spec.head_dim)).astype(np.float32).astype(np.float64)
    cache = OracleCache(spec, fill=0xA5)
    if spec.kind == "mla":
        g = Q.nvfp4_global_scale(np.abs(k).max())
        cache.store(k[:, 0], None, slots, k_scale=g)
    else:
        cache.store(k, v, slots, k_scale=np.float32(0.05), v_scale=np.float32(0.02))
    page, t = slots // spec.page_size, slots % spec.page_size
    for h in range(H):
        if spec.dtype in ("e4m3", "e5m2"):
            fmt = F.E4M3 if spec.dtype == "e4m3" else F.E5M2
            wk = Q.dequantize_fp8(Q.quantize_fp8(k[:, h], np.float32(0.05), fmt), np.float32(0.05), fmt)
            wv = Q.dequantize_fp8(Q.quantize_fp8(v[:, h], np.float32(0.02), fmt), np.float32(0.02), fmt)
            gk = cache.dequant(page, t, h, "k", np.float32(0.05), np.float32(0.02))
            gv = cache.dequant(page, t, h, "v", np.float32(0.05), np.float32(0.02))
        elif spec.dtype == "mx16":
            wk = Q.dequantize_mx16(*Q.quantize_mx16(k[:, h]))
            wv = Q.dequantize_mx16(*Q.quantize_mx16(v[:, h]))
            gk, gv = cache.dequant(page, t, h, "k"), cache.dequant(page, t, h, "v")
        else:
            wk = Q.dequantize_nvfp4(*Q.quantize_nvfp4(k[:, 0], g), g)
            wv = wk[:, :spec.v_dim]
            gk, gv = cache.dequant(page, t, 0, "k", g), cache.dequant(page, t, 0, "v", g)
        assert np.array_equal(gk, wk) and np.array_equal(gv, wv)
    # slots never stored keep the fill byte
    stored = np.zeros(n_tok, bool)
    stored[slots] = True
    free = np.flatnonzero(~stored)
    byte, _ = k_code_pos(spec, free[:, None] % spec.page_size, np.arange(spec.head_dim)[None, :])
    assert np.all(cache.k_codes[free[:, None] // spec.page_size, 0, byte] == 0xA5)


def test_negative_slots_are_skipped():
    spec = SPECS[0]
    cache = OracleCache(spec, fill=0x11)
    k = np.ones((2, 2, 64))
    cache.store(k, k, np.array([-1, 3]), k_scale=1.0, v_scale=1.0)
    byte, _ = k_code_pos(spec, np.array([3]), np.arange(64))
    assert np.all(cache.k_codes[0, 0, byte] == 0x38)
    assert np.count_nonzero(cache.k_codes != 0x11) == 2 * 64


def test_per_head_scales_round_trip_on_grid():
    """Per-head FP8 store: values built as (E4M3 value) * s_h round-trip
    exactly through store + dequant with the per-head scale array, and head h
    never uses another head's scale."""
    spec = CacheSpec("e4m3", "gqa", 3, 64, 64, 16, 4)
    rng = np.random.default_rng(13)
    grid = F.decode(np.arange(0, 0x7F), F.E4M3)           # finite non-negative E4M3 values
    s = np.array([0.25, 3.0, 0.0078125], np.float32)
    vals = rng.choice(grid, size=(20, 3, 64)) * rng.choice([-1, 1], size=(20, 3, 64))
    k = vals * s[None, :, None]
    v = vals[::-1] * s[None, :, None]
    oc = OracleCache(spec)
    slots = rng.permutation(4 * 16)[:20]
    oc.store(k, v, slots, k_scale=s, v_scale=s)
    page, t = slots // 16, slots % 16
    for h in range(3):
        assert np.array_equal(oc.dequant(page, t, h, "k", s, s), k[:, h])
        assert np.array_equal(oc.dequant(page, t, h, "v", s, s), v[:, h])
