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


# ------------------------------------------------------ dequantize_prev_kv ----
from oracle.paged import dequantize_prev_kv  # noqa: E402


def test_dequantize_prev_kv_identity_on_e4m3_grid():
    """MX16 blocks whose values E2M1 * 2^e are all E4M3 numbers (e in
    [-6, 6]) come back unchanged through FP4 -> FP8 with scale 1: every code
    decodes to exactly the dequantized FP4 value."""
    spec = CacheSpec("mx16", "gqa", 2, 128, 128, 16, 3)
    rng = np.random.default_rng(41)
    e2m1 = F.decode(np.arange(16), F.E2M1)
    # 16-element blocks: E2M1 values with the block max 4 or 6 (so the store
    # reproduces the exponent), times 2^e
    blocks = rng.choice(e2m1, size=(40, 2, 8, 16))
    blocks[..., 0] = rng.choice([4.0, 6.0, -4.0, -6.0], size=blocks.shape[:-1])
    e = rng.integers(-6, 5, size=blocks.shape[:-1] + (1,))
    x = (blocks * 2.0 ** e).reshape(40, 2, 128)
    oc = OracleCache(spec)
    slots = rng.permutation(48)[:40]
    oc.store(x, -x, slots)
    used = np.unique(slots // 16)
    dk, dv = dequantize_prev_kv(oc, used)
    for i, pg in enumerate(used):
        for h in range(2):
            xk = oc.dequant(np.full(16, pg), np.arange(16), h, "k")
            xv = oc.dequant(np.full(16, pg), np.arange(16), h, "v")
            assert np.array_equal(F.decode(dk[i, h], F.E4M3), xk)
            assert np.array_equal(F.decode(dv[i, h], F.E4M3), xv)


def test_dequantize_prev_kv_scale_and_saturation():
    """code = RNE_sat(x^ / s): doubling s halves every decoded value exactly
    (powers of two), and a scale small enough to overflow saturates at 448."""
    spec = CacheSpec("mx16", "gqa", 1, 128, 128, 16, 1)
    rng = np.random.default_rng(42)
    x = rng.standard_normal((16, 1, 128))
    oc = OracleCache(spec)
    oc.store(x, x, np.arange(16))
    d1, _ = dequantize_prev_kv(oc, [0], 1.0, 1.0)
    d2, _ = dequantize_prev_kv(oc, [0], 2.0, 2.0)
    f1, f2 = F.decode(d1, F.E4M3), F.decode(d2, F.E4M3)
    normal = np.abs(f1) >= 2.0 ** -5            # both stay in E4M3's normal range
    assert np.array_equal(f2[normal], f1[normal] / 2)
    ds, _ = dequantize_prev_kv(oc, [0], 1e-6, 1e-6)
    big = np.abs(oc.dequant(np.zeros(16, int), np.arange(16), 0, "k")) > 448e-6
    assert np.all(np.abs(F.decode(ds[0, 0], F.E4M3))[big] == 448.0)


def test_dequantize_prev_kv_nvfp4_error_bound():
    """NVFP4 -> E4M3 with s = 6 g: |dec(code) * s - x^| <= 2^-4 |x^| in E4M3's
    normal range (one RNE rounding to a 4-bit significand)."""
    spec = CacheSpec("nvfp4", "mla", 1, 576, 512, 64, 2)
    rng = np.random.default_rng(43)
    x = rng.standard_normal((100, 576)) * np.where(rng.random(576) < 0.03, 8.0, 1.0)
    g = Q.nvfp4_global_scale(np.abs(x).max())
    oc = OracleCache(spec)
    oc.store(x, None, np.arange(100), k_scale=g)
    s = np.float32(np.float32(6.0) * g)
    dk, dv = dequantize_prev_kv(oc, [0, 1], s, None, g)
    assert dv is None and dk.shape == (2, 64, 576)
    for i in range(2):
        x_hat = oc.dequant(np.full(64, i), np.arange(64), 0, "k", g)
        back = F.decode(dk[i], F.E4M3) * float(s)
        normal = np.abs(x_hat) >= 2.0 ** -6 * float(s)
        assert np.all(np.abs(back - x_hat)[normal] <= 2.0 ** -4 * np.abs(x_hat)[normal] * (1 + 1e-6))
        assert np.all(np.abs(back) <= 448.0 * float(s))


def test_kivi_cache_round_trip_on_grid():
    """KIVI-style cache: K rows on the E4M3 grid times power-of-two channel
    scales and V rows on the grid whose per-token scale is exact come back
    exactly; the V scale buffer holds each token's fl32(amax / 448) at float t
    of its (page, head) block. A swapped channel or token index fails."""
    rng = np.random.default_rng(31)
    spec = CacheSpec("e4m3", "gqa", 2, 64, 64, 32, 3, kivi=True)
    oc = OracleCache(spec)
    grid = F.decode(np.arange(0x7F), F.E4M3)                    # every finite magnitude
    T = 70
    ks = (2.0 ** rng.integers(-8, 4, (2, 64))).astype(np.float32)
    kc = rng.choice(grid, (T, 2, 64)) * np.where(rng.random((T, 2, 64)) < 0.5, -1, 1)
    k = kc * ks[None].astype(np.float64)
    vrow = rng.choice(grid, (T, 2, 64)) * np.where(rng.random((T, 2, 64)) < 0.5, -1, 1)
    vrow[:, :, 7] = 448.0                                        # every row's amax is 448 * (its factor)
    vfac = 2.0 ** rng.integers(-10, 6, (T, 2, 1))
    v = vrow * vfac / 448.0 * 448.0
    slots = rng.permutation(spec.num_pages * spec.page_size)[:T]
    oc.store(k, v, slots, k_scale=ks)
    page, t = slots // spec.page_size, slots % spec.page_size
    for h in range(2):
        assert np.array_equal(oc.dequant(page, t, h, "k", k_scale=ks), k[:, h])
        assert np.array_equal(oc.dequant(page, t, h, "v"), v[:, h])
        got = oc.v_token_scales()[page, h, t]
        assert np.array_equal(got, (np.float32(448.0 * vfac[:, h, 0]) / np.float32(448.0)).astype(np.float32))
    assert oc.v_scales.shape == (3, 2, 4 * 32) and spec.token_scale_block_bytes() == 128


def _owner_map(spec, fn, n_elem):
    """Token (t16) owning each byte of one tile of a (page, head) block, from
    the position function fn. Asserts that no byte (or its two nibbles) is
    shared by two tokens and that every byte of the tile is used."""
    t, d = np.meshgrid(np.arange(16), np.arange(n_elem), indexing="ij")
    byte, _ = fn(spec, t, d)
    size = int(byte.max()) + 1
    owner = np.full(size, -1)
    for tt, bb in zip(t.ravel(), np.asarray(byte).ravel()):
        assert owner[bb] in (-1, tt), f"byte {bb} holds codes of tokens {owner[bb]} and {tt}"
        owner[bb] = tt
    assert np.all(owner >= 0)
    return owner


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"{s.dtype}-{s.head_dim}-P{s.page_size}")
def test_layout_properties_the_header_states(spec):
    """Properties include/kvq.h states in words (and the decode kernels' loads
    rely on), checked on the layout functions without their formulas: every
    byte holds codes of one token only; GQA K puts token t16 of a tile in the
    t16-th 16-byte lane of every 256-byte group; FP8 V puts one element of
    four consecutive tokens in each 4-byte word; FP4 V and the MLA latent put
    four consecutive tokens of one 8- / 4-element group in each 16- / 8-byte
    unit, token by token."""
    D = spec.head_dim
    fp8 = spec.dtype in ("e4m3", "e5m2")
    if spec.kind == "gqa":
        k_owner = _owner_map(spec, k_code_pos, D)
        assert np.array_equal(k_owner, (np.arange(k_owner.size) % 256) // 16)
        v_owner = _owner_map(spec, v_code_pos, D)
        if fp8:
            # byte i of each word: token 4g + i, the word's four bytes one element
            words = v_owner.reshape(-1, 4)
            assert np.all(words % 4 == np.arange(4)) and np.all(words // 4 == words[:, :1] // 4)
            t, d = np.meshgrid(np.arange(16), np.arange(D), indexing="ij")
            byte, _ = v_code_pos(spec, t, d)
            word_elems = {}
            for dd, bb in zip(d.ravel(), np.asarray(byte).ravel()):
                word_elems.setdefault(bb // 4, set()).add(dd)
            assert all(len(e) == 1 for e in word_elems.values())
        else:
            # each 16-byte lane: tokens 4g..4g+3, one 4-byte word each, one 8-element group
            lanes = v_owner.reshape(-1, 16)
            assert np.all(lanes == lanes[:, ::4].repeat(4, axis=1))
            assert np.all(lanes[:, ::4] % 4 == np.arange(4)) and np.all(lanes[:, ::4] // 4 == lanes[:, :1] // 4)
    else:
        owner = _owner_map(spec, k_code_pos, D)
        # each 8-byte unit: tokens 4g..4g+3, two bytes (one 4-element group) each
        units = owner.reshape(-1, 8)
        assert np.all(units == units[:, ::2].repeat(2, axis=1))
        assert np.all(units[:, ::2] % 4 == np.arange(4)) and np.all(units[:, ::2] // 4 == units[:, :1] // 4)
