"""Paged quantized KV cache: byte layout, store and gather (CPU oracle).

TEST INFRASTRUCTURE (see ``oracle/formats.py``).

The pages do not describe paging. The PR #21954 analysis page ("code
analysis", create_buffers) names separate data buffers (k_buffer, v_buffer)
and separate block-scale buffers (k_scale_buffer, v_scale_buffer); the layout
below keeps that split. Paging itself (fixed-size pages reached through a
per-sequence page table, a slot = page * page_size + offset) is the reading
adopted for the paged store the workloads name.

Byte layout of one cache (all offsets in bytes; t = token index inside its
page, t16 = t % 16, tile = t // 16, d = element index, b = d // 16):

  every buffer is [num_pages][num_kv_heads][block], block = page_size * row
  bytes, made of 16-token tiles laid one after the other.

  KIVI-style FP8 caches (K scale per channel, V scale per token) add a V
  scale buffer of one binary32 per token: float t of the (page, kv head)
  block; the per-channel K scales are [Hkv, D] arrays held by the caller.

  GQA, FP8 (E4M3 / E5M2), row = D bytes, tile = 16 * D bytes:
    K: 256 * (d // 16) + 16 * t16 + d % 16
    V: 1024 * (d // 64) + 16 * (16 * (t16 // 4) + d % 16)
       + 4 * ((d // 16) % 4) + t16 % 4
  GQA, FP4 block-16 (E2M1 codes, 2 per byte, even d in the low nibble),
  tile = 8 * D code bytes and D scale bytes:
    K code byte:  256 * (d // 32) + 16 * t16 + (d % 32) // 2
    V code byte:  1024 * (d // 128) + 16 * (16 * (t16 // 4) + (d % 128) // 8)
                  + 4 * (t16 % 4) + (d % 8) // 2
    K scale byte: 32 * (b // 2) + 2 * t16 + b % 2
    V scale byte: 4 * ((D // 16) * (t16 // 4) + b) + t16 % 4
  MLA, NVFP4 (one latent row of Dk = 576 elements per token, the first
  Dv = 512 of them are V; num_kv_heads = 1), tile = 4608 code bytes and 576
  E4M3 scale bytes; g4 = t16 // 4, tt = t16 % 4:
    code byte, d < 512:  2 * (((d // 64 * 4 + g4) * 16 + (d % 64) // 4) * 4 + tt) + (d % 4) // 2
    code byte, d >= 512: 4096 + 2 * ((g4 * 16 + (d - 512) // 4) * 4 + tt) + (d % 4) // 2
    scale byte, b < 32:  4 * ((b // 4 * 4 + g4) * 4 + b % 4) + tt
    scale byte, b >= 32: 512 + 4 * (g4 * 4 + b - 32) + tt
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import quantize as Q
from .formats import E2M1, E4M3, E5M2, decode

TILE = 16


@dataclass
class CacheSpec:
    dtype: str          # "e4m3" | "e5m2" | "mx16" | "nvfp4"
    kind: str           # "gqa" | "mla"
    num_kv_heads: int
    head_dim: int       # GQA D; MLA Dk (latent + rope)
    v_dim: int          # GQA D; MLA Dv (latent)
    page_size: int
    num_pages: int
    kivi: bool = False  # FP8 GQA: K scales per channel, V scales per token (buffer below)

    def code_row_bytes(self) -> int:
        return self.head_dim if self.dtype in ("e4m3", "e5m2") else self.head_dim // 2

    def scale_row_bytes(self) -> int:
        return 0 if self.dtype in ("e4m3", "e5m2") else self.head_dim // 16

    def block_bytes(self) -> tuple[int, int]:
        return (self.page_size * self.code_row_bytes(), self.page_size * self.scale_row_bytes())

    def token_scale_block_bytes(self) -> int:
        """KIVI: one binary32 V scale per token of a (page, kv head) block, token t at float t."""
        return 4 * self.page_size if self.kivi else 0


# ---------------------------- layout formulas -----------------------------
def _tile_base(t, row_bytes):
    return (t // TILE) * TILE * row_bytes


def _mla_code_byte(t, d):
    t16 = t % TILE
    g4, tt = t16 // 4, t16 % 4
    lo = 2 * (((d // 64 * 4 + g4) * 16 + (d % 64) // 4) * 4 + tt) + (d % 4) // 2
    hi = 4096 + 2 * ((g4 * 16 + (d - 512) // 4) * 4 + tt) + (d % 4) // 2
    return _tile_base(t, 288) + np.where(d < 512, lo, hi)


def k_code_pos(spec: CacheSpec, t, d):
    """(byte offset inside the page-head block, nibble) of K element (t, d)."""
    t = np.asarray(t); d = np.asarray(d)
    t16 = t % TILE
    if spec.kind == "mla":
        assert spec.head_dim == 576 and spec.v_dim == 512
        return _mla_code_byte(t, d), d % 2
    if spec.dtype in ("e4m3", "e5m2"):
        return _tile_base(t, spec.head_dim) + 256 * (d // 16) + 16 * t16 + d % 16, np.zeros_like(d)
    base = _tile_base(t, spec.head_dim // 2)
    return base + 256 * (d // 32) + 16 * t16 + (d % 32) // 2, d % 2


def v_code_pos(spec: CacheSpec, t, d):
    t = np.asarray(t); d = np.asarray(d)
    t16 = t % TILE
    if spec.dtype in ("e4m3", "e5m2"):
        off = (1024 * (d // 64) + 16 * (16 * (t16 // 4) + d % 16)
               + 4 * ((d // 16) % 4) + t16 % 4)
        return _tile_base(t, spec.head_dim) + off, np.zeros_like(d)
    base = _tile_base(t, spec.head_dim // 2)
    off = (1024 * (d // 128) + 16 * (16 * (t16 // 4) + (d % 128) // 8)
           + 4 * (t16 % 4) + (d % 8) // 2)
    return base + off, d % 2


def k_scale_pos(spec: CacheSpec, t, b):
    t = np.asarray(t); b = np.asarray(b)
    if spec.kind == "mla":
        t16 = t % TILE
        g4, tt = t16 // 4, t16 % 4
        lo = 4 * ((b // 4 * 4 + g4) * 4 + b % 4) + tt
        hi = 512 + 4 * (g4 * 4 + b - 32) + tt
        return _tile_base(t, 36) + np.where(b < 32, lo, hi)
    return _tile_base(t, spec.head_dim // 16) + 32 * (b // 2) + 2 * (t % TILE) + b % 2


def v_scale_pos(spec: CacheSpec, t, b):
    t = np.asarray(t); b = np.asarray(b)
    t16 = t % TILE
    nb = spec.head_dim // 16
    return _tile_base(t, nb) + 4 * (nb * (t16 // 4) + b) + t16 % 4


# ------------------------------ cache model -------------------------------
def head_scale(scale, h) -> np.float32:
    """FP8 scale of KV head h: a per-tensor scalar (None = 1.0) or element h
    of a per-head sequence."""
    if scale is None:
        return np.float32(1.0)
    a = np.asarray(scale, dtype=np.float32)
    return np.float32(a) if a.ndim == 0 else a[h]


class OracleCache:
    """Byte-exact model of the cache buffers: arrays [num_pages, Hkv, block]."""

    def __init__(self, spec: CacheSpec, fill: int = 0):
        self.spec = spec
        cb, sb = spec.block_bytes()
        shape_c = (spec.num_pages, spec.num_kv_heads, cb)
        shape_s = (spec.num_pages, spec.num_kv_heads, sb)
        self.k_codes = np.full(shape_c, fill, dtype=np.uint8)
        self.v_codes = None if spec.kind == "mla" else np.full(shape_c, fill, dtype=np.uint8)
        self.k_scales = np.full(shape_s, fill, dtype=np.uint8) if sb else None
        self.v_scales = (np.full(shape_s, fill, dtype=np.uint8)
                         if sb and spec.kind != "mla" else None)
        if spec.kivi:
            assert spec.dtype in ("e4m3", "e5m2") and spec.kind == "gqa"
            # V token scales [num_pages, Hkv, page_size] binary32, kept as bytes
            # [num_pages, Hkv, 4 * page_size] like the device buffer
            self.v_scales = np.full((spec.num_pages, spec.num_kv_heads, 4 * spec.page_size), fill, dtype=np.uint8)

    def v_token_scales(self) -> np.ndarray:
        """KIVI: the V scale buffer as binary32 [num_pages, Hkv, page_size] (a view)."""
        return self.v_scales.view(np.float32)

    # -- writing codes for rows (page[i], head, t[i], all d) --
    def _put_codes(self, buf, pos_fn, page, head, t, codes):
        """codes [N, D]; page, t [N]."""
        d = np.arange(codes.shape[-1])[None, :]
        byte, nib = pos_fn(self.spec, t[:, None], d)
        byte = np.broadcast_to(byte, codes.shape)
        nib = np.broadcast_to(nib, codes.shape)
        pg = np.broadcast_to(page[:, None], codes.shape)
        if self.spec.dtype in ("e4m3", "e5m2"):
            buf[pg, head, byte] = codes
            return
        # two 4-bit codes per byte; both nibbles of a byte belong to the same
        # token in every layout, so each byte is written whole
        lo, hi = nib == 0, nib == 1
        assert np.array_equal(byte[lo], byte[hi])
        buf[pg[lo], head, byte[lo]] = (codes[lo] & 0xF) | ((codes[hi] & 0xF) << 4)

    def _put_scales(self, buf, pos_fn, page, head, t, sc):
        b = np.arange(sc.shape[-1])[None, :]
        pos = np.broadcast_to(pos_fn(self.spec, t[:, None], b), sc.shape)
        buf[np.broadcast_to(page[:, None], sc.shape), head, pos] = sc

    def store(self, k, v, slots, k_scale=None, v_scale=None):
        """Quantize and store tokens. k, v: float arrays [T, Hkv, D] (GQA) or
        k [T, Dk] with v None (MLA). slots[i] = page * page_size + offset;
        a negative slot skips the token. k_scale/v_scale: FP8 per-tensor
        scales (None = 1.0) or, per attention head (vLLM page, "Supported
        schemes"), sequences of Hkv scales, head h using element h; for NVFP4,
        k_scale is the global scale g. KIVI caches: k_scale [Hkv, D] channel
        scales (None = 1.0), v_scale unused (each token's own scale is
        computed here and written to the V scale buffer)."""
        s = self.spec
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        k = np.asarray(k, dtype=np.float64)[keep]
        if s.kind == "mla":
            k = k.reshape(k.shape[0], 1, s.head_dim)
        else:
            v = np.asarray(v, dtype=np.float64)[keep]
        page, t = slots[keep] // s.page_size, slots[keep] % s.page_size
        assert np.all(page < s.num_pages)
        for h in range(s.num_kv_heads):
            if s.kivi:
                fmt = E4M3 if s.dtype == "e4m3" else E5M2
                ksc = np.ones(s.head_dim, np.float32) if k_scale is None else np.asarray(k_scale, np.float32)[h]
                kc = Q.quantize_fp8(k[:, h], ksc[None, :], fmt)
                vc, vsc = Q.quantize_fp8_per_token(v[:, h], fmt)
                self._put_codes(self.k_codes, k_code_pos, page, h, t, kc)
                self._put_codes(self.v_codes, v_code_pos, page, h, t, vc)
                self.v_token_scales()[page, h, t] = vsc
            elif s.dtype in ("e4m3", "e5m2"):
                fmt = E4M3 if s.dtype == "e4m3" else E5M2
                kc = Q.quantize_fp8(k[:, h], head_scale(k_scale, h), fmt)
                vc = Q.quantize_fp8(v[:, h], head_scale(v_scale, h), fmt)
                self._put_codes(self.k_codes, k_code_pos, page, h, t, kc)
                self._put_codes(self.v_codes, v_code_pos, page, h, t, vc)
            elif s.dtype == "mx16":
                kc, ks = Q.quantize_mx16(k[:, h])
                vc, vs = Q.quantize_mx16(v[:, h])
                self._put_codes(self.k_codes, k_code_pos, page, h, t, kc)
                self._put_codes(self.v_codes, v_code_pos, page, h, t, vc)
                self._put_scales(self.k_scales, k_scale_pos, page, h, t, ks)
                self._put_scales(self.v_scales, v_scale_pos, page, h, t, vs)
            elif s.dtype == "nvfp4":
                kc, ks = Q.quantize_nvfp4(k[:, h], k_scale)
                self._put_codes(self.k_codes, k_code_pos, page, h, t, kc)
                self._put_scales(self.k_scales, k_scale_pos, page, h, t, ks)
            else:
                raise ValueError(s.dtype)

    # -- reading back dequantized rows --
    def _get_codes(self, buf, pos_fn, page, head, t, n):
        d = np.arange(n)[None, :]
        byte, nib = pos_fn(self.spec, t[:, None], d)
        raw = buf[page[:, None], head, byte].astype(np.int64)
        if self.spec.dtype in ("e4m3", "e5m2"):
            return raw
        return (raw >> (4 * nib)) & 0xF

    def dequant(self, page, t, head=0, which="k", k_scale=None, v_scale=None):
        """Dequantized float64 rows [N, dim] for tokens (page[i], t[i])."""
        s = self.spec
        page = np.atleast_1d(np.asarray(page, dtype=np.int64))
        t = np.atleast_1d(np.asarray(t, dtype=np.int64))
        n = s.head_dim
        if which == "k":
            codes = self._get_codes(self.k_codes, k_code_pos, page, head, t, n)
        else:
            if s.kind == "mla":
                return self.dequant(page, t, head, "k", k_scale)[:, : s.v_dim]
            codes = self._get_codes(self.v_codes, v_code_pos, page, head, t, n)
        if s.kivi:
            fmt = E4M3 if s.dtype == "e4m3" else E5M2
            if which == "k":
                ksc = np.ones(n, np.float32) if k_scale is None else np.asarray(k_scale, np.float32)[head]
                return decode(codes, fmt) * ksc.astype(np.float64)[None, :]
            vsc = self.v_token_scales()[page, head, t].astype(np.float64)
            return decode(codes, fmt) * vsc[:, None]
        if s.dtype in ("e4m3", "e5m2"):
            fmt = E4M3 if s.dtype == "e4m3" else E5M2
            sc = head_scale(k_scale if which == "k" else v_scale, head)
            return decode(codes, fmt) * float(sc)
        b = np.arange(n // 16)[None, :]
        if s.dtype == "mx16":
            sbuf, pfn = (self.k_scales, k_scale_pos) if which == "k" else (self.v_scales, v_scale_pos)
            sc = sbuf[page[:, None], head, pfn(s, t[:, None], b)]
            return Q.dequantize_mx16(codes, sc)
        sc = self.k_scales[page[:, None], head, k_scale_pos(s, t[:, None], b)]
        return Q.dequantize_nvfp4(codes, sc, k_scale)


# --------------------------------------------------------------------------
# dequantize_prev_kv (PR #21954 analysis page, "code analysis"): the FP4
# cache and its scales are turned into FP8 E4M3 (the dq_k_buffer /
# dq_v_buffer workspaces that create_buffers allocates) so that an FP8
# prefill kernel can read the quantized prefix; the review notes on the same
# page explain the FP8 target by the absence of an FP4 prefill kernel.
# Reading adopted (the page gives no formula): every token row of the listed
# pages is dequantized exactly and rounded once to binary32 (MX16: e2m1 * 2^e,
# exact; NVFP4: e2m1 * e4m3 * g), then re-encoded as E4M3 with a per-tensor
# scale s: code = encode_E4M3(fl32(x^ / s)), round to nearest even,
# saturating (s = None: 1.0). Output rows are token-major: GQA
# [n_pages, Hkv, page_size, D] for K and V, MLA [n_pages, page_size, Dk].
# --------------------------------------------------------------------------
def dequantize_prev_kv(cache: "OracleCache", pages, k_scale_out=None, v_scale_out=None, g=None):
    s = cache.spec
    assert s.dtype in ("mx16", "nvfp4")
    pages = np.asarray(pages, dtype=np.int64)
    t = np.arange(s.page_size)
    out = []
    for which in (("k", "v") if s.kind == "gqa" else ("k",)):
        sc = np.float32(1.0 if (k_scale_out if which == "k" else v_scale_out) is None
                        else (k_scale_out if which == "k" else v_scale_out))
        res = np.zeros((len(pages), s.num_kv_heads, s.page_size, s.head_dim), np.uint8)
        for i, pg in enumerate(pages):
            for h in range(s.num_kv_heads):
                x_hat = Q.fl32(cache.dequant(np.full(s.page_size, pg), t, h, which, g))
                res[i, h] = Q.quantize_fp8(x_hat, sc, E4M3)
        out.append(res if s.kind == "gqa" else res[:, 0])
    return out[0], (out[1] if s.kind == "gqa" else None)
