"""Seeded synthetic inputs for the quantized paged KV store and decode attention.

This module only draws random inputs (BF16 Q/K/V, sequence lengths, page
tables, slot mappings). It performs none of the method's arithmetic, so both
the HIP path and the CPU oracle may consume what it produces.

Distributions follow the K/V structure described on the "KV cache
quantization mechanism and traps" page (section on why Key and Value
distributions differ): Key outliers concentrate in a few channels that stay
large across tokens, Value varies along the token direction. The workload
shapes are the model shapes the pages name (Llama-3-8B/70B, Qwen3-235B-A22B,
DeepSeek-R1 MLA); their accuracy datasets are not used: these seeded caches
stand in for them.

Every random block is drawn from ``numpy.random.default_rng([seed, tag, ...])``
so any sequence / token chunk can be regenerated alone (the oracle regenerates
only the sequences it checks). Values are drawn in float32 and rounded to
BF16 (round to nearest even) on the host.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

CHUNK = 1024  # tokens per independently seeded block


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "e4m3" | "e5m2" | "mx16" | "nvfp4"
    kind: str                  # "gqa" | "mla"
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int              # GQA D; MLA Dk = latent + rope
    v_dim: int                 # GQA D; MLA Dv = latent
    page_size: int
    max_len: int
    min_len: int               # == max_len for fixed-length workloads
    new_tokens: int            # tokens stored per sequence by the timed step
    dist: str                  # "tiny" | "llama" | "qwen" | "mla"
    scale_mode: str = "amax"   # FP8: "amax" (calibrated per tensor) | "amax_head" (per KV head) | "one"
    #                            | "kivi" (K per channel, calibrated; V per token at store)
    seed: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 1 sequence, 1 layer, 4 query heads / 1 KV head, D 64, context 256
    "tiny": Workload("tiny", "e4m3", "gqa", 1, 4, 1, 64, 64, 16, 256, 256, 1, "tiny", seed=1),
    # Llama-3-8B decode layer, batch 8, context 20,480
    "llama3_8b": Workload("llama3_8b", "e4m3", "gqa", 8, 32, 8, 128, 128, 16, 20480, 20480, 1, "llama", seed=2),
    # Llama-3-70B one-GPU share, batch 32, lengths uniform in [16K, 32K]
    "llama3_70b": Workload("llama3_70b", "e4m3", "gqa", 32, 64, 8, 128, 128, 16, 32768, 16384, 1, "llama", seed=3),
    # Qwen3-235B-A22B attention shape, batch 64, context 32,768, 2,048-token chunk append
    "qwen3_235b": Workload("qwen3_235b", "mx16", "gqa", 64, 64, 4, 128, 128, 16, 32768, 32768, 2048, "qwen", seed=4),
    # DeepSeek-R1 MLA, 128 heads over one 512+64 latent, batch 64, context 65,536
    "dsr1_mla": Workload("dsr1_mla", "nvfp4", "mla", 64, 128, 1, 576, 512, 64, 65536, 65536, 1, "mla", seed=5),
}


# ------------------------------------------------------------------ bf16 --
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------ structure --
def seq_lens(w: Workload) -> np.ndarray:
    if w.min_len == w.max_len:
        return np.full(w.batch, w.max_len, dtype=np.int32)
    rng = np.random.default_rng([w.seed, 11])
    return rng.integers(w.min_len, w.max_len + 1, size=w.batch).astype(np.int32)


def page_table(w: Workload, lens: np.ndarray, spare_pages: int = 0, identity: bool = False):
    """Random permutation of the page pool handed out to the sequences in order.

    Returns (table int32 [B, max_pages] with -1 past each sequence's pages,
    num_pages of the pool)."""
    P = w.page_size
    need = [(int(L) + P - 1) // P for L in lens]
    total = sum(need) + spare_pages
    max_pages = max(1, (w.max_len + P - 1) // P)
    perm = (np.arange(total) if identity
            else np.random.default_rng([w.seed, 12]).permutation(total)).astype(np.int32)
    table = np.full((len(lens), max_pages), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, total


def slots_for(table_row: np.ndarray, positions: np.ndarray, page_size: int) -> np.ndarray:
    """Cache slot (page * page_size + offset) of each token position."""
    positions = np.asarray(positions, dtype=np.int64)
    return table_row[positions // page_size].astype(np.int64) * page_size + positions % page_size


# -------------------------------------------------------------- values --
def _outlier_channels(w: Workload, count: int) -> np.ndarray:
    rng = np.random.default_rng([w.seed, 13])
    dim = w.head_dim
    return np.stack([rng.choice(dim, size=count, replace=False) for _ in range(w.kv_heads)])


def _chunk_kv(w: Workload, b: int, c: int):
    """float32 K, V for tokens [c*CHUNK, (c+1)*CHUNK) of sequence b."""
    rng = np.random.default_rng([w.seed, 14, b, c])
    n, H, D = CHUNK, w.kv_heads, w.head_dim
    k = rng.standard_normal((n, H, D), dtype=np.float32)
    if w.dist == "tiny":
        ch = _outlier_channels(w, 2)
        for h in range(H):
            k[:, h, ch[h]] = (8.0 + 4.0 * rng.standard_normal((n, ch.shape[1]), dtype=np.float32))
    elif w.dist == "llama":
        ch = _outlier_channels(w, 4)
        for h in range(H):
            k[:, h, ch[h]] *= 10.0
    elif w.dist == "qwen":
        ch = _outlier_channels(w, 8)
        for h in range(H):
            k[:, h, ch[h]] = rng.standard_t(3.0, size=(n, ch.shape[1])).astype(np.float32)
    elif w.dist == "mla":
        ch = _outlier_channels(w, 16)
        k[:, 0, ch[0]] *= 8.0
    if w.kind == "mla":
        return k, None
    v = rng.standard_normal((n, H, D), dtype=np.float32)
    if w.dist == "llama":
        v *= rng.lognormal(0.0, 0.5, size=(n, 1, 1)).astype(np.float32)
    return k, v


def kv_rows(w: Workload, b: int, t0: int, t1: int):
    """BF16 bits of K and V for positions [t0, t1) of sequence b.

    GQA: k, v uint16 [n, Hkv, D]. MLA: k uint16 [n, Dk] (the latent row), v None."""
    ks, vs = [], []
    for c in range(t0 // CHUNK, (t1 - 1) // CHUNK + 1 if t1 > t0 else t0 // CHUNK):
        k, v = _chunk_kv(w, b, c)
        lo = max(t0 - c * CHUNK, 0)
        hi = min(t1 - c * CHUNK, CHUNK)
        ks.append(k[lo:hi])
        if v is not None:
            vs.append(v[lo:hi])
    if not ks:
        shape = (0, w.kv_heads, w.head_dim)
        k = np.zeros(shape, np.float32)
        v = None if w.kind == "mla" else np.zeros(shape, np.float32)
    else:
        k = np.concatenate(ks)
        v = np.concatenate(vs) if vs else None
    kb = bf16_bits(k)
    if w.kind == "mla":
        return kb.reshape(kb.shape[0], w.head_dim), None
    return kb, bf16_bits(v)


def queries(w: Workload) -> np.ndarray:
    """BF16 bits of the decode queries [B, Hq, Dk], N(0, 1)."""
    rng = np.random.default_rng([w.seed, 15])
    return bf16_bits(rng.standard_normal((w.batch, w.q_heads, w.head_dim), dtype=np.float32))


def sm_scale(w: Workload) -> float:
    """Softmax scale 1/sqrt(dot-product length) (the pages leave it open)."""
    return float(1.0 / np.sqrt(w.head_dim))


def random_cache_bytes(shapes: dict, dtype: str, seed: int, mx_codes=(0, 191)) -> dict:
    """Seeded random contents for the buffers of an FP4 cache, {name: shape}
    -> {name: uint8 array}: code buffers uniform over all 256 byte values
    (every E2M1 code in both nibbles); MX16 E8M0 scale codes from
    [mx_codes[0], mx_codes[1]), half of them within 10 of the middle; NVFP4
    E4M3 scale codes over every non-NaN magnitude with a random sign. Buffers
    are drawn in the order k_codes, v_codes, k_scales, v_scales."""
    rng = np.random.default_rng(seed)
    out = {}
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        shape = shapes.get(name)
        if shape is None:
            continue
        if name.endswith("codes"):
            out[name] = rng.integers(0, 256, shape, dtype=np.uint8)
        elif dtype == "mx16":
            mid = (mx_codes[0] + mx_codes[1]) // 2
            near = rng.integers(max(mx_codes[0], mid - 10), min(mx_codes[1], mid + 11), shape)
            wide = rng.integers(mx_codes[0], mx_codes[1], shape)
            out[name] = np.where(rng.random(shape) < 0.5, near, wide).astype(np.uint8)
        else:
            mag = rng.integers(0, 0x7F, shape)
            out[name] = (mag | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)
    return out


def extend_inputs(seed: int, prefix_lens, chunk_lens, hkv: int, group: int, head_dim: int, page_size: int,
                  max_code: int = 0x58) -> dict:
    """Seeded inputs of one extend-attention call: BF16 bits of Q [Nq, Hq, D]
    and of the chunk K/V [Nq, Hkv, D] (N(0,1)), chunk offsets cu_q [B+1],
    prefix_len [B], and E4M3 prefix workspaces dq_k / dq_v [n_pages, Hkv, P, D]
    of random codes with magnitude code <= max_code (0x58: |value| <= 30, no
    NaN) and a random sign; sequence b's prefix pages are consecutive from
    page_off[b], the sequences' page ranges in a shuffled order."""
    rng = np.random.default_rng([seed, 77])
    prefix_lens = np.asarray(prefix_lens, np.int32)
    chunk_lens = np.asarray(chunk_lens, np.int32)
    B = len(prefix_lens)
    npg = (prefix_lens + page_size - 1) // page_size
    order = rng.permutation(B)
    page_off = np.zeros(B, np.int32)
    off = 0
    for b in order:
        page_off[b] = off
        off += int(npg[b])
    n_pages = max(off, 1)
    shape = (n_pages, hkv, page_size, head_dim)
    codes = lambda: (rng.integers(0, max_code + 1, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)
    dq_k, dq_v = codes(), codes()
    cu = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int32)
    nq = int(cu[-1])
    q = bf16_bits(rng.standard_normal((nq, hkv * group, head_dim), dtype=np.float32))
    k = bf16_bits(rng.standard_normal((nq, hkv, head_dim), dtype=np.float32))
    v = bf16_bits(rng.standard_normal((nq, hkv, head_dim), dtype=np.float32))
    return dict(q=q, k_new=k, v_new=v, cu_q=cu, prefix_len=prefix_lens, page_off=page_off, dq_k=dq_k, dq_v=dq_v)
