"""Case builder shared by the GPU parity tests (not a test module).

A Case draws one workload's seeded BF16 inputs, runs the HIP path through the
C ABI (scale calibration, prefill store, append store, decode) and, for a
chosen subset of sequences, replays the same inputs through the CPU oracle.
Both sides only share the generated inputs.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

import quantized_paged_kv_store_amd as K
from oracle import quantize as Q
from oracle.attention import decode_attention, softmax_attention
from oracle.formats import E4M3, E5M2
from oracle.paged import CacheSpec, OracleCache
from quantized_paged_kv_store_amd import inputs as I

# padding bytes of never-written slots: NaN codes for FP8 and E8M0 scales
FILL = {"e4m3": 0x7F, "e5m2": 0x7F, "mx16": 0xFF, "nvfp4": 0xFF}
TOL_MAX_ABS = 4e-3
CACHE_SCALE_MODE = {"amax_head": "head", "kivi": "kivi"}


def cache_scale_mode(w) -> str:
    """The cache descriptor's scale mode for a workload's scale_mode."""
    return CACHE_SCALE_MODE.get(w.scale_mode, "tensor")


TOL_REL_L2 = 1e-3
_THREADS = min(16, os.cpu_count() or 4)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a - b))


def assert_close(got, want, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mab = float(np.max(np.abs(got - want))) if got.size else 0.0
    r = rel_l2(got, want)
    assert mab <= TOL_MAX_ABS and r <= TOL_REL_L2, f"{what}: max-abs {mab:.3e} rel-L2 {r:.3e}"
    return mab, r


class Case:
    def __init__(self, w: I.Workload, device="cuda", identity=False, spare_pages=0, lens=None, data=None, fill=None):
        """data: the host inputs of another Case of the same seed/shape (reused);
        fill: byte value of never-written slots (default FILL[dtype])."""
        self.w = w
        self.fill = FILL[w.dtype] if fill is None else fill
        self.data = data
        self.dev = torch.device(device)
        self.lens = I.seq_lens(w) if lens is None else np.asarray(lens, np.int32)
        self.table, self.npages = I.page_table(w, self.lens, spare_pages, identity)
        self.max_len = int(max(int(self.lens.max()), 1))
        self.prefill = np.maximum(self.lens - w.new_tokens, 0)
        self._rows = {}

    # ------------------------------------------------------------ inputs --
    def rows(self, b, t0, t1):
        return I.kv_rows(self.w, b, t0, t1)

    def _gather(self, ranges):
        """BF16 rows for [(b, t0, t1)] concatenated (threaded generation)."""
        if not ranges:
            return None, None, np.zeros(0, np.int64)
        with cf.ThreadPoolExecutor(_THREADS) as ex:
            parts = list(ex.map(lambda r: self.rows(*r), ranges))
        k = np.concatenate([p[0] for p in parts])
        v = None if self.w.kind == "mla" else np.concatenate([p[1] for p in parts])
        slots = np.concatenate([I.slots_for(self.table[b], np.arange(t0, t1), self.w.page_size)
                                for b, t0, t1 in ranges])
        return k, v, slots

    def _to_dev(self, a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)

    def _bf16(self, a):
        return self._to_dev(a).view(torch.bfloat16)

    # ------------------------------------------------------------ HIP path --
    def run_gpu(self, decode=True, append=False, split_target=0):
        """append: the last token of every sequence is not stored separately;
        kvq_decode_append stores it and decodes in one call (one new token per
        sequence required). append without decode leaves those tokens, as
        self.append_rows (device BF16 [B, ...] K and V), to the caller's own
        append call. split_target: decode workgroups the split planner aims
        at (0 = the library default)."""
        w = self.w
        assert not append or w.new_tokens == 1
        self.cache = K.kvq_alloc_pages(w.dtype, w.kind, w.kv_heads, w.head_dim, w.v_dim, w.page_size,
                                       self.npages, device=self.dev, fill=self.fill,
                                       scale_mode=cache_scale_mode(w))
        K.set_split_target(self.cache, split_target)
        pre = [(b, 0, int(self.prefill[b])) for b in range(w.batch) if self.prefill[b] > 0]
        new = [(b, int(self.prefill[b]), int(self.lens[b])) for b in range(w.batch) if self.lens[b] > self.prefill[b]]
        if self.data is None:
            self.data = {"pre": self._gather(pre), "new": self._gather(new)}
        kp, vp, sp = self.data["pre"]
        self.k_scale = self.v_scale = None
        if kp is not None and len(kp):
            kd, sd = self._bf16(kp), self._to_dev(sp)
            vd = None if vp is None else self._bf16(vp)
            if w.dtype in ("e4m3", "e5m2") and w.scale_mode == "kivi":
                self.k_scale = K.kvq_compute_scale(self.cache, kd)      # K channel scales; V per token
            elif w.dtype in ("e4m3", "e5m2") and w.scale_mode in ("amax", "amax_head"):
                if w.dist == "tiny":   # one scale for K and V jointly
                    self.k_scale = K.kvq_compute_scale(self.cache, kd, vd)
                    self.v_scale = self.k_scale
                else:
                    self.k_scale = K.kvq_compute_scale(self.cache, kd)
                    self.v_scale = K.kvq_compute_scale(self.cache, vd)
            elif w.dtype == "nvfp4":
                self.k_scale = K.kvq_compute_scale(self.cache, kd)
            K.kvq_store(self.cache, kd, vd, sd, self.k_scale, self.v_scale)
            del kd, vd, sd
        elif w.dtype == "nvfp4":
            self.k_scale = torch.ones(1, dtype=torch.float32, device=self.dev)
        self.host_amax = None
        if kp is not None and len(kp):
            if w.scale_mode == "amax_head":     # [Hkv] magnitudes per head (BF16 bits order like values)
                mag = lambda a: I.bf16_to_f32((a.reshape(len(a), w.kv_heads, -1) & 0x7FFF).max(axis=(0, 2)).astype(np.uint16))
                self.host_amax = (mag(kp), None if vp is None else mag(vp))
            elif w.scale_mode == "kivi":        # [Hkv, D] K magnitudes per channel
                mag = I.bf16_to_f32((kp.reshape(len(kp), w.kv_heads, -1) & 0x7FFF).max(axis=0).astype(np.uint16))
                self.host_amax = (mag, None)
            else:
                ak = float(np.abs(I.bf16_to_f32(kp)).max())
                av = None if vp is None else float(np.abs(I.bf16_to_f32(vp)).max())
                self.host_amax = (ak, av)
        del kp, vp
        kn, vn, sn = self.data["new"]
        self.new_inputs = (kn, vn, sn)
        if kn is not None and len(kn) and not append:
            self.new_dev = (self._bf16(kn), None if vn is None else self._bf16(vn), self._to_dev(sn))
            K.kvq_store(self.cache, *self.new_dev, self.k_scale, self.v_scale)
        self.q = I.queries(w)
        self.q_dev = self._bf16(self.q)
        self.table_dev = self._to_dev(self.table)
        self.lens_dev = self._to_dev(self.lens.astype(np.int32))
        if append:
            # row b = the token at position L_b - 1 (zeros where L_b = 0: nothing is stored)
            row = (w.kv_heads, w.head_dim) if w.kind == "gqa" else (w.head_dim,)
            kb = np.zeros((w.batch, *row), np.uint16)
            vb = None if w.kind == "mla" else np.zeros((w.batch, *row), np.uint16)
            i = 0
            for b in range(w.batch):
                if self.lens[b] > self.prefill[b]:
                    kb[b] = kn[i].reshape(row)
                    if vb is not None:
                        vb[b] = vn[i].reshape(row)
                    i += 1
            self.append_rows = (self._bf16(kb), None if vb is None else self._bf16(vb))
            if decode:
                self.out, self.lse = K.kvq_decode_append(
                    self.cache, *self.append_rows, self.q_dev, self.table_dev, self.lens_dev, self.max_len,
                    I.sm_scale(w), self.k_scale, self.v_scale)
        elif decode:
            self.out, self.lse = K.kvq_decode(self.cache, self.q_dev, self.table_dev, self.lens_dev, self.max_len,
                                              I.sm_scale(w), self.k_scale, self.v_scale)
        torch.cuda.synchronize(self.dev)
        return self

    def gpu_scales(self):
        if self.w.scale_mode == "kivi":
            return self.k_scale.cpu().numpy().astype(np.float32).reshape(self.w.kv_heads, -1), None
        if self.w.scale_mode == "amax_head":
            f = lambda t: None if t is None else t.cpu().numpy().astype(np.float32)
        else:
            f = lambda t: None if t is None else np.float32(t.cpu().numpy()[0])
        return f(self.k_scale), f(self.v_scale)

    # -------------------------------------------------------------- oracle --
    def oracle_scales(self):
        w = self.w
        if self.host_amax is None:
            return (np.float32(1.0) if w.dtype == "nvfp4" else None), None
        ak, av = self.host_amax
        if w.dtype in ("e4m3", "e5m2") and w.scale_mode == "kivi":
            fmt = E4M3 if w.dtype == "e4m3" else E5M2
            return Q.fp8_channel_scales(np.asarray(ak, np.float64)[None], fmt), None
        if w.dtype in ("e4m3", "e5m2") and w.scale_mode == "amax_head":
            fmt = E4M3 if w.dtype == "e4m3" else E5M2
            per_head = lambda a: Q.fp8_head_scales(np.asarray(a, np.float64)[None, :, None], fmt)
            if w.dist == "tiny":
                s = per_head(np.maximum(ak, av))
                return s, s
            return per_head(ak), per_head(av)
        if w.dtype in ("e4m3", "e5m2") and w.scale_mode == "amax":
            fmt = E4M3 if w.dtype == "e4m3" else E5M2
            if w.dist == "tiny":
                s = Q.fp8_scale(max(ak, av), fmt)
                return s, s
            return Q.fp8_scale(ak, fmt), Q.fp8_scale(av, fmt)
        if w.dtype == "nvfp4":
            return Q.nvfp4_global_scale(ak), None
        return None, None

    def oracle(self, batch_ids):
        """Oracle cache over the pages of `batch_ids` only (compacted ids)."""
        w = self.w
        P = w.page_size
        pages = []
        for b in batch_ids:
            n = (int(self.lens[b]) + P - 1) // P
            pages.extend(int(p) for p in self.table[b, :n])
        remap = {p: i for i, p in enumerate(pages)}
        otable = np.full_like(self.table, -1)
        for b in batch_ids:
            n = (int(self.lens[b]) + P - 1) // P
            otable[b, :n] = [remap[int(p)] for p in self.table[b, :n]]
        spec = CacheSpec(w.dtype, w.kind, w.kv_heads, w.head_dim, w.v_dim, P, max(len(pages), 1),
                         kivi=w.scale_mode == "kivi")
        oc = OracleCache(spec, fill=self.fill)
        ks, vs = self.oracle_scales()
        for b in batch_ids:
            L = int(self.lens[b])
            k, v = self.rows(b, 0, L)
            slots = I.slots_for(otable[b], np.arange(L), P)
            kf = I.bf16_to_f32(k)
            vf = None if v is None else I.bf16_to_f32(v)
            oc.store(kf, vf, slots, k_scale=ks, v_scale=vs)
        return oc, otable, np.array(pages, np.int64), (ks, vs)

    def oracle_decode(self, batch_ids):
        oc, otable, pages, (ks, vs) = self.oracle(batch_ids)
        qf = I.bf16_to_f32(self.q).astype(np.float64)
        out, lse = decode_attention(oc, qf, otable, self.lens, I.sm_scale(self.w), ks, vs, batch_ids=batch_ids)
        return out, lse, oc, pages

    def unquantized(self, b):
        """Attention on the raw BF16 K/V of sequence b (information only)."""
        w = self.w
        L = int(self.lens[b])
        k, v = self.rows(b, 0, L)
        kf = I.bf16_to_f32(k).astype(np.float64)
        qf = I.bf16_to_f32(self.q[b]).astype(np.float64)
        if w.kind == "mla":
            o, _ = softmax_attention(qf, kf, kf[:, :w.v_dim], I.sm_scale(w))
            return o
        vf = I.bf16_to_f32(v).astype(np.float64)
        G = w.group
        outs = []
        for h in range(w.kv_heads):
            o, _ = softmax_attention(qf[h * G:(h + 1) * G], kf[:, h], vf[:, h], I.sm_scale(w))
            outs.append(o)
        return np.concatenate(outs)

    # ----------------------------------------------------- byte compare --
    def gpu_pages(self, name, pages):
        """GPU bytes of buffer `name` for physical pages, shaped [n, Hkv, block]."""
        buf = self.cache.view(name)
        blk = buf.numel() // (self.npages * self.w.kv_heads)
        t = buf.view(self.npages, self.w.kv_heads, blk)
        idx = torch.from_numpy(np.asarray(pages, np.int64)).to(self.dev)
        return t.index_select(0, idx).cpu().numpy()
