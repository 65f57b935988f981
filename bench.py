#!/usr/bin/env python3
"""Benchmark of the quantized paged KV decode hot path on one MI355X.

One step = kvq_store of the new token(s) of every sequence + kvq_decode over
the whole cache (split-context decode kernel and its combine), on seeded
synthetic data already resident in HBM, launched eagerly on torch's current
stream (--graph replays the same launches from captured HIP graphs instead:
the library's calls allocate nothing and never synchronize; on this machine a
graph replay costs more than the eager launches it replaces). Prints ONE JSON
line.

value = algorithmic KV bytes per step (codes + block scales of every cached
token) / step time. Several copies of the cache are rotated so consecutive
steps do not hit the 256 MB Infinity Cache.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn effective KV GB/s (% HBM peak), 8B-shape FP8 bs8 ctx20K"
PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E, vendor figure
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, vendor figure
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 matrix peak, vendor figure


def measured_traffic(w, op="decode", fp8q=False):
    """HBM bytes per launch of the decode (op "decode"), dequantize_prev_kv
    (op "dequant_prev") or extend attention (op "extend") kernel from the
    committed rocprofv3 counter runs, or None when no measurement exists for
    this workload or the kernel's sources changed since it was taken."""
    import hashlib
    if op == "decode":
        kind = "gqa" if w.kind == "gqa" else "mla"
        mode = {"amax_head": "_head", "kivi": "_kivi", "one": "_one"}.get(w.scale_mode, "") + ("_fp8q" if fp8q else "")
        path = os.path.join(ROOT, "profiles", f"kvq_decode_{kind}_{w.name}_{w.dtype}{mode}_traffic.json")
    elif op == "extend":
        path = os.path.join(ROOT, "profiles", f"kvq_extend_attn_{w.name}_traffic.json")
    else:
        path = os.path.join(ROOT, "profiles", f"kvq_dequant_prev_{w.dtype}_{w.name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return int(round(1024 * (rec["fetch_size_kib_per_dispatch"] * rec["fetch_scale"]
                             + rec["write_size_kib_per_dispatch"] * rec["write_scale"])))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def setup(w, dev, rotate, fp8q=False):
    import torch

    import quantized_paged_kv_store_amd as K
    from quantized_paged_kv_store_amd import inputs as I

    lens = I.seq_lens(w)
    table, npages = I.page_table(w, lens)
    max_len = int(lens.max())
    pre = np.maximum(lens - w.new_tokens, 0)
    cache = K.kvq_alloc_pages(w.dtype, w.kind, w.kv_heads, w.head_dim, w.v_dim, w.page_size, npages,
                              device=dev, fill=0,
                              scale_mode={"amax_head": "head", "kivi": "kivi"}.get(w.scale_mode, "tensor"))
    # prefill, one sequence at a time (bounded host memory); scales first need the
    # whole prefill, so K (and V) are staged on the device
    n_pre = int(pre.sum())
    row = (w.kv_heads, w.head_dim) if w.kind == "gqa" else (w.head_dim,)
    kd = torch.empty((n_pre, *row), dtype=torch.bfloat16, device=dev)
    vd = torch.empty((n_pre, *row), dtype=torch.bfloat16, device=dev) if w.kind == "gqa" else None
    sd = torch.empty(n_pre, dtype=torch.int64, device=dev)
    off = 0
    for b in range(w.batch):
        n = int(pre[b])
        if n == 0:
            continue
        k, v = I.kv_rows(w, b, 0, n)
        kd[off:off + n] = torch.from_numpy(k).view(torch.bfloat16).reshape(n, *row).to(dev)
        if vd is not None:
            vd[off:off + n] = torch.from_numpy(v).view(torch.bfloat16).to(dev)
        sd[off:off + n] = torch.from_numpy(I.slots_for(table[b], np.arange(n), w.page_size)).to(dev)
        off += n
    ks = vs = None
    if w.dtype in ("e4m3", "e5m2") and w.scale_mode == "kivi":
        ks = K.kvq_compute_scale(cache, kd)          # K channel scales; V scales per token at store
    elif w.dtype in ("e4m3", "e5m2") and w.scale_mode in ("amax", "amax_head"):
        ks = K.kvq_compute_scale(cache, kd, vd) if w.dist == "tiny" else K.kvq_compute_scale(cache, kd)
        vs = ks if w.dist == "tiny" else K.kvq_compute_scale(cache, vd)
    elif w.dtype == "nvfp4":
        ks = K.kvq_compute_scale(cache, kd)
    K.kvq_store(cache, kd, vd, sd, ks, vs)
    torch.cuda.synchronize(dev)
    # the bulk store once more, timed: it writes the same bytes again
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    K.kvq_store(cache, kd, vd, sd, ks, vs)
    e1.record()
    torch.cuda.synchronize(dev)
    bulk_ms = e0.elapsed_time(e1)
    bulk_bytes = kd.numel() * 2 * (2 if vd is not None else 1) + n_pre * K.kvq_bytes_per_token(cache.desc)
    bulk = {"tokens": n_pre, "ms": round(bulk_ms, 4), "GBps": round(bulk_bytes / (bulk_ms * 1e-3) / 1e9, 1),
            "bytes": "BF16 rows read + codes and scales written"}
    del kd, vd, sd
    caches = [cache] + [K.Cache(cache.desc, cache.memory.clone()) for _ in range(rotate - 1)]
    # the new tokens stored by every step
    kn, vn, sn = [], [], []
    for b in range(w.batch):
        k, v = I.kv_rows(w, b, int(pre[b]), int(lens[b]))
        kn.append(k)
        if v is not None:
            vn.append(v)
        sn.append(I.slots_for(table[b], np.arange(int(pre[b]), int(lens[b])), w.page_size))
    new_k = torch.from_numpy(np.concatenate(kn)).view(torch.bfloat16).to(dev)
    new_v = torch.from_numpy(np.concatenate(vn)).view(torch.bfloat16).to(dev) if vn else None
    new_s = torch.from_numpy(np.concatenate(sn)).to(dev)
    q = torch.from_numpy(I.queries(w)).view(torch.bfloat16).to(dev)
    table_d = torch.from_numpy(table).to(dev)
    lens_d = torch.from_numpy(lens.astype(np.int32)).to(dev)
    out = torch.empty((w.batch, w.q_heads, w.v_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.q_heads), dtype=torch.float32, device=dev)
    need = K.kvq_decode_workspace_bytes(cache, w.batch, w.q_heads, max_len)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    # one new token per sequence: the same rows as [B, Hkv, D] ([B, 576] for MLA) for kvq_decode_append
    new_rows = None
    if w.new_tokens == 1 and int((lens >= 1).sum()) == w.batch:
        new_rows = (new_k.view(w.batch, *row), None if new_v is None else new_v.view(w.batch, *row))
    # FP8-domain attention: query scales calibrated once on the step's queries
    qs = K.kvq_compute_q_scale(cache, q) if fp8q else None
    return dict(caches=caches, new=(new_k, new_v, new_s), new_rows=new_rows, q=q, table=table_d, lens=lens_d, lens_h=lens,
                max_len=max_len, ks=ks, vs=vs, out=out, lse=lse, ws=ws, sm=I.sm_scale(w),
                bpt=K.kvq_bytes_per_token(cache.desc), fp8q=fp8q, qs=qs, bulk_store=bulk)


def run_loop(st, steps, do_store, do_decode, offset=0, fused=False):
    """fused: each step appends its token and decodes in one kvq_decode_append call."""
    import quantized_paged_kv_store_amd as K
    caches = st["caches"]
    for i in range(steps):
        c = caches[(i + offset) % len(caches)]
        if fused and st["fp8q"]:
            K.kvq_decode_append_fp8q(c, st["new_rows"][0], st["new_rows"][1], st["q"], st["table"], st["lens"],
                                     st["max_len"], st["sm"], st["qs"], st["ks"], st["vs"], out=st["out"],
                                     lse=st["lse"], workspace=st["ws"])
            continue
        if fused:
            K.kvq_decode_append(c, st["new_rows"][0], st["new_rows"][1], st["q"], st["table"], st["lens"],
                                st["max_len"], st["sm"], st["ks"], st["vs"], out=st["out"], lse=st["lse"],
                                workspace=st["ws"])
            continue
        if do_store:
            K.kvq_store(c, *st["new"], st["ks"], st["vs"])
        if do_decode and st["fp8q"]:
            K.kvq_decode_fp8q(c, st["q"], st["table"], st["lens"], st["max_len"], st["sm"], st["qs"], st["ks"],
                              st["vs"], out=st["out"], lse=st["lse"], workspace=st["ws"])
        elif do_decode:
            K.kvq_decode(c, st["q"], st["table"], st["lens"], st["max_len"], st["sm"], st["ks"], st["vs"],
                         out=st["out"], lse=st["lse"], workspace=st["ws"])


def capture(st, do_store, do_decode, fused=False):
    """One HIP graph per rotated cache copy holding the step's launches (the
    library neither allocates nor synchronizes, so the calls are capturable)."""
    import torch
    graphs = []
    for r in range(len(st["caches"])):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_loop(st, 1, do_store, do_decode, offset=r, fused=fused)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def timed(st, steps, do_store, do_decode, graphs=None, fused=False):
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if graphs:
        for i in range(steps):
            graphs[i % len(graphs)].replay()
    else:
        run_loop(st, steps, do_store, do_decode, fused=fused)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps     # ms per iteration


def cpu_baseline(w, seconds_hint=20.0, fp8q=False):
    """The float64 oracle, untuned, on a bounded sample of the same workload
    (fp8q: the FP8-domain oracle, query scales calibrated on the step's queries)."""
    from oracle.attention import decode_attention, decode_attention_fp8q, decode_attention_mla_fp8q
    from oracle.formats import E4M3, E5M2
    from oracle import quantize as Q
    from oracle.paged import CacheSpec, OracleCache
    from quantized_paged_kv_store_amd import inputs as I

    lens = I.seq_lens(w)
    b = 0
    L = int(lens[b])
    P = w.page_size
    npg = (L + P - 1) // P
    table = np.full((w.batch, max(1, (w.max_len + P - 1) // P)), -1, np.int32)
    table[b, :npg] = np.arange(npg)
    k, v = I.kv_rows(w, b, 0, L)
    kf = I.bf16_to_f32(k)
    vf = None if v is None else I.bf16_to_f32(v)
    ks = vs = None
    if w.dtype in ("e4m3", "e5m2") and w.scale_mode == "amax":
        fmt = E4M3 if w.dtype == "e4m3" else E5M2
        ks, vs = Q.fp8_scale(np.abs(kf).max(), fmt), Q.fp8_scale(np.abs(vf).max(), fmt)
    elif w.dtype in ("e4m3", "e5m2") and w.scale_mode == "amax_head":
        fmt = E4M3 if w.dtype == "e4m3" else E5M2
        ks, vs = Q.fp8_head_scales(kf, fmt), Q.fp8_head_scales(vf, fmt)
    elif w.dtype in ("e4m3", "e5m2") and w.scale_mode == "kivi":
        ks = Q.fp8_channel_scales(kf, E4M3 if w.dtype == "e4m3" else E5M2)
    elif w.dtype == "nvfp4":
        ks = Q.nvfp4_global_scale(np.abs(kf).max())
    oc = OracleCache(CacheSpec(w.dtype, w.kind, w.kv_heads, w.head_dim, w.v_dim, P, npg, kivi=w.scale_mode == "kivi"))
    t0 = time.perf_counter()
    oc.store(kf, vf, I.slots_for(table[b], np.arange(L), P), k_scale=ks, v_scale=vs)
    t_codec = time.perf_counter() - t0
    q = I.bf16_to_f32(I.queries(w)).astype(np.float64)
    if fp8q:
        qs = Q.fp8_query_scales(q, per_head=w.scale_mode == "amax_head")

    def decode_once():
        if fp8q and w.kind == "mla":
            decode_attention_mla_fp8q(oc, q, table, lens, I.sm_scale(w), qs, g=ks, batch_ids=[b])
        elif fp8q:
            decode_attention_fp8q(oc, q, table, lens, I.sm_scale(w), qs, ks, vs, batch_ids=[b])
        else:
            decode_attention(oc, q, table, lens, I.sm_scale(w), ks, vs, batch_ids=[b])
    t0 = time.perf_counter()
    decode_once()
    t_dec = time.perf_counter() - t0
    # the same decode with one host thread (BLAS limited to 1), reported beside
    t1 = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            decode_once()
            t1 = time.perf_counter() - t0
    except ImportError:
        pass
    rows = 2 * w.kv_heads if w.kind == "gqa" else 1
    bits = 8.0 if w.dtype in ("e4m3", "e5m2") else 4.5
    nbytes = L * rows * w.head_dim * bits / 8
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return {"value": round(nbytes / t_dec / 1e9, 4), "unit": "GB/s", "cores": int(blas),
            "host_cores_available": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"sequence {b} of {w.batch} ({L} tokens, all {w.kv_heads} KV heads): float64 oracle "
                      f"dequant + attention {t_dec:.2f} s; its quantize-and-store of the same tokens "
                      f"{t_codec:.2f} s (not in value)",
            "decode_s": round(t_dec, 3), "codec_s": round(t_codec, 3),
            "value_1_thread": None if t1 is None else round(nbytes / t1 / 1e9, 4),
            "decode_s_1_thread": None if t1 is None else round(t1, 3)}


def dequant_prev_cpu_baseline(w, n_pages=None):
    """The oracle's dequantize_prev_kv, untuned, on the pages of sequence 0
    of the same workload (at most 2,048 pages)."""
    from oracle import quantize as Q
    from oracle.paged import CacheSpec, OracleCache, dequantize_prev_kv
    from quantized_paged_kv_store_amd import inputs as I

    P = w.page_size
    if n_pages is None:
        n_pages = min(2048, int(I.seq_lens(w)[0]) // P)
    L = n_pages * P
    k, v = I.kv_rows(w, 0, 0, L)
    kf = I.bf16_to_f32(k)
    vf = None if v is None else I.bf16_to_f32(v)
    g = Q.nvfp4_global_scale(np.abs(kf).max()) if w.dtype == "nvfp4" else None
    oc = OracleCache(CacheSpec(w.dtype, w.kind, w.kv_heads, w.head_dim, w.v_dim, P, n_pages))
    oc.store(kf, vf, np.arange(L), k_scale=g)
    t0 = time.perf_counter()
    dequantize_prev_kv(oc, np.arange(n_pages), 0.02, None if w.kind == "mla" else 0.01, g=g)
    dt = time.perf_counter() - t0
    rows = 2 * w.kv_heads if w.kind == "gqa" else 1
    nbytes = L * rows * w.head_dim * (4.5 / 8 + 1.0)
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": 1,
            "host_cores_available": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{n_pages} pages ({L} tokens, all {w.kv_heads} KV heads) of sequence 0: "
                      f"oracle dequantize_prev_kv {dt:.2f} s"}


def bench_dequant_prev(w, args, dev):
    """kvq_dequantize_prev_kv over every page of the workload's cache: the
    FP4 prefix turned into E4M3 rows for an FP8 prefill kernel."""
    import torch

    import quantized_paged_kv_store_amd as K
    t0 = time.time()
    st = setup(w, dev, args.rotate)
    log(f"setup {time.time() - t0:.1f} s")
    caches = st["caches"]
    d = caches[0].desc
    npages = d.num_pages
    pages = torch.arange(npages, dtype=torch.int32, device=dev)
    g = st["ks"] if w.kind == "mla" else None
    ks_out = torch.tensor([0.02], dtype=torch.float32, device=dev)
    vs_out = None if w.kind == "mla" else torch.tensor([0.01], dtype=torch.float32, device=dev)
    dk, dv = K.kvq_dequantize_prev_kv(caches[0], pages, ks_out, vs_out, g=g)

    def loop(n, off=0):
        for i in range(n):
            K.kvq_dequantize_prev_kv(caches[(i + off) % len(caches)], pages, ks_out, vs_out, g=g, dq_k=dk, dq_v=dv)

    loop(args.warmup)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    loop(args.steps)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    K.kvq_profile_enable(True)
    loop(args.steps)
    torch.cuda.synchronize()
    tot, n = K.kvq_profile_read("dequant_prev")
    K.kvq_profile_enable(False)
    kern_ms = tot / max(n, 1)
    rows = 2 * d.num_kv_heads if w.kind == "gqa" else 1
    elems = float(npages) * d.page_size * rows * d.head_dim
    read_b, write_b = elems * (0.5 + 1 / 16), elems * 1.0
    value = (read_b + write_b) / (ms * 1e-3) / 1e9
    ach = (read_b + write_b) / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "dequantize_prev_kv effective GB/s (FP4 pages read + E4M3 rows written)", "value": round(value, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: every page of the cache ({npages} pages of {d.page_size} tokens, "
                               f"{d.num_kv_heads} kv head(s), head_dim {d.head_dim}, {w.dtype}) -> E4M3",
                   "cache_copies_rotated": args.rotate},
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": measured_traffic(w, "dequant_prev"),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                     "kernel": f"dequant_prev_{'nvfp4' if w.kind == 'mla' else 'mx16'}_kernel",
                     "kernel_ms": round(kern_ms, 5), "algorithmic_bytes_per_launch": read_b + write_b},
        "pct_hbm_peak": round(100 * value / PEAK_HBM_GBPS, 2),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = dequant_prev_cpu_baseline(w)
    print(json.dumps(res), flush=True)


def extend_flops(prefix, chunk, hq, d):
    """Algorithmic flops of extend attention: chunk token i of a sequence with
    prefix L0 scores and weighs L0 + i + 1 keys, 2 * d flops each for QK and PV
    per query head."""
    c = np.asarray(chunk, np.float64)
    return float(np.sum(c * np.asarray(prefix, np.float64) + c * (c + 1) / 2) * hq * 4 * d)


def extend_cpu_baseline(w, rows=256):
    """The oracle's extend_attention, untuned, on a few chunk rows of one
    sequence of the same shape (all query heads, full prefix)."""
    from oracle.attention import extend_attention
    from quantized_paged_kv_store_amd import inputs as I
    L0 = w.max_len - w.new_tokens
    inp = I.extend_inputs(9, [L0], [rows], w.kv_heads, w.group, w.head_dim, w.page_size)
    f = lambda a: I.bf16_to_f32(a).astype(np.float64)
    t0 = time.perf_counter()
    extend_attention(f(inp["q"]), f(inp["k_new"]), f(inp["v_new"]), inp["cu_q"], inp["prefix_len"], inp["dq_k"],
                     inp["dq_v"], inp["page_off"], 0.05, 0.05, I.sm_scale(w))
    dt = time.perf_counter() - t0
    fl = extend_flops([L0], [rows], w.q_heads, w.head_dim)
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas),
            "host_cores_available": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{rows} chunk rows x {w.q_heads} heads over a {L0}-token prefix: float64 oracle "
                      f"extend_attention {dt:.2f} s (E4M3 workspace decode included)"}


def bench_extend(w, args, dev):
    """One chunked-prefill step of the FP4 workload: kvq_store of the chunk
    (new_tokens per sequence), kvq_dequantize_prev_kv of every prefix page to
    E4M3, then kvq_extend_attention of the chunk over prefix + chunk."""
    import torch

    import quantized_paged_kv_store_amd as K
    from quantized_paged_kv_store_amd import inputs as I
    t0 = time.time()
    st = setup(w, dev, 1)
    log(f"setup {time.time() - t0:.1f} s")
    cache = st["caches"][0]
    lens = st["lens_h"]
    C = w.new_tokens
    prefix = (lens - C).astype(np.int32)
    assert np.all(prefix >= 0)
    table, _ = I.page_table(w, lens)
    P = w.page_size
    npg = (prefix + P - 1) // P
    pages = np.concatenate([table[b, :npg[b]] for b in range(w.batch)]).astype(np.int32)
    page_off = np.concatenate([[0], np.cumsum(npg)[:-1]]).astype(np.int32)
    pages_d = torch.from_numpy(pages).to(dev)
    s_k = torch.tensor([0.05], dtype=torch.float32, device=dev)
    s_v = torch.tensor([0.05], dtype=torch.float32, device=dev)
    dk, dv = K.kvq_dequantize_prev_kv(cache, pages_d, s_k, s_v)
    k_new, v_new, slots = st["new"]
    nq = w.batch * C
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    q = torch.randn((nq, w.q_heads, w.head_dim), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    cu = torch.arange(0, nq + 1, C, dtype=torch.int32, device=dev)
    prefix_d = torch.from_numpy(prefix).to(dev)
    off_d = torch.from_numpy(page_off).to(dev)
    out = torch.empty((nq, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((nq, w.q_heads), dtype=torch.float32, device=dev)
    sm = I.sm_scale(w)

    def step():
        K.kvq_store(cache, k_new, v_new, slots)
        K.kvq_dequantize_prev_kv(cache, pages_d, s_k, s_v, dq_k=dk, dq_v=dv)
        K.kvq_extend_attention(q, k_new, v_new, cu, prefix_d, dk, dv, off_d, s_k, s_v, C, sm, out=out, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    K.kvq_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ext_ms = K.kvq_profile_read("extend")[0] / args.steps
    dq_ms = K.kvq_profile_read("dequant_prev")[0] / args.steps
    sto_ms = K.kvq_profile_read("store")[0] / args.steps
    K.kvq_profile_enable(False)
    fl = extend_flops(prefix, [C] * w.batch, w.q_heads, w.head_dim)
    value = fl / (ms * 1e-3) / 1e12
    ach = fl / (ext_ms * 1e-3) / 1e12
    log(f"step {ms:.2f} ms: store {sto_ms:.3f} ms, dequantize_prev_kv {dq_ms:.3f} ms, extend {ext_ms:.2f} ms")
    res = {
        "metric": "extend attention TFLOP/s over an FP4 prefix (store chunk + dequantize_prev_kv + extend)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: batch {w.batch}, {C}-token chunk per sequence over a "
                               f"{int(prefix[0])}-token {w.dtype} prefix, {w.q_heads} q / {w.kv_heads} kv heads, "
                               f"head_dim {w.head_dim}, page {P}; prefix read through E4M3 workspaces "
                               f"(scales 0.05), chunk K/V BF16, causal within the chunk",
                   "algorithmic_flops_per_step": fl},
        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_F16_TFLOPS, 4), "traffic": measured_traffic(w, "extend"),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                     "kernel": "extend_attn_kernel (bf16 / fp16 MFMA)", "kernel_ms": round(ext_ms, 4)},
        "kernel_ms": {"extend": round(ext_ms, 4), "dequant_prev": round(dq_ms, 4), "store": round(sto_ms, 4)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = extend_cpu_baseline(w)
    print(json.dumps(res), flush=True)


def copy_reference(nbytes=1 << 30, reps=10, quiet=False):
    """A plain device copy of known size (src -> dst), the reference the HBM
    traffic counters are scaled by; also reported beside the roofline as the
    copy rate this GPU reaches (read + write bytes per second)."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    rec = {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms": round(ms, 4),
           "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}
    del src, dst
    torch.cuda.empty_cache()
    if not quiet:
        print(json.dumps(rec), flush=True)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 1,000 for a decode step: a serving loop's steady state; 100 for "
                         "--dequant-prev and --extend)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default steps / 10)")
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay captured HIP graphs instead of eager launches")
    ap.add_argument("--copy-ref", action="store_true", help="only run the 1 GiB reference copy (for counters)")
    ap.add_argument("--dequant-prev", action="store_true",
                    help="FP4 workloads: time kvq_dequantize_prev_kv over every page instead of the decode step")
    ap.add_argument("--extend", action="store_true",
                    help="FP4 GQA workload with a chunk: store + dequantize_prev_kv + extend attention per step")
    ap.add_argument("--kivi", action="store_true",
                    help="FP8 workloads: K scales per channel, V scales per token (KIVI-style)")
    ap.add_argument("--per-head-scales", action="store_true",
                    help="FP8 workloads: one calibrated k/v scale per KV head instead of per tensor")
    ap.add_argument("--kv-dtype", choices=("e4m3", "e5m2"), default=None,
                    help="FP8 GQA workloads: the cache's FP8 format (workload variant; default the workload's)")
    ap.add_argument("--scale", choices=("amax", "one"), default=None,
                    help="FP8 workloads: per-tensor scales calibrated from the prefill's amax, or 1.0")
    ap.add_argument("--fp8q", action="store_true",
                    help="FP8 GQA and NVFP4 MLA workloads: FP8-domain attention (query rounded to E4M3, QK on "
                         "FP8 MFMA; MLA keys as E4M3 codes of the latent / 8g)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 100 if (args.dequant_prev or args.extend) else 1000
    if args.warmup is None:
        args.warmup = max(args.steps // 10, 1)
    if args.copy_ref:
        copy_reference()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path shards across (sequence, KV head) with no "
              f"exchange, so a multi-GPU figure is N independent copies of this one; got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_paged_kv_store_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    if args.kv_dtype:
        assert w.dtype in ("e4m3", "e5m2") and w.kind == "gqa", "--kv-dtype applies to FP8 GQA workloads"
        w = w.with_(dtype=args.kv_dtype)
    if args.scale:
        assert w.dtype in ("e4m3", "e5m2"), "--scale applies to FP8 workloads"
        w = w.with_(scale_mode=args.scale)
    if args.per_head_scales:
        assert w.dtype in ("e4m3", "e5m2"), "per-head scales apply to FP8 caches"
        w = w.with_(scale_mode="amax_head")
    if args.kivi:
        assert w.dtype in ("e4m3", "e5m2") and w.kind == "gqa", "KIVI-style scales apply to FP8 GQA caches"
        w = w.with_(scale_mode="kivi")
    if args.fp8q:
        assert (w.dtype in ("e4m3", "e5m2") and w.kind == "gqa" and w.scale_mode != "kivi") or w.kind == "mla", \
            "FP8-domain attention applies to FP8 GQA caches with tensor or per-head scales and to the MLA latent"
    dev = torch.device("cuda:0")
    if args.dequant_prev:
        assert w.dtype in ("mx16", "nvfp4"), "dequantize_prev_kv reads FP4 caches"
        bench_dequant_prev(w, args, dev)
        return
    if args.extend:
        assert w.dtype == "mx16" and w.kind == "gqa" and w.new_tokens > 1, "extend runs on the FP4 chunk workload"
        bench_extend(w, args, dev)
        return
    t0 = time.time()
    st = setup(w, dev, args.rotate, args.fp8q)
    log(f"setup {time.time() - t0:.1f} s")
    # a decode step with one new token per sequence appends it and decodes in
    # one launch (kvq_decode_append); a chunked step stores, then decodes
    fused = st["new_rows"] is not None
    run_loop(st, args.warmup, True, True, fused=fused)
    torch.cuda.synchronize()
    use_graph = args.graph
    g_step = capture(st, True, True, fused) if use_graph else None
    g_sep = capture(st, True, True) if use_graph else None
    g_dec = capture(st, False, True) if use_graph else None
    g_store = capture(st, True, False) if use_graph else None
    if use_graph:
        for i in range(args.warmup):
            g_step[i % len(g_step)].replay()
    ms_step = timed(st, args.steps, True, True, g_step, fused=fused)
    ms_sep = timed(st, args.steps, True, True, g_sep) if fused else ms_step
    ms_dec = timed(st, args.steps, False, True, g_dec)
    ms_store = timed(st, args.steps, True, False, g_store)
    # per-kernel device time: the library brackets each launch with HIP events
    # on the launch stream while instrumentation is on
    import quantized_paged_kv_store_amd as K
    K.kvq_profile_enable(True)
    run_loop(st, args.steps, True, True, fused=fused)
    torch.cuda.synchronize()
    dec_tot, dec_n = K.kvq_profile_read("decode")
    mer_tot, mer_n = K.kvq_profile_read("merge")
    run_loop(st, args.steps, True, False)
    torch.cuda.synchronize()
    sto_tot, sto_n = K.kvq_profile_read("store")
    # the decode kernel alone, back to back with no store between launches
    run_loop(st, args.steps, False, True)
    torch.cuda.synchronize()
    dec_only_tot, dec_only_n = K.kvq_profile_read("decode")
    K.kvq_profile_read("merge")
    K.kvq_profile_enable(False)
    # the roofline uses the decode kernel as it runs inside the step
    kern_ms = dec_tot / max(dec_n, 1)
    kern_only_ms = dec_only_tot / max(dec_only_n, 1)
    merge_ms = mer_tot / max(mer_n, 1) if mer_n else 0.0
    store_kern_ms = sto_tot / max(sto_n, 1)
    kv_bytes = float(st["lens_h"].astype(np.int64).sum()) * st["bpt"]
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    dec_gbps = kv_bytes / (ms_dec * 1e-3) / 1e9
    log(f"step {ms_step * 1e3:.1f} us (store then decode {ms_sep * 1e3:.1f} us), decode {ms_dec * 1e3:.1f} us, "
        f"store {ms_store * 1e3:.1f} us, "
        f"{value:.0f} GB/s per step, {dec_gbps:.0f} GB/s decode")
    # the headline metric is the 8B FP8 decode step with per-tensor scales;
    # other workloads and modes name themselves
    variant = [m for m, on in (("KIVI-style scales", w.scale_mode == "kivi"),
                               ("per-KV-head scales", w.scale_mode == "amax_head"),
                               ("scale 1.0", w.scale_mode == "one"),
                               ("FP8-domain attention", args.fp8q)) if on]
    metric = METRIC if (w.name == "llama3_8b" and not variant) else (
        f"decode-attn effective KV GB/s (% HBM peak), {w.name} {w.dtype} bs{w.batch} ctx{w.max_len}"
        + "".join(f", {v}" for v in variant))
    res = {
        "metric": metric, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8" if args.fp8q else "bf16", "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.q_heads} q heads / {w.kv_heads} kv heads, head_dim {w.head_dim}, "
                        f"batch {w.batch}, context {w.max_len}, page {w.page_size}, {w.dtype} KV "
                        f"({w.scale_mode} scales); step = "
                        + ("append 1 new token/sequence + decode in one kvq_decode_append launch (+ split merge)"
                           if fused else f"store {w.new_tokens} new token(s)/sequence, then decode (+ split merge)")
                        + ("; FP8-domain attention: query rounded to E4M3 with calibrated q_scale, QK^T on "
                           "fp8 MFMA from the cached codes (kvq_decode_append_fp8q)" if args.fp8q else ""),
            "global_batch": w.batch, "seq_len": w.max_len, "kv_dtype": w.dtype,
            "compute": (("E4M3 query x E4M3 codes of the latent / 8g on fp8 MFMA (QK); latent dequantized to "
                         "fp16 (E2M1 x E4M3 exact) for the PV MFMAs; f32 accumulate" if args.fp8q else
                         "latent codes dequantized to fp16 (E2M1 x E4M3 exact) for QK and PV MFMAs, f32 accumulate")
                        if w.kind == "mla" else
                        "E4M3 query x cached FP8 codes on fp8 MFMA (QK); V codes to f16 MFMA operands (PV); f32 "
                        "accumulate" if args.fp8q else
                        "KV codes dequantized in registers to bf16 (QK) / f16 (PV) MFMA operands, f32 accumulate"),
            "cache_copies_rotated": args.rotate,
            "launch": "HIP graph replay per step" if use_graph else "eager launches",
        },
        "pct_hbm_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "decode_only_GBps": round(dec_gbps, 2), "decode_ms": round(ms_dec, 5), "store_ms": round(ms_store, 5),
        "store_then_decode_ms": round(ms_sep, 5),
        "context_tokens_per_s": round(float(st["lens_h"].sum()) / (ms_step * 1e-3), 1),
        "decode_tokens_per_s": round(w.batch / (ms_step * 1e-3), 1),
        "bulk_store": st["bulk_store"],
    }
    traffic = measured_traffic(w, fp8q=args.fp8q)
    if w.kind == "mla":
        ntok = float(st["lens_h"].astype(np.int64).sum())
        qk_flops, pv_flops = ntok * w.q_heads * w.head_dim * 2, ntok * w.q_heads * w.v_dim * 2
        flops = qk_flops + pv_flops
        # FP8-domain: QK at the fp8 peak, PV at the fp16 peak; the peak quoted
        # is the rate that would finish both at their own peaks in one time
        peak = (flops / (qk_flops / PEAK_FP8_TFLOPS + pv_flops / PEAK_F16_TFLOPS) if args.fp8q
                else PEAK_F16_TFLOPS)
        ach = flops / (kern_ms * 1e-3) / 1e12
        res["roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                           "frac": round(ach / peak, 4), "traffic": traffic,
                           "kernel": ("decode_mla_kernel (QK fp8 MFMA, PV fp16 MFMA)" if args.fp8q
                                      else "decode_mla_kernel (fp16 MFMA)"), "kernel_ms": round(kern_ms, 5),
                           "algorithmic_flops_per_launch": flops,
                           "hbm_GBps": round(kv_bytes / (kern_ms * 1e-3) / 1e9, 2)}
    else:
        ach = kv_bytes / (kern_ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(ach, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                           "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": traffic,
                           "kernel": f"decode_gqa_kernel ({w.dtype}, head_dim {w.head_dim}"
                                     + (", FP8-domain QK)" if args.fp8q else ")"),
                           "kernel_ms": round(kern_ms, 5), "algorithmic_bytes_per_launch": kv_bytes}
    res["roofline"]["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)"
    res["kernel_ms"] = {"decode": round(kern_ms, 5), "merge": round(merge_ms, 5), "store": round(store_kern_ms, 5),
                        "decode_without_store": round(kern_only_ms, 5)}
    res["decode_kernel_GBps"] = {"in_step": round(kv_bytes / (kern_ms * 1e-3) / 1e9, 2),
                                 "without_store": round(kv_bytes / (kern_only_ms * 1e-3) / 1e9, 2)}
    # information only, after the timed region: what a plain 1 GiB device copy reaches here
    res["device_copy_GBps_read_plus_write"] = copy_reference(quiet=True)["GBps_read_plus_write"]
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, fp8q=args.fp8q)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
