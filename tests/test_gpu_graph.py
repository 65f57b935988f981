"""The entry points captured in a HIP graph (store + decode, the one-launch
append step with tensor and KIVI-style scales and in the FP8 domain,
dequantize_prev_kv + extend attention): every replay, with eager work and synchronizations in between,
must reproduce the eager result."""
import numpy as np
import pytest
import torch

import quantized_paged_kv_store_amd as K
from quantized_paged_kv_store_amd import inputs as I
from tests.kvq_cases import Case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["llama3_8b", "tiny"])
def test_graph_replay_matches_eager(name):
    w = I.WORKLOADS[name].with_(batch=2, max_len=3000, min_len=3000) if name != "tiny" else I.WORKLOADS[name]
    c = Case(w).run_gpu()
    eager = c.out.cpu().numpy().copy()
    eager_lse = c.lse.cpu().numpy().copy()
    out = torch.full_like(c.out, float("nan"))
    lse = torch.full_like(c.lse, float("nan"))
    need = K.kvq_decode_workspace_bytes(c.cache, w.batch, w.q_heads, c.max_len)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=c.dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.kvq_store(c.cache, *c.new_dev, c.k_scale, c.v_scale)
        K.kvq_decode(c.cache, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(w), c.k_scale, c.v_scale,
                     out=out, lse=lse, workspace=ws)
    for _ in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager)
        assert np.array_equal(lse.cpu().numpy(), eager_lse)
        _ = (c.q_dev.float() * 2).sum().item()       # unrelated eager work between replays


@pytest.mark.parametrize("name", ["llama3_8b", "dsr1_mla"])
def test_graph_replay_append_matches_eager(name):
    """kvq_decode_append (one launch per step) captured in a HIP graph."""
    w = I.WORKLOADS[name].with_(batch=2, max_len=3000, min_len=3000)
    c = Case(w).run_gpu(append=True)
    eager = c.out.cpu().numpy().copy()
    eager_lse = c.lse.cpu().numpy().copy()
    kn, vn, _ = c.new_inputs
    row = (w.kv_heads, w.head_dim) if w.kind == "gqa" else (w.head_dim,)
    k_new = torch.from_numpy(kn.reshape(w.batch, *row)).to(c.dev).view(torch.bfloat16)
    v_new = None if vn is None else torch.from_numpy(vn.reshape(w.batch, *row)).to(c.dev).view(torch.bfloat16)
    out = torch.full_like(c.out, float("nan"))
    lse = torch.full_like(c.lse, float("nan"))
    need = K.kvq_decode_workspace_bytes(c.cache, w.batch, w.q_heads, c.max_len)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=c.dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.kvq_decode_append(c.cache, k_new, v_new, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(w),
                            c.k_scale, c.v_scale, out=out, lse=lse, workspace=ws)
    for _ in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager)
        assert np.array_equal(lse.cpu().numpy(), eager_lse)
        _ = (c.q_dev.float() * 2).sum().item()       # unrelated eager work between replays


def test_graph_replay_kivi_append_matches_eager():
    """KIVI-style scales: kvq_decode_append (per-token V scales written in the
    launch) captured in a HIP graph."""
    w = I.WORKLOADS["llama3_8b"].with_(batch=2, max_len=3000, min_len=3000, scale_mode="kivi")
    c = Case(w).run_gpu(append=True)
    eager = c.out.cpu().numpy().copy()
    kn, vn, _ = c.new_inputs
    k_new = torch.from_numpy(kn.reshape(w.batch, w.kv_heads, w.head_dim)).to(c.dev).view(torch.bfloat16)
    v_new = torch.from_numpy(vn.reshape(w.batch, w.kv_heads, w.head_dim)).to(c.dev).view(torch.bfloat16)
    out = torch.full_like(c.out, float("nan"))
    lse = torch.full_like(c.lse, float("nan"))
    need = K.kvq_decode_workspace_bytes(c.cache, w.batch, w.q_heads, c.max_len)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=c.dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.kvq_decode_append(c.cache, k_new, v_new, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(w),
                            c.k_scale, None, out=out, lse=lse, workspace=ws)
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager)
        _ = (c.q_dev.float() * 2).sum().item()


def test_graph_replay_dequant_prev_and_extend_match_eager():
    """kvq_dequantize_prev_kv followed by kvq_extend_attention, captured."""
    inp = I.extend_inputs(8, [300, 77], [40, 9], 2, 16, 128, 16)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    bf = lambda a: t(a).view(torch.bfloat16)
    q, kn, vn = bf(inp["q"]), bf(inp["k_new"]), bf(inp["v_new"])
    cu, pl, po = t(inp["cu_q"]), t(inp["prefix_len"]), t(inp["page_off"])
    cache = K.kvq_alloc_pages("mx16", "gqa", 2, 128, 128, 16, 32, device="cuda", fill=0)
    for name, arr in I.random_cache_bytes({"k_codes": (32, 2, 1024), "v_codes": (32, 2, 1024),
                                           "k_scales": (32, 2, 128), "v_scales": (32, 2, 128)},
                                          "mx16", 9, (110, 140)).items():
        cache.view(name).copy_(torch.from_numpy(arr.reshape(-1)))
    pages = t(np.arange(32, dtype=np.int32)[::-1].copy())
    s_k = torch.tensor([0.05], device="cuda")
    s_v = torch.tensor([0.05], device="cuda")
    dk = torch.empty((32, 2, 16, 128), dtype=torch.uint8, device="cuda")
    dv = torch.empty_like(dk)
    out = torch.empty((q.shape[0], 32, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((q.shape[0], 32), dtype=torch.float32, device="cuda")

    def step():
        K.kvq_dequantize_prev_kv(cache, pages, s_k, s_v, dq_k=dk, dq_v=dv)
        K.kvq_extend_attention(q, kn, vn, cu, pl, dk, dv, po, s_k, s_v, 40, 0.088, out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    eager, eager_lse, eager_dk = out.cpu().numpy().copy(), lse.cpu().numpy().copy(), dk.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        out.fill_(float("nan"))
        dk.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(dk.cpu().numpy(), eager_dk)
        assert np.array_equal(out.cpu().numpy(), eager) and np.array_equal(lse.cpu().numpy(), eager_lse)
        _ = (q.float() * 2).sum().item()


@pytest.mark.parametrize("name", ["llama3_8b", "dsr1_mla"])
def test_graph_replay_fp8q_append_matches_eager(name):
    """FP8-domain append step (kvq_decode_append_fp8q) captured in a HIP graph
    (GQA with per-head query scales; the MLA latent with one)."""
    w = I.WORKLOADS[name].with_(batch=2, max_len=3000, min_len=3000)
    if name == "llama3_8b":
        w = w.with_(scale_mode="amax_head")
    c = Case(w).run_gpu(decode=False, append=True)
    qs = K.kvq_compute_q_scale(c.cache, c.q_dev)
    need = K.kvq_decode_workspace_bytes(c.cache, w.batch, w.q_heads, c.max_len)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=c.dev)
    out = torch.empty((w.batch, w.q_heads, w.v_dim), dtype=torch.float32, device=c.dev)
    lse = torch.empty((w.batch, w.q_heads), dtype=torch.float32, device=c.dev)

    def step():
        K.kvq_decode_append_fp8q(c.cache, *c.append_rows, c.q_dev, c.table_dev, c.lens_dev, c.max_len,
                                 I.sm_scale(w), qs, c.k_scale, c.v_scale, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager, eager_lse = out.cpu().numpy().copy(), lse.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager) and np.array_equal(lse.cpu().numpy(), eager_lse)
        _ = (c.q_dev.float() * 2).sum().item()
