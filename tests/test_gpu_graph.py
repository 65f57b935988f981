"""kvq_store + kvq_decode captured in a HIP graph: every replay (with eager
work and synchronizations in between) must reproduce the eager result."""
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
