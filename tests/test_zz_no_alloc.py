"""kvq_decode_noalloc (split partials in the library's static device
workspace) against kvq_decode (partials in a caller workspace): the same
kernels and split plan on the same inputs, so the outputs and LSEs must be
bit-identical. Two no-alloc calls run back to back, the second on a smaller
batch with shorter sequences, before either is compared, so a partial left
behind by the first call would show in the second."""
import numpy as np
import pytest
import torch

import quantized_paged_kv_store_amd as K
from quantized_paged_kv_store_amd import inputs as I
from kvq_cases import Case


def _case(name, batch, max_len, min_len):
    w = I.WORKLOADS[name].with_(batch=batch, max_len=max_len, min_len=min_len)
    return w, Case(w).run_gpu(decode=False)


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["llama3_8b", "dsr1_mla"])
def test_noalloc_matches_decode(name):
    print(f"\nno-alloc decode, {name}", flush=True)
    big = _case(name, 4, 9000, 5000)
    small = _case(name, 2, 3000, 100)
    got = []
    for w, c in (big, small):
        assert K.kvq_decode_workspace_bytes(c.cache, w.batch, w.q_heads, c.max_len) > 0   # several splits
        out = torch.full((w.batch, w.q_heads, w.v_dim), float("nan"), device=c.dev)
        lse = torch.full((w.batch, w.q_heads), float("nan"), device=c.dev)
        K.kvq_decode_noalloc(c.cache, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(w), c.k_scale,
                             c.v_scale, out=out, lse=lse)
        got.append((out, lse))
    torch.cuda.synchronize()
    for (w, c), (out, lse) in zip((big, small), got):
        want, wlse = K.kvq_decode(c.cache, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(w), c.k_scale,
                                  c.v_scale)
        torch.cuda.synchronize()
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        assert np.all(np.isfinite(o))
        assert np.array_equal(o.view(np.uint32), want.cpu().numpy().view(np.uint32)), f"{name} B{w.batch}: out"
        assert np.array_equal(l.view(np.uint32), wlse.cpu().numpy().view(np.uint32)), f"{name} B{w.batch}: lse"
