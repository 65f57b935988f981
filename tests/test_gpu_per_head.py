"""Per-attention-head FP8 scales (vLLM page, "Supported schemes": k/v_scale =
[num_kv_heads]) through the HIP path: calibrated scales and stored codes
bit-exact with the oracle, decode (and the one-launch append step) within
tolerance of the oracle fed the same per-head dequantized values."""
import numpy as np
import pytest
import torch

import quantized_paged_kv_store_amd as K
from oracle import formats as F
from oracle import quantize as Q
from quantized_paged_kv_store_amd import inputs as I
from tests.kvq_cases import Case, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dtype,hkv,D", [("e4m3", 8, 128), ("e5m2", 3, 64), ("e4m3", 1, 128)])
def test_compute_scale_per_head_bit_exact(dtype, hkv, D):
    fmt = F.E4M3 if dtype == "e4m3" else F.E5M2
    cache = K.kvq_alloc_pages(dtype, "gqa", hkv, D, D, 16, 1, device=DEV, scale_per_head=True)
    rng = np.random.default_rng(31)
    for n0, n1 in ((1, 0), (777, 0), (20000, 13)):
        a = rng.standard_normal((n0, hkv, D)) * (10.0 ** rng.uniform(-3, 3, size=(1, hkv, 1)))
        b = rng.standard_normal((n1, hkv, D)) * 3 if n1 else None
        ab = I.bf16_to_f32(I.bf16_bits(a.astype(np.float32)))
        bb = None if b is None else I.bf16_to_f32(I.bf16_bits(b.astype(np.float32)))
        xa = torch.from_numpy(I.bf16_bits(ab)).to(DEV).view(torch.bfloat16)
        xb = None if bb is None else torch.from_numpy(I.bf16_bits(bb)).to(DEV).view(torch.bfloat16)
        out = K.kvq_compute_scale(cache, xa, xb).cpu().numpy()
        joint = ab if bb is None else np.concatenate([ab, bb])
        assert np.array_equal(out, Q.fp8_head_scales(joint, fmt))
    zero = torch.zeros((5, hkv, D), dtype=torch.bfloat16, device=DEV)
    assert np.all(K.kvq_compute_scale(cache, zero).cpu().numpy() == 1.0)


def _workload(dtype, lens, G=4, hkv=4, D=128, P=16):
    return I.Workload(f"per-head-{dtype}", dtype, "gqa", len(lens), G * hkv, hkv, D, D, P, max(lens), 0, 1,
                      "llama", scale_mode="amax_head", seed=33)


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_per_head_store_bytes_and_decode(dtype):
    lens = [0, 1, 17, 300, 2048, 5000]
    c = Case(_workload(dtype, lens), lens=lens).run_gpu()
    ks, vs = c.gpu_scales()
    oks, ovs = c.oracle_scales()
    assert ks.shape == (4,) and np.array_equal(ks, oks) and np.array_equal(vs, ovs)
    assert len(set(ks.tolist())) > 1                                   # the heads really differ
    ids = [1, 2, 3, 5]
    want, wlse, oc, pages = c.oracle_decode(ids)
    for name in ("k_codes", "v_codes"):
        assert np.array_equal(c.gpu_pages(name, pages), getattr(oc, name)), name
    assert_close(c.out.cpu().numpy()[ids], want[ids], f"per-head {dtype}")
    glse = c.lse.cpu().numpy()[ids]
    assert np.allclose(glse, wlse[ids], rtol=0, atol=1e-4)


def test_per_head_append_matches_store_then_decode():
    lens = [1, 16, 33, 1000, 3001]
    w = _workload("e4m3", lens, G=8, hkv=2)
    a = Case(w, lens=lens).run_gpu()
    b = Case(w, lens=lens, data=a.data).run_gpu(append=True)
    torch.cuda.synchronize()
    assert torch.equal(a.cache.memory, b.cache.memory)
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)


def test_per_head_llama3_8b_shape_sampled():
    """The 8B decode shape with per-KV-head scales; oracle on sequences 0 and 6."""
    w = I.WORKLOADS["llama3_8b"].with_(scale_mode="amax_head")
    c = Case(w).run_gpu()
    want, _, _, _ = c.oracle_decode([0, 6])
    assert_close(c.out.cpu().numpy()[[0, 6]], want[[0, 6]], "per-head llama3_8b")
