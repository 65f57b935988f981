"""KIVI-style FP8 scaling through the HIP path ("KV cache quantization
mechanism and traps" page, K and V distributions: K scales per channel, V
scales per token): calibrated channel scales, stored codes and per-token V
scales bit-exact with the oracle, decode (and the one-launch append step)
within tolerance of the oracle fed the same dequantized values."""
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
def test_compute_scale_per_channel_bit_exact(dtype, hkv, D):
    fmt = F.E4M3 if dtype == "e4m3" else F.E5M2
    cache = K.kvq_alloc_pages(dtype, "gqa", hkv, D, D, 16, 1, device=DEV, scale_mode="kivi")
    rng = np.random.default_rng(41)
    for n0, n1 in ((1, 0), (777, 0), (20000, 13)):
        a = rng.standard_normal((n0, hkv, D)) * (10.0 ** rng.uniform(-3, 3, size=(1, hkv, D)))
        a[:, 0, 3] = 0.0                                           # an all-zero channel -> 1.0
        b = rng.standard_normal((n1, hkv, D)) * 3 if n1 else None
        ab = I.bf16_to_f32(I.bf16_bits(a.astype(np.float32)))
        bb = None if b is None else I.bf16_to_f32(I.bf16_bits(b.astype(np.float32)))
        xa = torch.from_numpy(I.bf16_bits(ab)).to(DEV).view(torch.bfloat16)
        xb = None if bb is None else torch.from_numpy(I.bf16_bits(bb)).to(DEV).view(torch.bfloat16)
        out = K.kvq_compute_scale(cache, xa, xb).cpu().numpy()
        joint = ab if bb is None else np.concatenate([ab, bb])
        assert out.shape == (hkv * D,)
        assert np.array_equal(out.reshape(hkv, D), Q.fp8_channel_scales(joint, fmt))


def _workload(dtype, lens, G=4, hkv=4, D=128, P=16, dist="llama"):
    return I.Workload(f"kivi-{dtype}", dtype, "gqa", len(lens), G * hkv, hkv, D, D, P, max(lens), 0, 1,
                      dist, scale_mode="kivi", seed=43)


LENS = [0, 1, 15, 16, 17, 300, 2048, 5000]


@pytest.mark.parametrize("dtype,D,G,P", [("e4m3", 128, 4, 16), ("e5m2", 128, 8, 32), ("e4m3", 64, 3, 16),
                                         ("e4m3", 128, 16, 64), ("e4m3", 128, 4, 48)])
def test_kivi_store_bytes_and_decode(dtype, D, G, P):
    c = Case(_workload(dtype, LENS, G=G, hkv=2, D=D, P=P), lens=LENS).run_gpu()
    ks, vs = c.gpu_scales()
    oks, _ = c.oracle_scales()
    assert vs is None and np.array_equal(ks, oks)
    ids = [1, 2, 4, 6, 7]
    want, wlse, oc, pages = c.oracle_decode(ids)
    for name in ("k_codes", "v_codes", "v_scales"):
        assert np.array_equal(c.gpu_pages(name, pages), getattr(oc, name)), name
    assert_close(c.out.cpu().numpy()[ids], want[ids], f"kivi {dtype} D{D} G{G} P{P}")
    assert np.allclose(c.lse.cpu().numpy()[ids], wlse[ids], rtol=0, atol=1e-4)
    assert np.all(c.out.cpu().numpy()[0] == 0) and np.isneginf(c.lse.cpu().numpy()[0]).all()


def test_kivi_append_matches_store_then_decode():
    lens = [1, 16, 33, 1000, 3001]
    w = _workload("e4m3", lens, G=8, hkv=2)
    a = Case(w, lens=lens).run_gpu()
    b = Case(w, lens=lens, data=a.data).run_gpu(append=True)
    torch.cuda.synchronize()
    assert torch.equal(a.cache.memory, b.cache.memory)
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)
    want, _, _, _ = b.oracle_decode([0, 3, 4])
    assert_close(b.out.cpu().numpy()[[0, 3, 4]], want[[0, 3, 4]], "kivi append")


def test_kivi_llama3_8b_shape_sampled():
    """The 8B decode shape (batch 8, context 20,480) with KIVI-style scales, in
    the benchmark's launch configuration; oracle on sequences 0 and 6."""
    w = I.WORKLOADS["llama3_8b"].with_(scale_mode="kivi")
    c = Case(w).run_gpu(append=True)
    want, wlse, oc, pages = c.oracle_decode([0, 6])
    for name in ("k_codes", "v_codes", "v_scales"):
        assert np.array_equal(c.gpu_pages(name, pages), getattr(oc, name)), name
    assert_close(c.out.cpu().numpy()[[0, 6]], want[[0, 6]], "kivi llama3_8b")
    assert np.allclose(c.lse.cpu().numpy()[[0, 6]], wlse[[0, 6]], rtol=0, atol=1e-4)
