"""GPU parity of kvq_compute_scale / kvq_store against the oracle: codes and
scales must be bit-exact (whole cache buffers compared byte for byte,
including the padding bytes of slots never written)."""
import numpy as np
import pytest
import torch

import quantized_paged_kv_store_amd as K
from oracle import formats as F
from oracle import quantize as Q
from oracle.paged import CacheSpec, OracleCache
from quantized_paged_kv_store_amd import inputs as I
from tests.kvq_cases import FILL, Case

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16_dev(x32):
    return torch.from_numpy(I.bf16_bits(np.asarray(x32, np.float32))).to(DEV).view(torch.bfloat16)


def _store_both(spec, k32, v32, slots, k_scale=None, v_scale=None):
    """Store the same BF16 rows on the GPU and in the oracle; return both caches."""
    cache = K.kvq_alloc_pages(spec.dtype, spec.kind, spec.num_kv_heads, spec.head_dim, spec.v_dim,
                              spec.page_size, spec.num_pages, device=DEV, fill=FILL[spec.dtype])
    kb = I.bf16_to_f32(I.bf16_bits(np.asarray(k32, np.float32)))
    vb = None if v32 is None else I.bf16_to_f32(I.bf16_bits(np.asarray(v32, np.float32)))
    ksd = None if k_scale is None else torch.tensor([k_scale], dtype=torch.float32, device=DEV)
    vsd = None if v_scale is None else torch.tensor([v_scale], dtype=torch.float32, device=DEV)
    K.kvq_store(cache, _bf16_dev(kb), None if vb is None else _bf16_dev(vb),
                torch.from_numpy(np.asarray(slots, np.int64)).to(DEV), ksd, vsd)
    torch.cuda.synchronize()
    oc = OracleCache(spec, fill=FILL[spec.dtype])
    oc.store(kb, vb, slots, k_scale=k_scale, v_scale=v_scale)
    return cache, oc


def _assert_bytes_equal(cache, oc):
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        want = getattr(oc, name)
        if want is None:
            continue
        got = cache.view(name).cpu().numpy().reshape(want.shape)
        bad = np.flatnonzero(got.ravel() != want.ravel())
        assert bad.size == 0, f"{name}: {bad.size} bytes differ, first at {bad[:8]} got {got.ravel()[bad[:8]]} want {want.ravel()[bad[:8]]}"


def _values_fp8(fmt):
    mags = fmt.values[: fmt.max_code + 1]
    mids = (mags[1:] + mags[:-1]) / 2
    vals = np.concatenate([mags, mids])
    # one BF16 ulp either side of each midpoint
    b = I.bf16_bits(mids.astype(np.float32))
    near = np.concatenate([I.bf16_to_f32(b + 1), I.bf16_to_f32(b - 1)]).astype(np.float64)
    big = np.array([fmt.max_value * 1.03, fmt.max_value * 1.5, 1e30, 3.3e38, 2.0 ** -133, 2.0 ** -126])
    vals = np.concatenate([vals, near, big])
    return np.concatenate([vals, -vals, [0.0, -0.0]])


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_fp8_store_every_code_and_midpoint(dtype):
    fmt = F.E4M3 if dtype == "e4m3" else F.E5M2
    vals = _values_fp8(fmt)
    D, H = 128, 2
    n_tok = -(-vals.size // (D * H))
    x = np.zeros(n_tok * H * D)
    x[: vals.size] = vals
    k = x.reshape(n_tok, H, D)
    v = np.random.default_rng(0).permutation(x).reshape(n_tok, H, D)
    pages = -(-n_tok // 16) + 1
    spec = CacheSpec(dtype, "gqa", H, D, D, 16, pages)
    slots = np.random.default_rng(1).permutation(pages * 16)[:n_tok]
    cache, oc = _store_both(spec, k, v, slots)           # scales NULL -> 1.0
    _assert_bytes_equal(cache, oc)


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2"])
def test_fp8_store_every_code_and_midpoint_in_word_groups(dtype):
    """The same values stored in slot order, so V lane words are written whole
    (four consecutive tokens at a time); the run starts and ends mid-group."""
    fmt = F.E4M3 if dtype == "e4m3" else F.E5M2
    vals = _values_fp8(fmt)
    D, H = 128, 2
    n_tok = -(-vals.size // (D * H))
    x = np.zeros(n_tok * H * D)
    x[: vals.size] = vals
    k = x.reshape(n_tok, H, D)
    v = np.random.default_rng(0).permutation(x).reshape(n_tok, H, D)
    pages = -(-(n_tok + 3) // 16) + 1
    spec = CacheSpec(dtype, "gqa", H, D, D, 16, pages)
    slots = 3 + np.arange(n_tok)
    cache, oc = _store_both(spec, k, v, slots)
    _assert_bytes_equal(cache, oc)


@pytest.mark.parametrize("scale", [2.0 ** -70, 2.0 ** -59, 0.0123, 3.0, 2.0 ** 59, 2.0 ** 70])
def test_fp8_store_scale_range(scale):
    """Scales inside and outside the range where the store divides by a
    reciprocal and one correction; values from 2^-133 to 3e38 so that the
    quotients reach zero, every code and saturation."""
    rng = np.random.default_rng(7)
    D, H, n_tok = 128, 2, 96
    mag = 2.0 ** rng.uniform(-133, 127.5, (n_tok, H, D))
    k = np.where(rng.random((n_tok, H, D)) < 0.5, -mag, mag)
    v = rng.standard_normal((n_tok, H, D)) * scale * 100
    spec = CacheSpec("e4m3", "gqa", H, D, D, 16, 8)
    slots = np.concatenate([np.arange(1, 50), 64 + rng.permutation(47)])  # word groups, then single tokens
    cache, oc = _store_both(spec, k, v, slots, k_scale=scale, v_scale=scale)
    _assert_bytes_equal(cache, oc)


def test_fp8_store_word_groups_and_partial_words():
    """Runs that fill whole V lane words mixed with ones that do not: a run in
    reverse order, a group with a gap, a group split over two calls and a
    skipped slot; words shared with tokens that are not stored keep their
    bytes."""
    rng = np.random.default_rng(8)
    D, H, P = 64, 3, 32
    spec = CacheSpec("e4m3", "gqa", H, D, D, P, 6)
    runs = [np.arange(5, 42),                      # starts and ends mid-group
            np.arange(64, 84)[::-1],               # reverse order: no whole group
            np.array([96, 97, 99, 100, 101, 102, 103]),  # 96..99 has a gap
            np.array([128, 129])]                  # first half of a group
    slots = np.concatenate(runs)
    slots[20] = -1                                 # a skipped token inside a run
    n1 = slots.size
    k = rng.standard_normal((n1 + 2, H, D)) * 4
    v = rng.standard_normal((n1 + 2, H, D)) * rng.lognormal(0, 0.5, (n1 + 2, 1, 1))
    cache, oc = _store_both(spec, k[:n1], v[:n1], slots, k_scale=0.02, v_scale=0.01)
    # the second half of the split group in a second call
    kb = I.bf16_to_f32(I.bf16_bits(k[n1:].astype(np.float32)))
    vb = I.bf16_to_f32(I.bf16_bits(v[n1:].astype(np.float32)))
    s2 = np.array([130, 131])
    K.kvq_store(cache, _bf16_dev(kb), _bf16_dev(vb), torch.from_numpy(s2).to(DEV),
                torch.tensor([0.02], device=DEV), torch.tensor([0.01], device=DEV))
    torch.cuda.synchronize()
    oc.store(kb, vb, s2, k_scale=0.02, v_scale=0.01)
    _assert_bytes_equal(cache, oc)


@pytest.mark.parametrize("dtype,D,P", [("e4m3", 64, 16), ("e4m3", 128, 32), ("e5m2", 128, 16), ("e4m3", 128, 48),
                                       ("e5m2", 64, 80)])
def test_fp8_store_random_with_scale(dtype, D, P):
    rng = np.random.default_rng(2)
    H, n_tok = 3, 200
    k = rng.standard_normal((n_tok, H, D)) * 3
    v = rng.standard_normal((n_tok, H, D)) * rng.lognormal(0, 0.5, (n_tok, 1, 1))
    pages = -(-n_tok // P) + 2
    spec = CacheSpec(dtype, "gqa", H, D, D, P, pages)
    slots = rng.permutation(pages * P)[:n_tok]
    slots[5] = -1                                          # skipped token
    cache, oc = _store_both(spec, k, v, slots, k_scale=0.0123, v_scale=0.007)
    _assert_bytes_equal(cache, oc)


def _mx_blocks(rng):
    blocks = []
    mags = F.E2M1.values[:8]
    mids = (mags[1:] + mags[:-1]) / 2
    b = I.bf16_bits(mids.astype(np.float32))
    near = np.concatenate([mids, I.bf16_to_f32(b + 1), I.bf16_to_f32(b - 1), mags, [6.5, 7.0, 7.5, 7.96875]])
    for s in (1.0, -1.0):
        for i in range(0, near.size, 15):
            blk = np.zeros(16)
            blk[0] = 4.0                                    # e = 0
            chunk = s * near[i:i + 15]
            blk[1:1 + chunk.size] = chunk
            blocks.append(blk)
    for _ in range(400):                                    # wide exponent range
        blocks.append(rng.standard_normal(16) * 2.0 ** rng.integers(-140, 120))
    blocks.append(np.zeros(16))
    z = np.zeros(16); z[3] = -0.0; blocks.append(z)
    blocks.append(np.full(16, 2.0 ** -133))                # e clamps to -127
    blocks.append(np.array([3e38] + [1.0] * 15))
    return np.array(blocks)


@pytest.mark.parametrize("P", [16, 48])
def test_mx16_store_bruteforce_blocks(P):
    rng = np.random.default_rng(3)
    blocks = _mx_blocks(rng)
    D, H = 128, 2
    per_tok = H * D // 16
    n_tok = -(-len(blocks) // per_tok)
    x = np.zeros((n_tok * per_tok, 16))
    x[: len(blocks)] = blocks
    k = x.reshape(n_tok, H, D)
    v = x[rng.permutation(len(x))].reshape(n_tok, H, D)
    pages = -(-n_tok // P) + 1
    spec = CacheSpec("mx16", "gqa", H, D, D, P, pages)
    slots = rng.permutation(pages * P)[:n_tok]
    cache, oc = _store_both(spec, k, v, slots)
    _assert_bytes_equal(cache, oc)


def test_nvfp4_store_with_computed_global_scale():
    rng = np.random.default_rng(4)
    n_tok = 300
    lat = rng.standard_normal((n_tok, 576))
    lat[:, rng.choice(576, 16, replace=False)] *= 8
    lat[7, 32:48] = 0.0                                     # an all-zero block
    lat[9, :16] = 1e-6                                      # a block whose E4M3 scale underflows
    latb = I.bf16_to_f32(I.bf16_bits(lat.astype(np.float32)))
    spec = CacheSpec("nvfp4", "mla", 1, 576, 512, 64, -(-n_tok // 64) + 1)
    cache = K.kvq_alloc_pages("nvfp4", "mla", 1, 576, 512, 64, spec.num_pages, device=DEV, fill=0xFF)
    g_dev = K.kvq_compute_scale(cache, _bf16_dev(latb))
    g = np.float32(g_dev.cpu().numpy()[0])
    assert g == Q.nvfp4_global_scale(np.abs(latb).max())
    slots = rng.permutation(spec.num_pages * 64)[:n_tok]
    K.kvq_store(cache, _bf16_dev(latb), None, torch.from_numpy(slots.astype(np.int64)).to(DEV), g_dev)
    torch.cuda.synchronize()
    oc = OracleCache(spec, fill=0xFF)
    oc.store(latb, None, slots, k_scale=g)
    _assert_bytes_equal(cache, oc)


@pytest.mark.parametrize("mag", [2.0 ** -56, 2.0 ** -40, 2.0 ** 50, 2.0 ** 100])
def test_nvfp4_store_extreme_magnitudes(mag):
    """Latents scaled so that the block divisors E4M3(s) * g fall inside and
    outside the range where the store divides by a reciprocal."""
    rng = np.random.default_rng(6)
    n_tok = 70
    lat = rng.standard_normal((n_tok, 576)) * mag
    lat[3, 64:80] *= 2.0 ** -30                             # blocks far below the tensor maximum
    latb = I.bf16_to_f32(I.bf16_bits(lat.astype(np.float32)))
    spec = CacheSpec("nvfp4", "mla", 1, 576, 512, 64, 3)
    cache = K.kvq_alloc_pages("nvfp4", "mla", 1, 576, 512, 64, spec.num_pages, device=DEV, fill=0xFF)
    g_dev = K.kvq_compute_scale(cache, _bf16_dev(latb))
    g = np.float32(g_dev.cpu().numpy()[0])
    slots = np.arange(2, 2 + n_tok)
    K.kvq_store(cache, _bf16_dev(latb), None, torch.from_numpy(slots.astype(np.int64)).to(DEV), g_dev)
    torch.cuda.synchronize()
    oc = OracleCache(spec, fill=0xFF)
    oc.store(latb, None, slots, k_scale=g)
    _assert_bytes_equal(cache, oc)


@pytest.mark.parametrize("dtype", ["e4m3", "e5m2", "nvfp4"])
def test_compute_scale_bit_exact(dtype):
    rng = np.random.default_rng(5)
    cache = K.kvq_alloc_pages(dtype, "mla" if dtype == "nvfp4" else "gqa", 1, 576 if dtype == "nvfp4" else 128,
                              512 if dtype == "nvfp4" else 128, 16 if dtype != "nvfp4" else 64, 1, device=DEV)
    for n0, n1 in ((1, 0), (1001, 0), (123457, 77), (3_000_001, 999)):
        a = rng.standard_normal(n0) * 10.0 ** rng.uniform(-3, 3)
        b = rng.standard_normal(n1) * 7 if n1 else None
        ab = I.bf16_to_f32(I.bf16_bits(a.astype(np.float32)))
        bb = None if b is None else I.bf16_to_f32(I.bf16_bits(b.astype(np.float32)))
        out = K.kvq_compute_scale(cache, _bf16_dev(ab), None if bb is None else _bf16_dev(bb))
        amax = max(np.abs(ab).max(), 0 if bb is None else np.abs(bb).max())
        want = Q.nvfp4_global_scale(amax) if dtype == "nvfp4" else Q.fp8_scale(amax, F.E4M3 if dtype == "e4m3" else F.E5M2)
        assert np.float32(out.cpu().numpy()[0]) == want
    zero = torch.zeros(100, dtype=torch.bfloat16, device=DEV)
    assert K.kvq_compute_scale(cache, zero).item() == 1.0


def test_tiny_workload_store_bytes():
    c = Case(I.WORKLOADS["tiny"]).run_gpu(decode=False)
    ks, vs = c.gpu_scales()
    oks, ovs = c.oracle_scales()
    assert ks == oks and vs == ovs
    oc, otable, pages, _ = c.oracle([0])
    for name in ("k_codes", "v_codes"):
        got = c.gpu_pages(name, pages)
        assert np.array_equal(got, getattr(oc, name)), name


def test_llama3_8b_store_bytes_sampled():
    """Full Llama-3-8B-shaped workload (batch 8, 20,480 tokens): prefill and
    the appended token, compared byte for byte on sequences 0 and 7."""
    c = Case(I.WORKLOADS["llama3_8b"]).run_gpu(decode=False)
    ks, vs = c.gpu_scales()
    oks, ovs = c.oracle_scales()
    assert ks == oks and vs == ovs
    oc, otable, pages, _ = c.oracle([0, 7])
    for name in ("k_codes", "v_codes"):
        assert np.array_equal(c.gpu_pages(name, pages), getattr(oc, name)), name
