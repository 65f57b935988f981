"""Full-size parity on the larger workloads, in the launch configuration the
benchmark uses: codes/scales of sampled sequences compared byte for byte,
decode outputs of sampled sequences within max-abs 4e-3 / rel-L2 1e-3 of the
float64 oracle. The quantization error against unquantized BF16 attention is
printed as information."""
import numpy as np
import pytest

from quantized_paged_kv_store_amd import inputs as I
from tests.kvq_cases import Case, assert_close, rel_l2

pytestmark = pytest.mark.gpu


def _check_case(c, ids, what):
    oc, otable, pages, _ = c.oracle(ids)
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        want = getattr(oc, name)
        if want is not None:
            assert np.array_equal(c.gpu_pages(name, pages), want), f"{what}: {name} differ"
    want, wlse, _, _ = c.oracle_decode(ids)
    got = c.out.cpu().numpy()
    mab, r = assert_close(got[ids], want[ids], what)
    assert np.allclose(c.lse.cpu().numpy()[ids], wlse[ids], rtol=0, atol=1e-4), what
    q = rel_l2(got[ids[0]], c.unquantized(ids[0]))
    print(f"{what}: max-abs {mab:.2e} rel-L2 {r:.2e}; quantization error vs BF16 attention rel-L2 {q:.3e}")


def test_llama3_70b_share_fp8_variants():
    """Batch 32, 64/8 heads, lengths U[16K, 32K]; E4M3 and E5M2, each with
    scale 1.0 and with the calibrated amax scale."""
    base = I.WORKLOADS["llama3_70b"]
    data = None
    lens = I.seq_lens(base)
    ids = [int(np.argmin(lens)), int(np.argmax(lens))]
    for dtype in ("e4m3", "e5m2"):
        for mode in ("amax", "one"):
            c = Case(base.with_(dtype=dtype, scale_mode=mode), data=data).run_gpu()
            data = c.data
            _check_case(c, ids, f"llama3_70b {dtype} scale={mode}")
            del c


def test_qwen3_235b_fp4_chunk_store_and_decode():
    """Batch 64, 64/4 heads, context 32,768, FP4 block-16: the last 2,048
    tokens of every sequence go through the chunk store, then decode."""
    c = Case(I.WORKLOADS["qwen3_235b"]).run_gpu()
    _check_case(c, [0, 63], "qwen3_235b mx16")


def test_dsr1_mla_nvfp4_sampled():
    """Batch 64, 128 heads over one 576-element latent, context 65,536, page
    64, NVFP4 with a computed global scale; oracle on sequences 0 and 63."""
    c = Case(I.WORKLOADS["dsr1_mla"]).run_gpu()
    _check_case(c, [0, 63], "dsr1_mla nvfp4")
