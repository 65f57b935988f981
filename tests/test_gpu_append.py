"""GPU parity of kvq_decode_append (append the token at position L-1 of every
sequence, then decode, in one launch) against kvq_store followed by
kvq_decode on the same inputs: the cache bytes must be bit-identical, the
outputs identical, and both within tolerance of the oracle."""
import numpy as np
import pytest
import torch

from quantized_paged_kv_store_amd import inputs as I
from tests.kvq_cases import Case, assert_close

pytestmark = pytest.mark.gpu

# ragged lengths: empty, single token, tile and page boundaries, several splits
LENS = [0, 1, 15, 16, 17, 64, 65, 100, 1000, 3001]


def _pair(w, lens):
    a = Case(w, lens=lens).run_gpu()
    b = Case(w, lens=lens, data=a.data).run_gpu(append=True)
    torch.cuda.synchronize()
    return a, b


def _check(a, b, what, oracle_ids):
    assert torch.equal(a.cache.memory, b.cache.memory), f"{what}: cache bytes differ"
    assert torch.equal(a.out, b.out), f"{what}: outputs differ"
    assert torch.equal(a.lse, b.lse), f"{what}: lse differ"
    want, wlse, _, _ = b.oracle_decode(oracle_ids)
    got = b.out.cpu().numpy()
    assert_close(got[oracle_ids], want[oracle_ids], what)
    glse = b.lse.cpu().numpy()[oracle_ids]
    ok = np.isfinite(wlse[oracle_ids])
    assert np.all(np.isneginf(glse[~ok]))
    assert np.allclose(glse[ok], wlse[oracle_ids][ok], rtol=0, atol=1e-4)


@pytest.mark.parametrize("dtype,D,G,P", [
    ("e4m3", 128, 4, 16), ("e5m2", 64, 3, 64), ("e4m3", 128, 16, 32), ("mx16", 128, 8, 16), ("mx16", 128, 4, 32),
])
def test_append_gqa(dtype, D, G, P):
    w = I.Workload(f"append-{dtype}", dtype, "gqa", len(LENS), 2 * G, 2, D, D, P, max(LENS), 0, 1, "llama", seed=21)
    a, b = _pair(w, LENS)
    _check(a, b, f"append {dtype} D{D} G{G} P{P}", [0, 1, 4, 9])


@pytest.mark.parametrize("dtype,D,G,P,target", [("e4m3", 128, 4, 48, 100), ("mx16", 128, 8, 80, 90),
                                                ("e5m2", 64, 2, 48, 140)])
def test_append_gqa_pages_of_several_tiles(dtype, D, G, P, target):
    """Pages of 3 and 5 tiles and splits that start inside a page: the
    appended token's tile is found by division, and a wave whose first tile
    pair (loaded before the length is known) holds it reads that pair again
    after the append."""
    w = I.Workload(f"append-{dtype}-{P}", dtype, "gqa", len(LENS), 2 * G, 2, D, D, P, max(LENS), 0, 1, "llama",
                   seed=23)
    a = Case(w, lens=LENS).run_gpu(split_target=target)
    b = Case(w, lens=LENS, data=a.data).run_gpu(append=True, split_target=target)
    torch.cuda.synchronize()
    _check(a, b, f"append {dtype} D{D} G{G} P{P} target {target}", [0, 1, 4, 7, 9])


@pytest.mark.parametrize("hq,P", [(128, 64), (64, 16), (16, 64)])
def test_append_mla(hq, P):
    w = I.Workload(f"append-mla-{hq}", "nvfp4", "mla", len(LENS), hq, 1, 576, 512, P, max(LENS), 0, 1, "mla",
                   seed=22)
    a, b = _pair(w, LENS)
    _check(a, b, f"append mla Hq{hq} P{P}", [1, 2, 9])


def test_append_llama3_8b_full_size():
    """The benchmark workload at full size, in the launch configuration the
    benchmark times (batch 8, context 20,480, FP8 E4M3)."""
    w = I.WORKLOADS["llama3_8b"]
    a = Case(w).run_gpu()
    b = Case(w, data=a.data).run_gpu(append=True)
    torch.cuda.synchronize()
    assert torch.equal(a.cache.memory, b.cache.memory)
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)
