"""GPU parity of kvq_decode against the oracle (same seeded inputs, oracle
computed in float64 from its own quantization of them): max-abs <= 4e-3 and
rel-L2 <= 1e-3 on every checked output, LSE within 1e-4."""

import numpy as np
import pytest
import torch

import quantized_paged_kv_store_amd as K
from oracle import quantize as Q
from quantized_paged_kv_store_amd import inputs as I
from tests.kvq_cases import Case, assert_close, rel_l2

pytestmark = pytest.mark.gpu


def _check(c, batch_ids, what):
    want, wlse, _, _ = c.oracle_decode(batch_ids)
    got = c.out.cpu().numpy()
    glse = c.lse.cpu().numpy()
    res = assert_close(got[batch_ids], want[batch_ids], what)
    ok = np.isfinite(wlse[batch_ids])
    assert np.all(np.isneginf(glse[batch_ids][~ok])), what
    assert np.allclose(glse[batch_ids][ok], wlse[batch_ids][ok], rtol=0, atol=1e-4), what
    return res


def test_tiny_workload_decode():
    c = Case(I.WORKLOADS["tiny"]).run_gpu()
    mab, r = _check(c, [0], "tiny")
    q_err = rel_l2(c.out.cpu().numpy()[0], c.unquantized(0))
    print(f"tiny: max-abs {mab:.2e} rel-L2 {r:.2e}; quantization error vs BF16 attention rel-L2 {q_err:.3e}")


RAGGED = [0, 1, 15, 16, 17, 31, 33, 100, 257, 1000, 3001]


@pytest.mark.parametrize("dtype,D,G,P", [
    ("e4m3", 128, 4, 16), ("e4m3", 64, 1, 16), ("e4m3", 128, 16, 32), ("e5m2", 128, 8, 16),
    ("e5m2", 64, 3, 64), ("mx16", 128, 16, 16), ("mx16", 128, 4, 32), ("mx16", 128, 1, 16),
])
def test_ragged_lengths(dtype, D, G, P):
    hkv = 2
    w = I.Workload(f"ragged-{dtype}", dtype, "gqa", len(RAGGED), G * hkv, hkv, D, D, P, max(RAGGED), 0, 1,
                   "llama", seed=7)
    c = Case(w, lens=RAGGED).run_gpu()
    ids = list(range(len(RAGGED)))
    _check(c, ids, f"{dtype} D{D} G{G} P{P}")
    got = c.out.cpu().numpy()
    assert np.all(got[0] == 0) and np.all(np.isneginf(c.lse.cpu().numpy()[0]))


@pytest.mark.parametrize("dtype,D,G,P,target", [
    ("e4m3", 128, 4, 48, 90), ("mx16", 128, 8, 80, 64), ("e5m2", 64, 2, 48, 0), ("e4m3", 128, 16, 80, 200),
])
def test_pages_of_several_tiles_with_unaligned_splits(dtype, D, G, P, target):
    """Pages of 3 and 5 tiles (page sizes 48 and 80, not powers of two), with
    split targets that start splits inside a page: the page and tile-in-page
    of every load (the first pair's before the length is known, the rest
    from the staged page ids) come from divisions by the tiles per page."""
    hkv = 2
    w = I.Workload(f"pages-{dtype}-{P}", dtype, "gqa", len(RAGGED), G * hkv, hkv, D, D, P, max(RAGGED), 0, 1,
                   "llama", seed=17)
    c = Case(w, lens=RAGGED).run_gpu(split_target=target)
    _check(c, list(range(len(RAGGED))), f"{dtype} D{D} G{G} P{P} target {target}")


@pytest.mark.parametrize("dtype,hkv,G", [("e4m3", 32, 1), ("mx16", 16, 2)])
def test_many_kv_heads(dtype, hkv, G):
    """Many KV heads per page (32 and 16: 32 of them make a 64 KB FP8 page of 16
    tokens), including multi-head attention (G = 1)."""
    lens = [0, 5, 300, 2049]
    w = I.Workload(f"heads-{dtype}-{hkv}", dtype, "gqa", len(lens), G * hkv, hkv, 128, 128, 16, max(lens), 0, 1,
                   "llama", seed=19)
    c = Case(w, lens=lens).run_gpu()
    _check(c, list(range(len(lens))), f"{dtype} Hkv{hkv} G{G}")


class _TinyBlocksCase(Case):
    """K and V rows of every fifth token scaled by 2^-130 (input generation
    only; both sides see the same BF16 rows, many of them BF16 subnormals):
    every 16-element block of those rows has amax below 2^-124, so the store
    gives it E8M0 scale code 0, i.e. 2^-127."""

    def rows(self, b, t0, t1):
        k, v = super().rows(b, t0, t1)
        sel = (np.arange(t0, t1) % 5) == 2
        kf, vf = I.bf16_to_f32(k).copy(), I.bf16_to_f32(v).copy()
        kf[sel] *= np.float32(2.0 ** -130)
        vf[sel] *= np.float32(2.0 ** -130)
        return I.bf16_bits(kf), I.bf16_bits(vf)


def test_mx16_code0_blocks():
    """MX16 decode over blocks with E8M0 code 0 next to ordinary ones. The
    decode kernels take code 0 as 2^-126 (the scaled converts refuse the
    subnormal 2^-127); those blocks are below 1e-36, so the outputs still meet
    the parity bound against the oracle's exact 2^-127. Codes and scale bytes
    are compared byte for byte (the store quantizes subnormal BF16 inputs)."""
    lens = [17, 200, 1000]
    w = I.Workload("mx16-code0", "mx16", "gqa", len(lens), 8, 2, 128, 128, 16, max(lens), 0, 1, "llama", seed=23)
    c = _TinyBlocksCase(w, lens=lens).run_gpu()
    k, v = c.rows(2, 0, 10)
    _, sk = Q.quantize_mx16(I.bf16_to_f32(k[2]).astype(np.float64))
    _, sv = Q.quantize_mx16(I.bf16_to_f32(v[2]).astype(np.float64))
    assert np.all(sk == 0) and np.all(sv == 0)          # the scaled rows are all code-0 blocks
    ids = [0, 1, 2]
    want, wlse, oc, pages = c.oracle_decode(ids)
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert np.array_equal(c.gpu_pages(name, pages), getattr(oc, name)), name
    _check(c, ids, "mx16 code-0 blocks")


def test_single_token_equals_value_row():
    w = I.Workload("one", "e4m3", "gqa", 3, 8, 2, 128, 128, 16, 1, 1, 1, "llama", seed=8)
    c = Case(w).run_gpu()
    oc, otable, _, (ks, vs) = c.oracle([0, 1, 2])
    got = c.out.cpu().numpy()
    for b in range(3):
        for h in range(2):
            vrow = oc.dequant(otable[b, 0], 0, h, "v", ks, vs)[0]
            assert np.allclose(got[b, 4 * h:4 * h + 4], vrow[None, :], rtol=1e-6, atol=0)


def test_split_count_invariance():
    """1 split (direct write), a few, and many splits agree. They are not
    bit-identical: each split rounds its own p = 2^(s - m_split + 15) to fp16
    (unit roundoff 2^-11), so two split counts differ by up to ~2.5e-4 rel-L2."""
    w = I.WORKLOADS["llama3_8b"].with_(batch=2, max_len=6000, min_len=6000)
    c = Case(w).run_gpu(decode=False)
    outs = []
    for target in (1, 64, 100000):
        with K.split_target(c.cache, target):
            o, l = K.kvq_decode(c.cache, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(w),
                                c.k_scale, c.v_scale)
            outs.append((o.cpu().numpy(), l.cpu().numpy()))
    for o, l in outs[1:]:
        assert rel_l2(o, outs[0][0]) < 3e-4 and np.allclose(l, outs[0][1], atol=1e-5)


def _decode_at_target(c, w, target):
    """kvq_decode with the split planner aimed at `target` workgroups; also
    returns the workspace size that plan needs."""
    with K.split_target(c.cache, int(target)):
        ws = K.kvq_decode_workspace_bytes(c.cache, len(c.lens), w.q_heads, c.max_len)
        o, l = K.kvq_decode(c.cache, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(w),
                            c.k_scale, c.v_scale)
        torch.cuda.synchronize()
        return o, l, ws


@pytest.mark.parametrize("kind", ["gqa", "mla"])
def test_many_splits_merge(kind):
    """More than 64 splits of one sequence (the merge then holds two split
    LSEs per lane) up to the planners' cap of 128: GQA, 40,000 tokens at
    16-token tiles (125 splits); MLA, 8,192 tokens at 32-token steps (128
    splits). Checked against the oracle and against a launch with a few long
    splits, which differs only by each split's own fp16 rounding of p."""
    if kind == "gqa":
        w = I.WORKLOADS["llama3_8b"].with_(batch=1, max_len=40000, min_len=40000)
        c = Case(w).run_gpu(decode=False)
    else:
        w = I.Workload("mla-splits", "nvfp4", "mla", 1, 16, 1, 576, 512, 64, 8192, 0, 1, "mla", seed=11)
        c = Case(w, lens=[8192]).run_gpu(decode=False)
    dv = c.cache.desc.v_dim
    o_many, l_many, ws_many = _decode_at_target(c, w, "100000")
    o_few, l_few, _ = _decode_at_target(c, w, "1")
    # workspace = splits x (dv + 1) floats per (sequence, head), two 256-byte alignments
    assert ws_many > 64 * w.q_heads * (dv + 1) * 4 + 512, ws_many
    assert ws_many <= 128 * w.q_heads * (dv + 1) * 4 + 512, ws_many
    c.out, c.lse = o_many, l_many
    _check(c, [0], f"{kind} many splits")
    assert rel_l2(o_many.cpu().numpy(), o_few.cpu().numpy()) < 3e-4
    # fp32 sums of unrounded weights over differently placed splits: the oracle's LSE bound
    assert np.allclose(l_many.cpu().numpy(), l_few.cpu().numpy(), rtol=0, atol=1e-4)


def _tile_signs(t):
    """BF16 bits of +1 for tokens in 16-token tiles 0, 1, 4, 5, ... and -1 in
    tiles 2, 3, 6, 7, ...: every 4 tiles sum to 0."""
    return np.where((t >> 5) & 1, np.uint16(0xBF80), np.uint16(0x3F80))


def test_max_length_property():
    """The longest context decode accepts: 2,097,152 tokens = 128 splits of
    1,024 tiles. Every K row is the same, so the softmax weights are uniform;
    V cycles through 7 rows. Then out = the count-weighted mean of the 7
    dequantized V rows and LSE = sm_scale q.k^ + ln L, both from the oracle's
    quantizer on those rows only. V's first 16 elements are +-1 instead, by
    16-token tile in the pattern + + - - (see _tile_signs): their mean is
    exactly 0, and a lost, repeated or misplaced tile or 32-token step moves
    them by at least 16 / L = 7.6e-6, above the 1e-6 tolerance (the LSE
    alone would move by only ln(L / (L - 16)) = 7.6e-6, below its 1e-4)."""
    from oracle import quantize as Q
    from oracle.formats import E4M3
    L, P = 128 * 1024 * 16, 16
    w = I.Workload("maxlen", "e4m3", "gqa", 1, 4, 1, 128, 128, P, L, L, 0, "llama", seed=12)
    rng = np.random.default_rng(12)
    k0 = I.bf16_bits(rng.standard_normal(128).astype(np.float32))
    v7 = I.bf16_bits(rng.standard_normal((7, 128)).astype(np.float32))
    c = Case(w, lens=[L])
    t = np.arange(L)
    kp = np.broadcast_to(k0, (L, 1, 128)).copy()   # rows [n, Hkv, D]
    vp = v7[t % 7][:, None, :].copy()
    vp[:, 0, :16] = _tile_signs(t)[:, None]
    c.data = {"pre": (kp, vp, I.slots_for(c.table[0], t, P)), "new": (None, None, np.zeros(0, np.int64))}
    c.run_gpu()
    assert K.kvq_decode_workspace_bytes(c.cache, 1, 4, L) == 4 * 128 * (128 + 1) * 4  # 128 splits
    ks, vs = c.oracle_scales()
    khat = Q.dequantize_fp8(Q.quantize_fp8(I.bf16_to_f32(k0).astype(np.float64), ks, E4M3), ks, E4M3)
    vhat = Q.dequantize_fp8(Q.quantize_fp8(I.bf16_to_f32(v7).astype(np.float64), vs, E4M3), vs, E4M3)
    counts = np.bincount(t % 7, minlength=7).astype(np.float64)
    want = counts @ vhat / L
    want[:16] = 0.0      # +-1 (symmetric codes) in equal numbers
    q = I.bf16_to_f32(c.q[0]).astype(np.float64)
    want_lse = I.sm_scale(w) * (q @ khat) + np.log(L)
    got, glse = c.out.cpu().numpy()[0], c.lse.cpu().numpy()[0]
    assert np.allclose(got, want[None, :], rtol=1e-5, atol=1e-6), np.abs(got - want).max()
    assert np.allclose(glse, want_lse, rtol=0, atol=1e-4), (glse, want_lse)


def test_mla_max_length_property():
    """MLA at the longest accepted context (2,097,152 tokens, 128 splits of
    256 pages of 64). The query's first 512 dims are zero and every latent row
    has the same rope dims, so the weights are uniform while the value part
    (dims 0..511) cycles through 7 rows: out = their count-weighted mean after
    NVFP4 rounding, LSE = sm_scale q_rope.k^_rope + ln L (the oracle's
    quantizer on the 7 rows; the rope dims are whole 16-element blocks). The
    first 16-element block is +-1 by 16-token tile (+ + - -): its mean is 0,
    and a lost, repeated or misplaced tile or 32-token step moves it by at
    least 16 / L, above the 1e-6 tolerance."""
    from oracle import quantize as Q
    L, P = 128 * 1024 * 16, 64
    w = I.Workload("mla-maxlen", "nvfp4", "mla", 1, 16, 1, 576, 512, P, L, L, 0, "mla", seed=13)
    rng = np.random.default_rng(13)
    rows = I.bf16_bits(np.concatenate([rng.standard_normal((7, 512)), np.tile(rng.standard_normal(64), (7, 1))],
                                      axis=1).astype(np.float32))
    c = Case(w, lens=[L])
    t = np.arange(L)
    lat_rows = rows[t % 7]
    lat_rows[:, :16] = _tile_signs(t)[:, None]
    c.data = {"pre": (lat_rows, None, I.slots_for(c.table[0], t, P)), "new": (None, None, np.zeros(0, np.int64))}
    c.run_gpu(decode=False)
    qz = c.q.copy()
    qz[..., :512] = 0
    o, l = K.kvq_decode(c.cache, c._bf16(qz), c.table_dev, c.lens_dev, L, I.sm_scale(w), c.k_scale, None)
    torch.cuda.synchronize()
    g, _ = c.oracle_scales()
    lat = Q.dequantize_nvfp4(*Q.quantize_nvfp4(I.bf16_to_f32(rows).astype(np.float64), g), g)
    counts = np.bincount(t % 7, minlength=7).astype(np.float64)
    want = counts @ lat[:, :512] / L
    want[:16] = 0.0      # a block of equal magnitudes: +-(the same value) in equal numbers
    q = I.bf16_to_f32(qz[0]).astype(np.float64)
    want_lse = I.sm_scale(w) * (q[:, 512:] @ lat[0, 512:]) + np.log(L)
    got, glse = o.cpu().numpy()[0], l.cpu().numpy()[0]
    assert np.allclose(got, want[None, :], rtol=1e-5, atol=1e-6), np.abs(got - want).max()
    assert np.allclose(glse, want_lse, rtol=0, atol=1e-4), (glse, want_lse)


def test_llama3_8b_decode_sampled():
    """The benchmark workload at full size (batch 8, 20,480 tokens, FP8 E4M3,
    launch configuration as timed); oracle on sequences 0 and 5."""
    c = Case(I.WORKLOADS["llama3_8b"]).run_gpu()
    mab, r = _check(c, [0, 5], "llama3_8b")
    q_err = rel_l2(c.out.cpu().numpy()[0], c.unquantized(0))
    print(f"llama3_8b: max-abs {mab:.2e} rel-L2 {r:.2e}; quantization error vs BF16 attention rel-L2 {q_err:.3e}")


@pytest.mark.parametrize("hq,P", [(128, 64), (64, 16), (128, 32), (16, 64), (96, 16), (40, 32), (1, 64), (128, 48),
                                  (64, 96)])
def test_mla_ragged_lengths(hq, P):
    lens = [0, 1, 17, 64, 100, 1000, 2500]
    w = I.Workload(f"mla-ragged-{hq}", "nvfp4", "mla", len(lens), hq, 1, 576, 512, P, max(lens), 0, 1, "mla", seed=9)
    c = Case(w, lens=lens).run_gpu()
    ids = list(range(len(lens)))
    _check(c, ids, f"mla Hq{hq} P{P}")
    assert np.all(c.out.cpu().numpy()[0] == 0)


def test_mla_split_count_invariance():
    w = I.WORKLOADS["dsr1_mla"].with_(batch=2, max_len=9000, min_len=9000)
    c = Case(w).run_gpu(decode=False)
    outs = []
    for target in (1, 32, 100000):
        with K.split_target(c.cache, target):
            o, l = K.kvq_decode(c.cache, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(w), c.k_scale, None)
            outs.append((o.cpu().numpy(), l.cpu().numpy()))
    for o, l in outs[1:]:
        assert rel_l2(o, outs[0][0]) < 3e-4 and np.allclose(l, outs[0][1], atol=1e-5)


class _RampCase(Case):
    """The 64 rope dims of latent row t scaled by 1 + 0.015 t (input generation
    only; both sides see the same BF16 rows). They enter the scores but not
    V, so the largest score of each 32-token step keeps climbing while the
    outputs stay unit-scale: the MLA kernel's lazy reference maximum moves
    again and again inside one split and its accumulators are rescaled."""

    def rows(self, b, t0, t1):
        k, v = super().rows(b, t0, t1)
        kf = I.bf16_to_f32(k)
        kf[:, 512:] *= (1.0 + 0.015 * np.arange(t0, t1, dtype=np.float32))[:, None]
        return I.bf16_bits(kf), v


@pytest.mark.parametrize("hq,P,target", [(128, 64, "3"), (64, 16, "3"), (128, 64, None)])
def test_mla_reference_moves(hq, P, target):
    lens = [3000, 1500, 33]
    w = I.Workload(f"mla-ramp-{hq}", "nvfp4", "mla", len(lens), hq, 1, 576, 512, P, max(lens), 0, 1, "mla", seed=19)
    # the inputs do what the test is for: on sequence 0, head 0, the running
    # maximum of the (log2-domain) scores rises past the reference + 2^8 many
    # times after the first 32-token step
    c = _RampCase(w, lens=lens)
    k, _ = c.rows(0, 0, lens[0])
    q = I.bf16_to_f32(I.queries(w))[0, 0]
    s2 = (I.bf16_to_f32(k) @ q) * I.sm_scale(w) / np.log(2.0)
    ref, moves = s2[:32].max(), 0
    for t0 in range(32, lens[0], 32):
        m = s2[t0:t0 + 32].max()
        if m > ref + 8.0:
            ref, moves = m, moves + 1
    assert moves >= 5, moves
    # target 3: one split per sequence, the direct output path
    c.run_gpu(split_target=0 if target is None else int(target))
    ids = [0, 1, 2]
    what = f"mla ramp Hq{hq} P{P} target {target}"
    want, wlse, _, _ = c.oracle_decode(ids)
    assert_close(c.out.cpu().numpy()[ids], want[ids], what)
    # LSE: these scores reach ~10^2, so their fp32 accumulation error counts.
    # An LSE moves by at most the largest error of its scores, and a score's
    # error is at most sm_scale * gamma_576 * sum_i |q_i k_i| (k^ within 1.5x
    # of the BF16 row for NVFP4), so that bound (plus 1e-4) is the tolerance.
    gamma = 576 * 2.0 ** -24 / (1 - 576 * 2.0 ** -24)
    qa = np.abs(I.bf16_to_f32(I.queries(w)))
    glse = c.lse.cpu().numpy()
    for b in ids:
        ka = np.abs(I.bf16_to_f32(c.rows(b, 0, lens[b])[0]))
        tol = 1e-4 + I.sm_scale(w) * gamma * 1.5 * float((qa[b] @ ka.T).max())
        assert np.allclose(glse[b], wlse[b], rtol=0, atol=tol), (what, b, tol, np.abs(glse[b] - wlse[b]).max())


@pytest.mark.parametrize("dtype", ["e4m3", "mx16"])
def test_one_workspace_serves_calls_of_any_shape(dtype):
    """One workspace, sized for the largest call, serves calls of different
    batch sizes and split counts in any order, with results bit-identical to
    calls on fresh workspaces (nothing of an earlier call's partials leaks)."""
    lens = [0, 1, 17, 2000, 9000, 20000]
    w = I.Workload(f"merge-{dtype}", dtype, "gqa", len(lens), 16, 4, 128, 128, 16, max(lens), 0, 1, "llama",
                   seed=71)
    c = Case(w, lens=lens).run_gpu(decode=False)
    shapes = [(6, 20000), (3, 2000), (6, 20000), (4, 9000), (1, 1), (6, 20000)]
    need = max(K.kvq_decode_workspace_bytes(c.cache, b, w.q_heads, m) for b, m in shapes)
    shared = torch.full((need,), 0x7F, dtype=torch.uint8, device=c.dev)        # NaN bytes to start with
    for b, m in shapes:
        lens_b = torch.clamp(c.lens_dev[:b], max=m).contiguous()
        q = c.q_dev[:b].contiguous()
        table = c.table_dev[:b].contiguous()
        o1, l1 = K.kvq_decode(c.cache, q, table, lens_b, m, I.sm_scale(w), c.k_scale, c.v_scale, workspace=shared)
        o2, l2 = K.kvq_decode(c.cache, q, table, lens_b, m, I.sm_scale(w), c.k_scale, c.v_scale)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (b, m)
    want, wlse, _, _ = c.oracle_decode([3, 5])
    o, l = K.kvq_decode(c.cache, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(w), c.k_scale, c.v_scale,
                        workspace=shared)
    assert_close(o.cpu().numpy()[[3, 5]], want[[3, 5]], f"merge {dtype}")
    assert np.allclose(l.cpu().numpy()[[3, 5]], wlse[[3, 5]], rtol=0, atol=1e-4)
