"""FP8-domain decode through the HIP path (vLLM "Quantized KV Cache" page:
with an FP8 cache the attention runs in FP8, the query quantized like K and V,
q_scale per tensor or per query head): query scales calibrated on the GPU
bit-exact with the oracle's, and kvq_decode_fp8q / kvq_decode_append_fp8q
within the parity tolerance of oracle.attention.decode_attention_fp8q fed the
same stored codes and the same scales. On the NVFP4 MLA latent the keys are
the E4M3 rows of the dequantize_prev_kv step (output scale 8g), checked
against oracle.attention.decode_attention_mla_fp8q."""
import numpy as np
import pytest
import torch

import quantized_paged_kv_store_amd as K
from oracle import formats as F
from oracle import quantize as Q
from oracle.attention import decode_attention_fp8q, decode_attention_mla_fp8q, mla_fp8_keys, quantize_query_fp8
from quantized_paged_kv_store_amd import inputs as I
from tests.kvq_cases import Case, assert_close, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda"
LENS = [0, 1, 15, 16, 17, 300, 2048, 5000]


def _workload(dtype, lens, G=4, hkv=2, D=128, P=16, per_head=False):
    return I.Workload(f"fp8q-{dtype}", dtype, "gqa", len(lens), G * hkv, hkv, D, D, P, max(lens), 0, 1, "llama",
                      scale_mode="amax_head" if per_head else "amax", seed=61)


@pytest.mark.parametrize("per_head,hq,D", [(False, 32, 128), (True, 32, 128), (True, 12, 64), (False, 7, 64)])
def test_compute_q_scale_bit_exact(per_head, hq, D):
    hkv = 1 if hq % 2 else 4 if hq % 4 == 0 else 2
    cache = K.kvq_alloc_pages("e4m3", "gqa", hkv, D, D, 16, 1, device=DEV, scale_mode="head" if per_head else "tensor")
    rng = np.random.default_rng(hq + D)
    for n in (0, 1, 333, 4096):
        q = rng.standard_normal((n, hq, D)) * (10.0 ** rng.uniform(-3, 3, size=(1, hq, 1)))
        if n:
            q[:, 1] = 0.0                                             # an all-zero head -> 1.0
        qb = I.bf16_bits(q.astype(np.float32))
        got = K.kvq_compute_q_scale(cache, torch.from_numpy(qb).to(DEV).view(torch.bfloat16)).cpu().numpy()
        want = Q.fp8_query_scales(I.bf16_to_f32(qb), per_head)
        assert got.dtype == np.float32 and np.array_equal(got, want), n


def _q_scale(c, per_head, how):
    """Calibrated on the decode queries themselves ("cal"), 1.0 (None), or a
    stale scale 1/8 of the calibrated one so that queries saturate."""
    if how == "none":
        return None, None
    s = K.kvq_compute_q_scale(c.cache, c.q_dev.view(c.w.batch, c.w.q_heads, c.w.head_dim))
    host = s.cpu().numpy()
    assert np.array_equal(host, Q.fp8_query_scales(I.bf16_to_f32(c.q), per_head))
    if how == "stale":
        s = s * 0.125
        host = (host * np.float32(0.125)).astype(np.float32)
    return s, host


def _lse_bound(c, oc, otable, qf, qs_host, ks, vs, ids):
    """LSE tolerance of the FP8-domain path: 1e-4 plus the FP8 matrix cores'
    own accumulation error. gfx950's v_mfma_f32_16x16x32_{fp8,bf8}_fp8 is not
    an exact fp32 accumulate: measured over 4M random dot products, the error
    of one 32-element product reaches 2^-11.3 of the sum of |products| when
    the products span many binades (it is exact over a few binades and with
    subnormal codes). Taken as 2^-10 of sm * sum_d |q^_d k^_d| for the worst
    token of each (sequence, head): the LSE moves by at most the largest
    score error."""
    w = c.w
    codes, s = quantize_query_fp8(qf, qs_host)
    qh = F.decode(codes.astype(np.int64), F.E4M3) * s[None, :, None].astype(np.float64)
    bound = np.full((w.batch, w.q_heads), 1e-4)
    P, G = w.page_size, w.group
    for b in ids:
        L = int(c.lens[b])
        if L == 0:
            continue
        t = np.arange(L)
        page = otable[b][t // P].astype(np.int64)
        for h in range(w.kv_heads):
            kh = np.abs(oc.dequant(page, t % P, h, "k", ks, vs))                 # [L, D]
            worst = (np.abs(qh[b, h * G:(h + 1) * G]) @ kh.T).max(axis=1)       # [G]
            bound[b, h * G:(h + 1) * G] += 2.0 ** -10 * I.sm_scale(w) * worst
    return bound


def _check(c, out, lse, qs_host, ids, what):
    oc, otable, pages, (ks, vs) = c.oracle(ids)
    qf = I.bf16_to_f32(c.q).astype(np.float64)
    want, wlse = decode_attention_fp8q(oc, qf, otable, c.lens, I.sm_scale(c.w), qs_host, ks, vs, batch_ids=ids)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert_close(o[ids], want[ids], what)
    bound = _lse_bound(c, oc, otable, qf, qs_host, ks, vs, ids)
    fin = np.isfinite(wlse[ids])
    assert np.array_equal(fin, np.isfinite(l[ids]))
    assert np.all(np.abs(l[ids][fin] - wlse[ids][fin]) <= bound[ids][fin]), what
    for b in ids:
        if c.lens[b] == 0:
            assert np.all(o[b] == 0) and np.isneginf(l[b]).all()


@pytest.mark.parametrize("dtype,D,G,P,per_head,how", [
    ("e4m3", 128, 4, 16, False, "cal"),
    ("e4m3", 128, 16, 32, True, "cal"),
    ("e5m2", 128, 8, 16, False, "cal"),
    ("e4m3", 64, 3, 16, True, "cal"),
    ("e5m2", 64, 1, 64, True, "stale"),
    ("e4m3", 128, 4, 16, False, "stale"),
    ("e4m3", 128, 2, 16, False, "none"),
    ("e4m3", 128, 4, 48, True, "cal"),
])
def test_fp8q_decode_matches_oracle(dtype, D, G, P, per_head, how):
    c = Case(_workload(dtype, LENS, G=G, D=D, P=P, per_head=per_head), lens=LENS).run_gpu(decode=False)
    qs, qs_host = _q_scale(c, per_head, how)
    out, lse = K.kvq_decode_fp8q(c.cache, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(c.w), qs,
                                 c.k_scale, c.v_scale)
    torch.cuda.synchronize()
    _check(c, out, lse, qs_host, [0, 1, 2, 4, 6, 7], f"fp8q {dtype} D{D} G{G} P{P} {how}")


def test_fp8q_append_matches_store_then_decode():
    lens = [1, 16, 33, 1000, 3001]
    w = _workload("e4m3", lens, G=8, per_head=True)
    a = Case(w, lens=lens).run_gpu(decode=False)
    b = Case(w, lens=lens, data=a.data).run_gpu(decode=False, append=True)
    qs, qs_host = _q_scale(a, True, "cal")
    oa, la = K.kvq_decode_fp8q(a.cache, a.q_dev, a.table_dev, a.lens_dev, a.max_len, I.sm_scale(w), qs,
                               a.k_scale, a.v_scale)
    ob, lb = K.kvq_decode_append_fp8q(b.cache, *b.append_rows, b.q_dev, b.table_dev, b.lens_dev, b.max_len,
                                      I.sm_scale(w), qs, b.k_scale, b.v_scale)
    torch.cuda.synchronize()
    for name in ("k_codes", "v_codes"):            # (the scratch differs: only a's calibrated q_scale)
        assert torch.equal(a.cache.view(name), b.cache.view(name)), name
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    _check(b, ob, lb, qs_host, [0, 3, 4], "fp8q append")


def test_fp8q_llama3_8b_shape_sampled():
    """The 8B decode shape (batch 8, context 20,480, tensor scales) in the
    benchmark's launch configuration (one-launch append step); oracle on
    sequences 0 and 6."""
    w = I.WORKLOADS["llama3_8b"]
    c = Case(w).run_gpu(decode=False, append=True)
    qs, qs_host = _q_scale(c, False, "cal")
    out, lse = K.kvq_decode_append_fp8q(c.cache, *c.append_rows, c.q_dev, c.table_dev, c.lens_dev, c.max_len,
                                        I.sm_scale(w), qs, c.k_scale, c.v_scale)
    torch.cuda.synchronize()
    _check(c, out, lse, qs_host, [0, 6], "fp8q llama3_8b")


# ------------------------------------------------------------------ MLA --
def _mla_workload(lens, hq=128, P=64, seed=23):
    return I.Workload(f"fp8q-mla-{hq}", "nvfp4", "mla", len(lens), hq, 1, 576, 512, P, max(lens), 0, 1, "mla",
                      seed=seed)


def _mla_q_scale(c, how):
    """Per-tensor query scale calibrated on the decode queries ("cal"), 1.0
    (None), or 1/8 of the calibrated one so that queries saturate."""
    if how == "none":
        return None, None
    s = K.kvq_compute_q_scale(c.cache, c.q_dev.view(c.w.batch, c.w.q_heads, c.w.head_dim))
    host = s.cpu().numpy()
    assert host.shape == (1,) and np.array_equal(host, Q.fp8_query_scales(I.bf16_to_f32(c.q), False))
    if how == "stale":
        s = s * 0.125
        host = (host * np.float32(0.125)).astype(np.float32)
    return s, host


def _mla_lse_bound(oc, otable, qh, lens, g, sm, ids):
    """1e-4 plus the FP8 matrix cores' accumulation error, taken (as for the
    GQA caches above) as 2^-10 of sm * sum_d |q^_d k8^_d| for the worst token
    of each (sequence, head), with k8^ the E4M3 key rows times 8g."""
    bound = np.full(qh.shape[:2], 1e-4)
    for b in ids:
        L = int(lens[b])
        if L == 0:
            continue
        k8, s8 = mla_fp8_keys(oc, otable[b], L, g)
        kh = np.abs(F.decode(k8.astype(np.int64), F.E4M3)) * np.float64(s8)
        bound[b] += 2.0 ** -10 * sm * (np.abs(qh[b]) @ kh.T).max(axis=1)
    return bound


def _mla_check(c, out, lse, qs_host, ids, what):
    oc, otable, _, (g, _) = c.oracle(ids)
    qf = I.bf16_to_f32(c.q).astype(np.float64)
    sm = I.sm_scale(c.w)
    want, wlse = decode_attention_mla_fp8q(oc, qf, otable, c.lens, sm, qs_host, g=g, batch_ids=ids)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    mab, r = assert_close(o[ids], want[ids], what)
    codes, s = quantize_query_fp8(qf, qs_host)
    qh = F.decode(codes.astype(np.int64), F.E4M3) * s[None, :, None].astype(np.float64)
    bound = _mla_lse_bound(oc, otable, qh, c.lens, g, sm, ids)
    fin = np.isfinite(wlse[ids])
    assert np.array_equal(fin, np.isfinite(l[ids])), what
    err = np.abs(l[ids][fin] - wlse[ids][fin])
    assert np.all(err <= bound[ids][fin]), (what, float(err.max()))
    for b in ids:
        if c.lens[b] == 0:
            assert np.all(o[b] == 0) and np.isneginf(l[b]).all()
    return mab, r


@pytest.mark.parametrize("hq,P,how", [(128, 64, "cal"), (128, 16, "none"), (64, 32, "cal"), (40, 64, "stale"),
                                      (16, 16, "cal"), (1, 64, "cal"), (128, 48, "cal")])
def test_mla_fp8q_matches_oracle(hq, P, how):
    lens = [0, 1, 17, 64, 100, 1000, 2500]
    c = Case(_mla_workload(lens, hq, P), lens=lens).run_gpu(decode=False)
    qs, qs_host = _mla_q_scale(c, how)
    out, lse = K.kvq_decode_fp8q(c.cache, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(c.w), qs,
                                 c.k_scale, None)
    torch.cuda.synchronize()
    _mla_check(c, out, lse, qs_host, list(range(len(lens))), f"mla fp8q Hq{hq} P{P} {how}")


def test_mla_fp8q_splits_and_append():
    """Several splits per sequence (the merge path), and the one-launch
    append bit-identical to store + decode."""
    lens = [9000, 4097, 33, 2]
    w = _mla_workload(lens, seed=29)
    a = Case(w, lens=lens).run_gpu(decode=False)
    b = Case(w, lens=lens, data=a.data).run_gpu(decode=False, append=True)
    qs, qs_host = _mla_q_scale(a, "cal")
    outs = []
    for target in (1, 0, 4096):
        with K.split_target(a.cache, target):
            outs.append(K.kvq_decode_fp8q(a.cache, a.q_dev, a.table_dev, a.lens_dev, a.max_len, I.sm_scale(w), qs,
                                          a.k_scale, None))
    ob, lb = K.kvq_decode_append_fp8q(b.cache, b.append_rows[0], None, b.q_dev, b.table_dev, b.lens_dev, b.max_len,
                                      I.sm_scale(w), qs, b.k_scale, None)
    torch.cuda.synchronize()
    for name in ("k_codes", "k_scales"):
        assert torch.equal(a.cache.view(name), b.cache.view(name)), name
    assert torch.equal(outs[1][0], ob) and torch.equal(outs[1][1], lb)
    for o, l in outs:
        _mla_check(a, o, l, qs_host, [0, 1, 2, 3], "mla fp8q splits")


def test_mla_fp8q_dsr1_shape_sampled():
    """The DeepSeek-R1 MLA decode shape (batch 64, 128 heads, context 65,536,
    page 64) in the benchmark's launch configuration (one-launch append
    step); oracle on sequences 0 and 63. Prints the quantization error of
    both MLA paths against BF16 attention on the unquantized latent."""
    w = I.WORKLOADS["dsr1_mla"]
    c = Case(w).run_gpu(decode=False, append=True)
    qs, qs_host = _mla_q_scale(c, "cal")
    out, lse = K.kvq_decode_append_fp8q(c.cache, c.append_rows[0], None, c.q_dev, c.table_dev, c.lens_dev,
                                        c.max_len, I.sm_scale(w), qs, c.k_scale, None)
    o16, _ = K.kvq_decode(c.cache, c.q_dev, c.table_dev, c.lens_dev, c.max_len, I.sm_scale(w), c.k_scale, None)
    torch.cuda.synchronize()
    mab, r = _mla_check(c, out, lse, qs_host, [0, 63], "mla fp8q dsr1")
    ref = c.unquantized(0)
    print(f"dsr1_mla FP8-domain: max-abs {mab:.2e} rel-L2 {r:.2e} against the oracle; against BF16 attention "
          f"rel-L2 {rel_l2(out.cpu().numpy()[0], ref):.3e} (fp16 path {rel_l2(o16.cpu().numpy()[0], ref):.3e})")
