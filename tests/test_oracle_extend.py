"""Pins for oracle.attention.extend_attention (extend attention over a
quantized prefix read through E4M3 workspaces: PR #21954 analysis page,
"code analysis", dequantize_prev_kv and the FP8 prefill it feeds).

- against torch's scaled_dot_product_attention in float64 with a causal
  mask offset by the prefix length, on prefixes whose values sit exactly on
  the E4M3 grid (so the workspace codes hold them exactly);
- causality: changing chunk token j moves only rows j and later;
- closed forms (single key; zero query = mean of the visible values);
- the workspace's page indexing (page_off, page size) against a permuted
  page order.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import formats as F
from oracle.attention import extend_attention
from quantized_paged_kv_store_amd.inputs import bf16_bits, bf16_to_f32


def _grid_prefix(rng, n, hkv, d, s):
    """E4M3 codes (no NaN) and their values times s."""
    mag = rng.integers(0, 0x7F, (n, hkv, d))
    codes = (mag | (rng.integers(0, 2, (n, hkv, d)) << 7)).astype(np.uint8)
    return codes, F.decode(codes.astype(np.int64), F.E4M3) * s


def _case(seed, lens0, lens_c, hkv=2, G=3, D=32, P=16, s_k=0.125, s_v=0.0625):
    """Random extend inputs; every sequence's prefix pages are consecutive in
    the workspace, in reverse sequence order (page_off exercised)."""
    rng = np.random.default_rng(seed)
    B = len(lens0)
    npg = [(l + P - 1) // P for l in lens0]
    page_off = np.zeros(B, np.int64)
    off = 0
    for b in reversed(range(B)):
        page_off[b] = off
        off += npg[b]
    n_pages = max(off, 1)
    dq_k = np.zeros((n_pages, hkv, P, D), np.uint8)
    dq_v = np.zeros((n_pages, hkv, P, D), np.uint8)
    pk, pv = [], []
    for b in range(B):
        ck, vk = _grid_prefix(rng, lens0[b], hkv, D, s_k)
        cv, vv = _grid_prefix(rng, lens0[b], hkv, D, s_v)
        t = np.arange(lens0[b])
        dq_k[page_off[b] + t // P, :, t % P] = ck
        dq_v[page_off[b] + t // P, :, t % P] = cv
        pk.append(vk)
        pv.append(vv)
    cu = np.concatenate([[0], np.cumsum(lens_c)])
    nq = int(cu[-1])
    bf = lambda a: bf16_to_f32(bf16_bits(a.astype(np.float32))).astype(np.float64)
    q = bf(rng.standard_normal((nq, hkv * G, D)))
    kn = bf(rng.standard_normal((nq, hkv, D)))
    vn = bf(rng.standard_normal((nq, hkv, D)))
    return dict(q=q, k_new=kn, v_new=vn, cu_q=cu, prefix_len=np.asarray(lens0), dq_k=dq_k, dq_v=dq_v,
                page_off=page_off, s_k=np.float32(s_k), s_v=np.float32(s_v)), pk, pv


def test_matches_torch_sdpa_with_offset_causal_mask():
    sm = 0.17
    args, pk, pv = _case(1, [37, 0, 16, 5], [9, 4, 1, 20])
    out, lse = extend_attention(**args, sm_scale=sm)
    G = args["q"].shape[1] // args["k_new"].shape[1]
    cu = args["cu_q"]
    for b in range(4):
        L0, C = len(pk[b]), cu[b + 1] - cu[b]
        r = slice(cu[b], cu[b + 1])
        K = np.concatenate([pk[b], args["k_new"][r]])              # [L0 + C, Hkv, D]
        V = np.concatenate([pv[b], args["v_new"][r]])
        Kt = torch.from_numpy(K.transpose(1, 0, 2)).repeat_interleave(G, 0)[None]
        Vt = torch.from_numpy(V.transpose(1, 0, 2)).repeat_interleave(G, 0)[None]
        qt = torch.from_numpy(args["q"][r].transpose(1, 0, 2).copy())[None]
        mask = torch.from_numpy(np.arange(L0 + C)[None, :] <= (L0 + np.arange(C))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=sm)
        assert np.allclose(out[r], ref[0].numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-13)
        s = sm * np.einsum("chd,lhd->chl", args["q"][r], np.repeat(K, G, axis=1))
        s = np.where(mask.numpy()[:, None, :], s, -np.inf)
        assert np.allclose(lse[r], logsumexp(s, axis=2), rtol=1e-13)


def test_causality_within_the_chunk():
    args, _, _ = _case(2, [20], [12])
    base, _ = extend_attention(**args, sm_scale=0.2)
    j = 5
    args["k_new"] = args["k_new"].copy()
    args["v_new"] = args["v_new"].copy()
    args["k_new"][j] += 1.0
    args["v_new"][j] -= 2.0
    moved, _ = extend_attention(**args, sm_scale=0.2)
    assert np.array_equal(moved[:j], base[:j])
    assert np.all(np.abs(moved[j:] - base[j:]).max(axis=(1, 2)) > 0)


def test_closed_forms():
    # empty prefix, one chunk token: the output is that token's value row
    args, _, _ = _case(3, [0], [1])
    out, lse = extend_attention(**args, sm_scale=0.3)
    G = args["q"].shape[1] // args["k_new"].shape[1]
    assert np.array_equal(out[0], np.repeat(args["v_new"][0], G, axis=0))
    s = 0.3 * np.einsum("hd,hd->h", args["q"][0], np.repeat(args["k_new"][0], G, axis=0))
    assert np.allclose(lse[0], s, rtol=1e-14)
    # zero query: uniform weights over the L0 + i + 1 visible keys
    args, pk, pv = _case(4, [10], [6])
    args["q"] = np.zeros_like(args["q"])
    out, lse = extend_attention(**args, sm_scale=1.0)
    for i in range(6):
        vis = np.concatenate([pv[0], args["v_new"][: i + 1]])     # [n, Hkv, D]
        want = np.repeat(vis.mean(axis=0), out.shape[1] // vis.shape[1], axis=0)
        assert np.allclose(out[i], want, rtol=1e-13, atol=1e-15)
        assert np.allclose(lse[i], np.log(10 + i + 1), rtol=1e-14)


def test_workspace_page_order_is_followed():
    """Moving every sequence's pages elsewhere in the workspace (page_off
    updated) does not change the result."""
    args, _, _ = _case(5, [33, 18], [4, 3], P=16)
    a, _ = extend_attention(**args, sm_scale=0.25)
    n = args["dq_k"].shape[0]
    perm_k = np.zeros((n + 3,) + args["dq_k"].shape[1:], np.uint8)
    perm_v = np.zeros_like(perm_k)
    # sequence 1's pages (offset 0, 2 pages) move to 3.., sequence 0's (offset 2, 3 pages) to 5..
    npg = [3, 2]
    old = args["page_off"]
    new_off = np.array([5, 3])
    for b in range(2):
        perm_k[new_off[b]:new_off[b] + npg[b]] = args["dq_k"][old[b]:old[b] + npg[b]]
        perm_v[new_off[b]:new_off[b] + npg[b]] = args["dq_v"][old[b]:old[b] + npg[b]]
    perm_k[:3] = 0x7E                                                # garbage elsewhere
    b_args = dict(args, dq_k=perm_k, dq_v=perm_v, page_off=new_off)
    b, _ = extend_attention(**b_args, sm_scale=0.25)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("rows", [[0, 3], [5]])
def test_row_selection_matches_full(rows):
    args, _, _ = _case(6, [21, 7], [4, 3])
    full, fl = extend_attention(**args, sm_scale=0.21)
    part, pl = extend_attention(**args, sm_scale=0.21, rows=rows)
    assert np.array_equal(part[rows], full[rows]) and np.array_equal(pl[rows], fl[rows])
    others = np.setdiff1d(np.arange(full.shape[0]), rows)
    assert np.all(np.isnan(part[others]))
