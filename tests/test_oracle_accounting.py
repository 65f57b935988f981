"""Pins for oracle/accounting.py against figures the pages print
(tests/golden/llama3_70b_kv_gib.txt, tests/golden/capacity_ratios.txt)."""
import os

import pytest

from oracle import accounting as A

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            yield line.split()


def _kv(name):
    return {r[0]: float(r[1]) for r in _rows(name)}


def test_llama3_70b_fp16_bytes_per_token():
    # 2 (K+V) x 80 layers x 8 KV heads x 128 head_dim x 2 bytes
    assert A.kv_bytes_per_token(80, 8, 128, "fp16") == 327_680
    assert A.kv_bytes_per_token(80, 8, 128, "e4m3") == 163_840
    assert A.kv_bytes_per_token(80, 8, 128, "mx16") == 92_160


def test_llama3_70b_gib_table():
    rows = list(_rows("llama3_70b_kv_gib.txt"))
    assert len(rows) == 9
    for ctx, batch, fp16, fp8, int4 in rows:
        ctx, batch = int(ctx), int(batch)
        for dtype, printed in (("fp16", fp16), ("e4m3", fp8), ("int4", int4)):
            got = A.kv_cache_gib(80, 8, 128, dtype, ctx, batch)
            # printed to one decimal (the page rounds halves up: 1.25 -> 1.3)
            assert abs(got - float(printed)) <= 0.05 + 1e-9, (ctx, batch, dtype, got, printed)


def test_capacity_ratios_printed_on_pages():
    g = _kv("capacity_ratios.txt")
    assert round(A.capacity_ratio("bf16", "mx16"), 2) == g["bf16_over_fp4blk16"]
    assert round(A.capacity_ratio("e4m3", "mx16"), 2) == g["fp8_over_fp4blk16"]
    assert A.capacity_ratio("bf16", "nvfp4") == pytest.approx(16 / 4.5)
    # BF16 -> FP8 doubles the token capacity (vLLM run, Cloudflare Kimi run)
    assert A.capacity_ratio("bf16", "e4m3") == 2.0
    assert g["vllm_fp8_tokens_fp8"] / g["vllm_fp8_tokens_bf16"] == A.capacity_ratio("bf16", "e4m3")
    assert g["kimi_fp8_tokens"] / g["kimi_bf16_tokens"] == pytest.approx(2.0, rel=0.01)


def test_decode_bytes_per_workload():
    # Llama-3-8B shape: 8 KV heads x 128 x (K + V) x 1 byte = 2048 B/token
    assert A.decode_kv_bytes([20480] * 8, 8, 128, "e4m3") == 8 * 20480 * 2048
    # Qwen3 shape FP4 block-16: 4 heads x 128 x 2 x 4.5 bits = 576 B/token
    assert A.decode_kv_bytes([1], 4, 128, "mx16") == 576
    # DeepSeek MLA NVFP4: one 576-element latent row, 4.5 bits = 324 B/token
    assert A.decode_kv_bytes([1], 1, 576, "nvfp4", kind="mla") == 324
