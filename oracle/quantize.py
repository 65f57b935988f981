"""Quantizers for new K/V tokens: FP8 per-tensor / per-head / KIVI-style
(per-channel K, per-token V), FP4 block-16 (E8M0), NVFP4 two-level.

TEST INFRASTRUCTURE (CPU oracle; see ``oracle/formats.py``).

Floating point: every step the method performs in binary32 is done here with
numpy float32 scalars/arrays, whose +,*,/ are IEEE round-to-nearest-even; all
other arithmetic is exact (table lookups, float64 products of short
significands, powers of two).
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1, E4M3, E5M2, Format, decode, encode

E2M1_MAX = 6.0   # SGLang PR #21954 analysis page, review-feedback section
MX_BLOCK = 16    # SGLang Quantized KV Cache page, "Supported formats / FP4"


def fl32(x) -> np.ndarray:
    """Round to binary32 (RNE)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------
# FP8, one scale per tensor.
# SGLang page, "Scaling factors": FP8 needs a scale per tensor (k_scale,
# v_scale), taken from the checkpoint or a file, defaulting to 1.0 when none
# is given. vLLM page, "Scale calibration": scales may be estimated once and
# then kept fixed. Reading adopted: calibrated scale = amax / format maximum,
# computed in binary32; an all-zero tensor gets 1.0 (any scale is exact there).
# --------------------------------------------------------------------------
def fp8_scale(amax: float, fmt: Format) -> np.float32:
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(fmt.max_value))


def fp8_head_scales(x, fmt: Format) -> np.ndarray:
    """Per-attention-head scales (vLLM page, "Supported schemes": one scale per
    KV head, k/v_scale = [num_kv_heads]): fp8_scale of the amax of each head
    h = x[..., h, :] of a [tokens, Hkv, D] tensor."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=(0, 2)) if x.shape[0] else np.zeros(x.shape[1])
    return np.array([fp8_scale(a, fmt) for a in amax], dtype=np.float32)



def fp8_query_scales(q, per_head: bool) -> np.ndarray:
    """Calibrated E4M3 query scales for FP8-domain attention (vLLM page,
    "Supported schemes": q_scale = [num_heads] or [1]; "Scale calibration":
    estimated once from a batch of tokens): fp8_scale(amax / 448) of every
    query head h = q[..., h, :] of a [tokens, Hq, D] tensor, or of the whole
    tensor -> float32 [Hq] or [1]."""
    if per_head:
        return fp8_head_scales(q, E4M3)
    x = np.asarray(q, dtype=np.float64)
    return np.array([fp8_scale(np.abs(x).max() if x.size else 0.0, E4M3)], dtype=np.float32)

# --------------------------------------------------------------------------
# KIVI-style asymmetric scaling ("KV cache quantization mechanism and traps",
# the section on why K and V distributions differ): Key outliers sit in fixed
# channels, so K gets one scale per channel; Value varies from token to
# token, so V gets one scale per token. The page reports KIVI with 2-bit
# integers; reading adopted for this cache: the same FP8 codes as the
# per-tensor path, K scale per (kv head, channel) = fl32(amax over the
# calibration tokens / format max), fixed afterwards; V scale per (token, kv
# head) = fl32(amax of that token's row / format max), computed when the
# token is stored; an all-zero channel or row gets 1.0.
# --------------------------------------------------------------------------
def fp8_channel_scales(x, fmt: Format) -> np.ndarray:
    """[tokens, Hkv, D] -> [Hkv, D]: fp8_scale of the amax of every channel."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=0) if x.shape[0] else np.zeros(x.shape[1:])
    return np.vectorize(lambda a: fp8_scale(a, fmt), otypes=[np.float32])(amax).astype(np.float32)


def quantize_fp8_per_token(x, fmt: Format) -> tuple[np.ndarray, np.ndarray]:
    """Rows [N, D] -> (codes [N, D], scales [N]): each row with its own
    fp8_scale(amax of the row)."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=-1) if x.shape[-1] else np.zeros(x.shape[:-1])
    s = np.array([fp8_scale(a, fmt) for a in amax.reshape(-1)], dtype=np.float32).reshape(amax.shape)
    return quantize_fp8(x, s[..., None], fmt), s


def quantize_fp8(x, scale, fmt: Format) -> np.ndarray:
    """codes = encode(fl32(x / scale)); x holds BF16 values (exact in fp32);
    scale is a binary32 scalar or an array broadcast against x. A finite x
    whose binary32 quotient overflows lies past every format maximum and
    saturates like any other such value (the overflow reading: saturate)."""
    x32 = fl32(x)
    with np.errstate(over="ignore"):
        q = (x32 / np.asarray(scale, dtype=np.float32)).astype(np.float64)
    q = np.where(np.isinf(q) & np.isfinite(x32), np.copysign(fmt.max_value, q), q)
    return encode(q, fmt)


def dequantize_fp8(codes, scale, fmt: Format) -> np.ndarray:
    return decode(codes, fmt) * float(scale)


# --------------------------------------------------------------------------
# FP4 E2M1, blocks of 16 consecutive elements, one 8-bit power-of-two scale
# per block computed from the block itself (SGLang page: "Supported formats /
# FP4" and the FP4 tip under "Scaling factors"; PR #21954 analysis page,
# BlockFP4KVMethod with block_size 16).
# Reading adopted (the pages say only "8-bit exponent scale", framed as OCP
# MXFP4): the OCP microscaling rule, shared exponent = floor(log2(amax_b))
# minus the largest exponent of E2M1 (2), so that the block maximum lands in
# [4, 8) before element rounding; clamped to the E8M0 range [-127, 127];
# amax_b = 0 gives -127. Elements are x * 2**-e rounded to E2M1 (saturating).
# --------------------------------------------------------------------------
def mx_block_exponent(amax_b: np.ndarray) -> np.ndarray:
    """Shared exponent per block, int64. floor(log2 a) taken exactly with frexp."""
    amax_b = np.asarray(amax_b, dtype=np.float64)
    _, ex = np.frexp(amax_b)          # amax = m * 2**ex, m in [0.5, 1)
    e = (ex.astype(np.int64) - 1) - 2
    e = np.where(amax_b == 0, -127, e)
    return np.clip(e, -127, 127)


def quantize_mx16(x) -> tuple[np.ndarray, np.ndarray]:
    """x [..., D] (D % 16 == 0) -> (element codes [..., D] uint8 in 0..15, E8M0 codes [..., D/16])."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    xb = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    amax = np.abs(xb).max(axis=-1)
    e = mx_block_exponent(amax)
    scaled = xb * np.ldexp(1.0, -e)[..., None]        # exact (power of two)
    codes = encode(scaled, E2M1).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def dequantize_mx16(codes, scale_codes) -> np.ndarray:
    codes = np.asarray(codes)
    d = codes.shape[-1]
    vals = decode(codes, E2M1).reshape(codes.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    s = np.ldexp(1.0, np.asarray(scale_codes, dtype=np.int64) - 127)
    return (vals * s[..., None]).reshape(codes.shape)


# --------------------------------------------------------------------------
# NVFP4-style two-level scaling (PR #21954 analysis page, NVFP4KVMethod):
# a binary32 per-tensor global scale and an E4M3 scale per 16-element block,
# E2M1 elements. The page says targets differ on whether E2M1_MAX enters the
# global scale; reading adopted: the stored global scale g is the dequant
# multiplier, g = amax_tensor / (E2M1_MAX * 448), so x^ = e2m1 * e4m3 * g.
# Per block: s = fl32(amax_b / fl32(6 g)) rounded to E4M3 (saturating);
# sd = fl32(dec(s_code) * g); element = E2M1(fl32(x / sd)), or signed zero
# when sd == 0.
# --------------------------------------------------------------------------
def nvfp4_global_scale(amax: float) -> np.float32:
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E2M1_MAX * E4M3.max_value))


def quantize_nvfp4(x, g) -> tuple[np.ndarray, np.ndarray]:
    """x [..., D] -> (E2M1 codes [..., D], E4M3 block-scale codes [..., D/16])."""
    g = np.float32(g)
    x32 = fl32(x)
    d = x32.shape[-1]
    assert d % MX_BLOCK == 0
    xb = x32.reshape(x32.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    amax_b = np.abs(xb).max(axis=-1)
    denom = np.float32(np.float32(E2M1_MAX) * g)
    s = (amax_b / denom).astype(np.float32)
    s_code = encode(s.astype(np.float64), E4M3)
    sd = (decode(s_code, E4M3).astype(np.float32) * g).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (xb / sd[..., None]).astype(np.float32)
    zero = (sd == 0)[..., None] & np.ones_like(xb, dtype=bool)
    q = np.where(zero, np.where(np.signbit(xb), -0.0, 0.0), q)
    codes = encode(q.astype(np.float64), E2M1).reshape(x32.shape)
    return codes, s_code


def dequantize_nvfp4(codes, s_codes, g) -> np.ndarray:
    codes = np.asarray(codes)
    d = codes.shape[-1]
    vals = decode(codes, E2M1).reshape(codes.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    sc = decode(s_codes, E4M3)
    return (vals * sc[..., None] * float(np.float32(g))).reshape(codes.shape)


FP8_FORMATS = {"e4m3": E4M3, "e5m2": E5M2}
