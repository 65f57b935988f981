"""Exact value tables and round-to-nearest-even encoders for the KV code formats.

TEST INFRASTRUCTURE. This package is the CPU oracle: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it. It shares no code with the HIP library.

Sources (the pages):
  * SGLang "Quantized KV Cache" page, section "Supported formats / FP8":
    the two 8-bit float formats E5M2 (5 exponent, 2 mantissa bits, range to
    57344) and E4M3 (4 exponent, 3 mantissa bits). The same section prints
    +-240 for E4M3, which is the maximum of the FNUZ variant (exponent bias 8);
    the page's own scale-file example names ``float8_e4m3fn`` (OCP "FN",
    bias 7, maximum 448). We use E4M3FN; ``e4m3fnuz_max()`` below reproduces
    the 240 figure so the reading is pinned by a test.
  * Same page, section "Supported formats / FP4": E2M1 elements (1 sign,
    2 exponent, 1 mantissa bit) whose blocks share one 8-bit exponent scale.
  * SGLang PR #21954 analysis page, review-feedback section: the E2M1
    maximum 6.0 (``E2M1_MAX``).

Every table is built from the bit-field definition of the format (sign,
biased exponent, mantissa, subnormals at exponent field 0). Encoding is a
search over the sorted table of finite magnitudes: nearest value, ties to the
code whose least significant bit is 0, magnitudes at or above the largest
finite value saturate to it, and the sign bit is kept (so -0.0 encodes to the
negative-zero code). The pages do not state a rounding or overflow rule; this
is the reading adopted (IEEE default rounding, saturation because E4M3FN and
E2M1 have no infinity).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Format:
    name: str
    bits: int            # 8 or 4
    values: np.ndarray   # float64 value of every code (NaN for NaN codes)
    max_code: int        # positive code of the largest finite magnitude
    sign_bit: int        # mask of the sign bit in a code

    @property
    def max_value(self) -> float:
        return float(self.values[self.max_code])


def _minifloat_value(code: int, ebits: int, mbits: int, bias: int,
                     special: str) -> float:
    """Value of a sign/exponent/mantissa code.

    ``special``: "ieee" = all-ones exponent holds Inf (mantissa 0) and NaN;
    "fn" = only the all-ones exponent with all-ones mantissa is NaN (E4M3FN);
    "fnuz" = only the negative-zero pattern is NaN; "none" = no specials.
    """
    sign = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    emax_field = (1 << ebits) - 1
    if special == "ieee" and e == emax_field:
        v = math.inf if m == 0 else math.nan
    elif special == "fn" and e == emax_field and m == (1 << mbits) - 1:
        v = math.nan
    elif special == "fnuz" and sign == 1 and e == 0 and m == 0:
        return math.nan
    elif e == 0:
        v = (m / (1 << mbits)) * 2.0 ** (1 - bias)
    else:
        v = (1.0 + m / (1 << mbits)) * 2.0 ** (e - bias)
    return -v if sign else v


def _make(name, bits, ebits, mbits, bias, special) -> Format:
    vals = np.array([_minifloat_value(c, ebits, mbits, bias, special)
                     for c in range(1 << bits)], dtype=np.float64)
    half = 1 << (bits - 1)
    pos = vals[:half]
    finite = np.isfinite(pos)
    max_code = int(np.nonzero(finite)[0].max())
    return Format(name, bits, vals, max_code, half)


E4M3 = _make("e4m3fn", 8, 4, 3, 7, "fn")
E5M2 = _make("e5m2", 8, 5, 2, 15, "ieee")
E2M1 = _make("e2m1", 4, 2, 1, 1, "none")

FORMATS = {"e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1}


def e4m3fnuz_max() -> float:
    """Largest finite E4M3 value when the exponent bias is 8 (FNUZ variant)."""
    vals = [_minifloat_value(c, 4, 3, 8, "fnuz") for c in range(128)]
    return max(v for v in vals if math.isfinite(v))


def e8m0_value(code) -> np.ndarray:
    """Power-of-two scale 2**(code-127); code 255 is NaN (OCP E8M0)."""
    code = np.asarray(code, dtype=np.int64)
    out = np.ldexp(1.0, code - 127).astype(np.float64)
    return np.where(code == 255, np.nan, out)


def decode(codes, fmt: Format) -> np.ndarray:
    """Code -> exact float64 value (table lookup)."""
    codes = np.asarray(codes, dtype=np.int64)
    return fmt.values[codes]


def encode(x, fmt: Format) -> np.ndarray:
    """float64 values -> codes (uint8), nearest value, ties to even code, saturating.

    Inputs must be finite; a non-finite input raises ValueError (the store
    contract takes finite BF16 tensors).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("encode: non-finite input")
    mags = fmt.values[: fmt.max_code + 1]          # ascending for these formats
    assert np.all(np.diff(mags) > 0)
    a = np.abs(x)
    hi = np.searchsorted(mags, a, side="left")      # mags[hi-1] < a <= mags[hi]
    hi_c = np.minimum(hi, fmt.max_code)
    lo_c = np.maximum(hi - 1, 0)
    d_hi = mags[hi_c] - a
    d_lo = a - mags[lo_c]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    code = np.where(pick_hi, hi_c, lo_c)
    code = np.where(a >= fmt.max_value, fmt.max_code, code)
    code = np.where(a == 0.0, 0, code)
    code = code | np.where(np.signbit(x), fmt.sign_bit, 0)
    return code.astype(np.uint8)
