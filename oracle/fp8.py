"""Exact 256-entry decode tables for the OCP 8-bit float formats and their
fnuz variants.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import this package; only the tests, the smoke check and the
benchmark's CPU-baseline leg do.

Source.  "fp8 KV cache in the in-tree prefill kernel" (AMD-Ecosystem/flashinfer
PR #368), Architecture / design notes, the paragraph on the OCP spellings: the
E4M3 exponent bias is 7 and the E5M2 bias is 15 (the gfx942 "fnuz" variants are
one greater, 8 and 16).  The same page, Architecture / design notes, paragraph
"Dequant goes through ...", records the bug these tables exist to catch: a
decoder that uses the wrong bias (2x error) or mishandles denormals.

The pages give only the biases.  The remaining facts are those of the OCP 8-bit
floating point specification, which the pages name but do not restate:
  * e4m3 ("e4m3fn"): 1 sign, 4 exponent, 3 mantissa bits; no infinities; the
    only NaN encodings are S.1111.111 (0x7F, 0xFF); max finite 448.
  * e5m2: 1 sign, 5 exponent, 2 mantissa bits; IEEE-754-like; exponent 11111
    with mantissa 0 is +-inf, with mantissa != 0 NaN; max finite 57344.
Both have signed zero and subnormals (exponent field 0).

The gfx942 "fnuz" variants (same page: a KV cache may also be fnuz fp8 there;
biases 8 and 16) follow the fnuz convention, which the pages also leave to
the format's definition: no infinities, no negative zero, and the single NaN
encoding 0x80 (sign bit alone); every other code decodes with the formula
below, so e4m3fnuz reaches 240 at 0x7F and e5m2fnuz 57344 at 0x7F.

Two constructions that share nothing but the format parameters:
  * ``table_closed_form``: decodes each code's bit fields with the textbook
    formula (-1)^s * 2^(e-bias) * (1 + m/2^M), subnormal 2^(1-bias) * m/2^M.
  * ``table_ulp_ladder``: walks the non-negative codes in order and adds the
    spacing between neighbours (one unit in the last place, which doubles at
    every binade above the first normal one), in exact rationals.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# name -> (exponent bits, mantissa bits, exponent bias)
FORMATS = {
    "e4m3": (4, 3, 7),
    "e5m2": (5, 2, 15),
    "e4m3fnuz": (4, 3, 8),
    "e5m2fnuz": (5, 2, 16),
}


def _is_special(fmt: str, code: int) -> str | None:
    """Return 'nan', '+inf', '-inf' or None for a code of ``fmt``."""
    ebits, mbits, _ = FORMATS[fmt]
    sign = code >> 7
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    emax_field = (1 << ebits) - 1
    if fmt.endswith("fnuz"):
        # fnuz: no infinities and no negative zero; the one NaN is 0x80
        return "nan" if code == 0x80 else None
    if fmt == "e4m3":
        # OCP E4M3: only the all-ones exponent *and* all-ones mantissa is NaN.
        if e == emax_field and m == (1 << mbits) - 1:
            return "nan"
        return None
    # e5m2: IEEE-style specials on the all-ones exponent.
    if e == emax_field:
        if m == 0:
            return "-inf" if sign else "+inf"
        return "nan"
    return None


def table_closed_form(fmt: str, bias: int | None = None) -> np.ndarray:
    """Decode all 256 codes from their bit fields.  ``bias`` may be overridden
    only to build the negative control (the wrong-bias decoder)."""
    ebits, mbits, fbias = FORMATS[fmt]
    if bias is None:
        bias = fbias
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sp = _is_special(fmt, code)
        if sp == "nan":
            out[code] = np.nan
            continue
        if sp == "+inf":
            out[code] = np.inf
            continue
        if sp == "-inf":
            out[code] = -np.inf
            continue
        s = code >> 7
        e = (code >> mbits) & ((1 << ebits) - 1)
        m = code & ((1 << mbits) - 1)
        if e == 0:
            mag = 2.0 ** (1 - bias) * (m / 2.0 ** mbits)
        else:
            mag = 2.0 ** (e - bias) * (1.0 + m / 2.0 ** mbits)
        out[code] = -mag if s else mag
    return out


def table_ulp_ladder(fmt: str) -> np.ndarray:
    """Second construction: magnitudes by accumulating the spacing between
    consecutive codes.  The first 2^(M+1) codes (subnormals and the first normal
    binade) are spaced by the smallest subnormal 2^(1-bias-M); every later
    binade of 2^M codes doubles the spacing.  Specials are placed by the format
    rules, and the sign bit mirrors the magnitude."""
    ebits, mbits, bias = FORMATS[fmt]
    step0 = Fraction(1, 2 ** (bias - 1 + mbits))  # 2^(1-bias-M)
    mags = []
    v = Fraction(0)
    for k in range(128):
        mags.append(v)
        # binade of code k: 0 = subnormals, 1 = first normal binade, ...  The
        # gap from code k to code k+1 is the spacing inside k's binade:
        # step0 for binades 0 and 1, doubling for each binade after that.
        binade = k // (1 << mbits)
        v = v + step0 * (2 ** max(0, binade - 1))
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sp = _is_special(fmt, code)
        if sp == "nan":
            out[code] = np.nan
        elif sp == "+inf":
            out[code] = np.inf
        elif sp == "-inf":
            out[code] = -np.inf
        else:
            mag = float(mags[code & 0x7F])
            out[code] = -mag if code & 0x80 else mag
    return out


_TABLES: dict[str, np.ndarray] = {}


def fp8_table(fmt: str) -> np.ndarray:
    """The decode table used by the oracle (the closed form; tests require the
    ladder construction to agree on every code)."""
    if fmt not in _TABLES:
        t = table_closed_form(fmt)
        t.setflags(write=False)
        _TABLES[fmt] = t
    return _TABLES[fmt]


def max_finite(fmt: str) -> float:
    t = fp8_table(fmt)
    return float(np.nanmax(t[np.isfinite(t)]))
