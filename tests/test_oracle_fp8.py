"""Pins for the oracle's fp8 decode tables (CPU only).

The tables are pinned to: a second, independent construction (the ULP ladder);
hand-derived anchor codes stored under tests/golden/ with their citation; the
library cast of torch, a special case that must agree on every code; and a
negative control showing that the pins reject the wrong-bias decoder the pages
warn about ("fp8 KV cache in the in-tree prefill kernel", Architecture / design
notes, the vec_cast paragraph).
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_anchors.txt")


def _anchors():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, code, val = line.split()
            rows.append((fmt, int(code, 16), float(val)))
    return rows


def _same(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e4m3fnuz", "e5m2fnuz"])
def test_two_constructions_agree(fmt):
    a = fp8.table_closed_form(fmt)
    b = fp8.table_ulp_ladder(fmt)
    for c in range(256):
        assert _same(a[c], b[c]), (fmt, hex(c), a[c], b[c])


def test_anchor_codes():
    rows = _anchors()
    assert len(rows) >= 20
    for fmt, code, val in rows:
        got = fp8.fp8_table(fmt)[code]
        assert _same(got, val), (fmt, hex(code), got, val)


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2),
                                     ("e4m3fnuz", torch.float8_e4m3fnuz), ("e5m2fnuz", torch.float8_e5m2fnuz)])
def test_library_cast_agrees(fmt, tdt):
    ref = torch.arange(256, dtype=torch.uint8).view(tdt).to(torch.float64).numpy()
    t = fp8.fp8_table(fmt)
    for c in range(256):
        assert _same(t[c], ref[c]), (fmt, hex(c), t[c], ref[c])


def test_wrong_bias_is_caught():
    """Negative control: the fnuz bias (8) applied to OCP e4m3 data gives
    0x38 = 0.5, which the anchors must reject."""
    wrong = fp8.table_closed_form("e4m3", bias=8)
    assert wrong[0x38] == 0.5
    bad = [c for f, c, v in _anchors() if f == "e4m3" and not _same(wrong[c], v)]
    assert bad, "the anchors did not notice a wrong exponent bias"


def test_denormals_present_and_ordered():
    for fmt, nsub in (("e4m3", 7), ("e5m2", 3)):
        t = fp8.fp8_table(fmt)
        sub = t[1:1 + nsub]
        assert np.all(sub > 0) and np.all(np.diff(sub) > 0)
        # equally spaced by the smallest subnormal
        assert np.allclose(np.diff(np.concatenate([[0.0], sub])), sub[0], rtol=0, atol=0)
        pos = t[:0x7F] if fmt == "e4m3" else t[:0x7C]
        assert np.all(np.diff(pos) > 0)  # magnitudes increase with the code


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e4m3fnuz", "e5m2fnuz"])
def test_every_finite_code_is_exact_in_2byte_types(fmt):
    """Every finite fp8 value is exactly an fp16 and a bf16 value, so a kernel
    may widen the raw code into q's 2-byte type with no rounding."""
    t = fp8.fp8_table(fmt)
    fin = t[np.isfinite(t)]
    assert np.array_equal(fin.astype(np.float16).astype(np.float64), fin)
    bf = torch.from_numpy(fin).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf, fin)


def test_max_finite():
    assert fp8.max_finite("e4m3") == 448.0
    assert fp8.max_finite("e5m2") == 57344.0
    assert fp8.max_finite("e4m3fnuz") == 240.0
    assert fp8.max_finite("e5m2fnuz") == 57344.0


def test_fnuz_with_the_ocp_bias_is_caught():
    """Negative control for the fnuz tables: the page's latent vec_cast bug
    decodes fnuz with the OCP bias (2x too large); the anchors must reject it."""
    for fmt, ocp_bias in (("e4m3fnuz", 7), ("e5m2fnuz", 15)):
        wrong = fp8.table_closed_form(fmt, bias=ocp_bias)
        bad = [c for f, c, v in _anchors() if f == fmt and not _same(wrong[c], v)]
        assert bad, fmt


def test_fnuz_specials():
    for fmt in ("e4m3fnuz", "e5m2fnuz"):
        t = fp8.fp8_table(fmt)
        assert np.isnan(t[0x80]) and np.sum(np.isnan(t)) == 1 and np.all(np.isfinite(t[~np.isnan(t)]))
        assert not np.any(np.signbit(t[np.isfinite(t) & (t == 0)]))  # no negative zero


def test_fnuz_codes_read_as_ocp():
    """The format identities the decode kernel's fnuz widening rests on,
    checked on all 256 codes of the oracle's tables.  e4m3fnuz (bias 8) read
    as OCP e4m3 (bias 7) is exactly twice its value, except 0x7F / 0xFF (+-240,
    an OCP NaN) and 0x80 (the fnuz NaN, OCP -0).  e5m2fnuz (bias 16) with its
    exponent lowered by one, read as OCP e5m2 (bias 15), is its exact value
    for every code with exponent >= 2 -- the top binade included -- while
    exponents 0 and 1 fall outside that reading."""
    e4_ocp, e4_fnuz = fp8.fp8_table("e4m3"), fp8.fp8_table("e4m3fnuz")
    for c in range(256):
        if c in (0x7F, 0xFF):
            assert math.isnan(e4_ocp[c]) and abs(e4_fnuz[c]) == 240.0
        elif c == 0x80:
            assert math.isnan(e4_fnuz[c]) and e4_ocp[c] == 0.0 and math.copysign(1, e4_ocp[c]) < 0
        else:
            assert e4_ocp[c] == 2.0 * e4_fnuz[c], hex(c)
    e5_ocp, e5_fnuz = fp8.fp8_table("e5m2"), fp8.fp8_table("e5m2fnuz")
    for c in range(256):
        e = (c >> 2) & 0x1F
        if c == 0x80:
            continue
        if e >= 2:
            assert e5_ocp[c - 4] == e5_fnuz[c], hex(c)
        elif c & 0x7F:
            # exponents 0 and 1: twice the value, not representable one binade lower
            assert e5_ocp[c] == 2.0 * e5_fnuz[c], hex(c)
    assert np.isinf(e5_ocp[0x7C]) and e5_fnuz[0x7C] == 32768.0  # the top binade is finite in fnuz
