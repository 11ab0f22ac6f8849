"""Pins of the oracle's FP8 codec and scale derivation (CPU only).

Each check ties the oracle to something other than itself: the values the pages
print (tests/golden/fp8_formats.json), torch's float8 dtypes, an exhaustive or
brute-force search, or exact rational arithmetic.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp8_formats.json")))
FMTS = ["e4m3fn", "e4m3fnuz", "e5m2", "e5m2fnuz"]


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ---- values printed on the pages ----------------------------------------------

@pytest.mark.parametrize("fmt", ["e4m3fn", "e4m3fnuz", "e5m2"])
def test_max_matches_pages(fmt):
    assert oracle.fp8_max(fmt) == GOLDEN["max"][fmt]["value"]
    # and the largest finite decoded code is that max
    vals = oracle.decode(fmt, np.arange(256))
    assert np.nanmax(vals[np.isfinite(vals)]) == GOLDEN["max"][fmt]["value"]


@pytest.mark.parametrize("fmt", FMTS)
def test_levels_per_octave(fmt):
    fam = fmt[:4]
    want = GOLDEN["mantissa_levels_per_octave"][fam]["value"]
    vals = oracle.decode(fmt, np.arange(128))
    for lo in (1.0, 2.0, 0.25, 16.0):
        n = np.sum((vals >= lo) & (vals < 2 * lo))
        assert n == want, (fmt, lo, n)


@pytest.mark.parametrize("fmt", ["e4m3fnuz", "e5m2fnuz"])
def test_fnuz_unsigned_zero_and_finite(fmt):
    # no code decodes to -0 and no code decodes to +-inf; a negative tiny value encodes to 0x00
    vals = oracle.decode(fmt, np.arange(256))
    assert not np.any(np.isinf(vals))
    assert not np.any((vals == 0) & np.signbit(vals))
    assert oracle.encode(fmt, [-1e-30, -0.0])[0] == 0 and oracle.encode(fmt, [-0.0])[0] == 0


# ---- library reference: torch's float8 dtypes ---------------------------------

@pytest.mark.parametrize("fmt", FMTS)
def test_decode_all_codes_matches_torch(fmt):
    ours = oracle.decode(fmt, np.arange(256))
    ref = pins.torch_decode_table(fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("fmt", FMTS)
def test_closed_form_limits(fmt):
    import torch
    fi = torch.finfo(pins.TORCH_DTYPES[fmt])
    vals = oracle.decode(fmt, np.arange(128))
    pos = vals[np.isfinite(vals) & (vals > 0)]
    assert pos.max() == fi.max
    assert pos.min() == fi.smallest_normal / 2 ** {"e4m3fn": 3, "e4m3fnuz": 3, "e5m2": 2, "e5m2fnuz": 2}[fmt]
    normals = pos[pos >= fi.smallest_normal]
    assert normals.min() == fi.smallest_normal


# ---- exhaustive round trip ------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
def test_roundtrip_all_codes(fmt):
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(fmt, codes)
    fin = np.isfinite(vals)
    back = oracle.encode(fmt, vals[fin].astype(np.float32))
    assert np.array_equal(back, codes[fin])


@pytest.mark.parametrize("fmt", FMTS)
def test_saturation(fmt):
    m = oracle.fp8_max(fmt)
    codes = oracle.encode(fmt, [m * 1.01, -m * 1.01, m * 1e6, np.inf, -np.inf, m])
    maxcode = oracle.encode(fmt, [m])[0]
    assert list(codes[:2]) == [maxcode, maxcode | 0x80]
    assert codes[2] == maxcode and codes[3] == maxcode and codes[4] == (maxcode | 0x80)


# ---- brute-force nearest-value search ------------------------------------------

def _sweep_values(fmt, rng):
    m = oracle.fp8_max(fmt)
    out = []
    # every bf16 pattern that is finite, at three scales
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    for s in (1.0, 2.0 ** -7, 1.7 / 3.0):
        out.append((f * np.float32(s)).astype(np.float32))
    # midpoints of adjacent fp8 values, +-0..3 fp32 ulps, both signs
    _, vals = pins.positive_grid(fmt)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    near = [mids]
    for k in range(1, 4):
        up, dn = mids.copy(), mids.copy()
        for _ in range(k):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
        near += [up, dn]
    near = np.concatenate(near)
    out += [near, -near, vals.astype(np.float32), -vals.astype(np.float32)]
    # random values spread over the format's range, subnormals included
    e = rng.uniform(np.log2(m) - 30, np.log2(m) + 1, 400000)
    r = (np.exp2(e) * rng.choice([-1.0, 1.0], e.size)).astype(np.float32)
    out.append(r)
    out.append(np.array([0.0, -0.0, 1e-30, -1e-30, 1e-45, -1e-45], np.float32))
    return np.concatenate(out)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_matches_bruteforce_nearest(fmt):
    rng = np.random.default_rng(7)
    y = _sweep_values(fmt, rng)
    ours = oracle.encode(fmt, y)
    ref = pins.nearest_encode(fmt, y)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (fmt, y[bad[:5]], ours[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_matches_torch_in_range(fmt):
    rng = np.random.default_rng(11)
    y = _sweep_values(fmt, rng)
    m = np.float32(oracle.fp8_max(fmt))
    y = y[np.abs(y) <= m]
    ours = oracle.encode(fmt, y)
    ref = pins.torch_encode(fmt, y)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (fmt, y[bad[:5]], ours[bad[:5]], ref[bad[:5]])


# ---- scale derivation -----------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
def test_scale_closed_forms(fmt):
    m = oracle.fp8_max(fmt)
    s64, s, i = oracle.scale_from_amax(fmt, m)
    assert s64 == 1.0 and s == 1.0 and i == 1.0
    for j in range(-20, 21):
        s64, s, i = oracle.scale_from_amax(fmt, 2.0 ** j)
        assert s == np.float32(m * 2.0 ** -j) and i == np.float32(2.0 ** j / m)
    # all-zero group: the eps clamp
    s64, s, i = oracle.scale_from_amax(fmt, 0.0, 1e-12)
    assert s64 == m / 1e-12
    assert s == pins.rn32(Fraction(m) / Fraction(1e-12))
    assert i == pins.rn32(Fraction(1e-12) / Fraction(m))


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_is_correctly_rounded_quotient(fmt):
    # for amax >= eps the fp64-then-fp32 scale equals the exact quotient rounded once
    rng = np.random.default_rng(3)
    m = oracle.fp8_max(fmt)
    bits = rng.integers(0x2C00, 0x7F80, 400).astype(np.uint32)  # positive bf16 above eps
    amaxes = (bits << 16).view(np.float32)
    for a in amaxes:
        s64, s, i = oracle.scale_from_amax(fmt, float(a))
        assert s == pins.rn32(Fraction(m) / Fraction(float(a))), a
        assert s64 == float(Fraction(m) / Fraction(float(a)))  # the IEEE fp64 quotient
        assert i == pins.rn32(1 / Fraction(s64))  # reciprocal of the fp64 scale, rounded once
        assert abs(float(i) * float(s) - 1.0) <= 2.0 ** -23


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_mx_scale_pow2_floor(fmt):
    m = oracle.fp8_max(fmt)
    rng = np.random.default_rng(5)
    for a in np.exp2(rng.uniform(-30, 30, 500)).astype(np.float32):
        e, s, i = oracle.mx_scale_from_amax(fmt, float(a))
        k = 127 - e
        assert s == 2.0 ** k and i == 2.0 ** -k
        # largest power of two with a * 2^k <= fmax
        assert float(a) * 2.0 ** k <= m < float(a) * 2.0 ** (k + 1)
    e, s, i = oracle.mx_scale_from_amax(fmt, m)
    assert e == 127 and s == 1.0


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_mx_scale_ocp_rule(fmt):
    # OCP MX: shared exponent = floor(log2 amax) - floor(log2 fmax)
    emax = {"e4m3fn": 8, "e5m2": 15}[fmt]
    for a in (1.0, 3.0, 448.0, 500.0, 0.001, 65504.0):
        e, s, i = oracle.mx_scale_from_amax(fmt, a, mode=oracle.MX_OCP)
        assert e - 127 == int(np.floor(np.log2(a))) - emax
