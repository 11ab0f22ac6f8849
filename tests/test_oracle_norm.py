"""Pins of the oracle's normalization (RMSNorm / LayerNorm stored as bf16) that
feeds the fused norm + rowwise quantization (CPU only). Each pin is a property the
definition fixes: exact invariances, closed forms on special rows, the moments of
the output, and an independent fp64 evaluation within the bf16 rounding."""
import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)
    synth.build(force=False)


def _f(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def _scale_bits(x, k):
    """bf16 bits of x * 2^k (exact: exponent field shift, no overflow here)."""
    e = ((x >> 7) & 0xFF).astype(np.int32)
    assert np.all((e == 0) | ((e + k > 0) & (e + k < 255)))
    out = x.copy()
    nz = e != 0
    out[nz] = ((x[nz] & 0x807F) | (((e[nz] + k) & 0xFF) << 7)).astype(np.uint16)
    return out


@pytest.mark.parametrize("layer", [False, True])
def test_power_of_two_scaling_is_exact(layer):
    """With norm_eps = 0 every step scales exactly: norm(2^k x) == norm(x) bit for bit
    (a misplaced mean, square or root breaks it)."""
    x = synth.normal_bf16((6, 96), 21, 1.0)
    g = synth.normal_bf16((1, 96), 22, 0.5).reshape(96)
    b = synth.normal_bf16((1, 96), 23, 0.5).reshape(96)
    y0 = oracle.norm_row(x, g, b if layer else None, layer, 0.0)
    for k in (-5, 3, 9):
        assert np.array_equal(oracle.norm_row(_scale_bits(x, k), g, b if layer else None, layer, 0.0), y0), k


def test_layernorm_of_constant_row_is_beta():
    x = np.full((3, 64), 0x4040, np.uint16)  # 3.0
    g = synth.normal_bf16((1, 64), 24, 1.0).reshape(64)
    b = synth.normal_bf16((1, 64), 25, 1.0).reshape(64)
    y = oracle.norm_row(x, g, b, True, 1e-5)
    assert np.array_equal(y, np.broadcast_to(b, (3, 64)))


def test_output_moments():
    """gamma = 1: RMSNorm rows have mean square 1, LayerNorm rows mean 0 and
    variance 1 (up to norm_eps and the bf16 storage)."""
    x = synth.normal_bf16((8, 1024), 26, 3.0)
    one = np.full(1024, 0x3F80, np.uint16)
    yr = _f(oracle.norm_row(x, one, None, False, 1e-6))
    assert np.allclose((yr ** 2).mean(1), 1.0, rtol=4e-3)
    yl = _f(oracle.norm_row(x, one, np.zeros(1024, np.uint16), True, 1e-6))
    assert np.allclose(yl.mean(1), 0.0, atol=4e-3)
    assert np.allclose(yl.var(1), 1.0, rtol=4e-3)


@pytest.mark.parametrize("layer", [False, True])
def test_matches_fp64_evaluation(layer):
    """An independent fp64 evaluation of the textbook formula: every stored value is
    within one bf16 rounding (plus the fp32 steps) of it."""
    rm = synth.log_uniform_row_mult(5, 27, -6, 6)
    x = synth.normal_bf16((5, 200), 28, 1.0, row_mult=rm)
    g = synth.normal_bf16((1, 200), 29, 1.0).reshape(200)
    b = synth.normal_bf16((1, 200), 30, 1.0).reshape(200)
    eps = 1e-5
    xf, gf, bf = _f(x), _f(g), _f(b)
    if layer:
        mu = xf.mean(1, keepdims=True)
        ref = (xf - mu) / np.sqrt(xf.var(1, keepdims=True) + eps) * gf + bf
    else:
        ref = xf / np.sqrt((xf ** 2).mean(1, keepdims=True) + eps) * gf
    y = _f(oracle.norm_row(x, g, b if layer else None, layer, eps))
    assert np.all(np.abs(y - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6)


def test_quantization_is_quant_row_of_the_stored_norm():
    x = synth.normal_bf16((4, 256), 31, 1.0)
    g = synth.normal_bf16((1, 256), 32, 1.0).reshape(256)
    y, q, s, i = oracle.norm_quant_row(x, g, None, False, 1e-6, "e4m3fn")
    rq, rs, ri = oracle.quant_row(y, "e4m3fn")
    assert np.array_equal(q, rq) and np.array_equal(s, rs) and np.array_equal(i, ri)


# ---- the row statistics: exact sums rounded once to fp64 ------------------------------

from fractions import Fraction  # noqa: E402


def _exact(bits):
    """Exact value of each bf16 bit pattern as a Fraction (bf16 -> fp32 -> fp64 is exact)."""
    return [Fraction(float(v)) for v in oracle.bf16_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)]


def _exact_sums(row):
    xs = _exact(row)
    return float(sum(xs, Fraction(0))), float(sum((v * v for v in xs), Fraction(0)))


def _bits(values):
    """bf16 bit patterns of values that are exactly bf16 (checked)."""
    f = np.asarray(values, np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f32(b), f), "not a bf16 value"
    return b


def _wide_rows(rows, cols, seed):
    """bf16 patterns with uniformly random sign, exponent field 0..254 (subnormals and
    values up to 2^127) and mantissa: sums that no fixed-width accumulator holds."""
    rng = np.random.default_rng(seed)
    e = rng.integers(0, 255, (rows, cols))
    return ((rng.integers(0, 2, (rows, cols)) << 15) | (e << 7) | rng.integers(0, 128, (rows, cols))).astype(np.uint16)


@pytest.mark.parametrize("kind", ["normal", "spread", "wide", "narrow_wide"])
def test_stats_are_the_exact_sums_rounded_once(kind):
    """s1 and s2 equal the Fraction sums of the exact bf16 values, rounded by Python's
    correctly rounded int/int division: on N(0,1) rows, rows spread over 2^-8..2^8,
    and rows whose terms span the whole bf16 range (2^-133 .. 2^127)."""
    if kind == "normal":
        x = synth.normal_bf16((6, 4096), 41, 1.0)
    elif kind == "spread":
        x = synth.normal_bf16((6, 512), 42, 1.0, row_mult=synth.log_uniform_row_mult(6, 43, -8, 8))
    elif kind == "wide":
        x = _wide_rows(6, 300, 44)
    else:
        x = _wide_rows(20, 5, 45)
    s1, s2 = oracle.norm_stats(x)
    for r in range(x.shape[0]):
        e1, e2 = _exact_sums(x[r])
        assert s1[r] == e1 and s2[r] == e2, (kind, r, s1[r], e1, s2[r], e2)


def _alternatives(row):
    """The row sums under accumulations the definition rules out: fp32 and fp64 in
    column order, x87 long double in column order, and fp64 pairwise."""
    v = oracle.bf16_to_f32(row).astype(np.float64)
    out = {}
    out["fp32"] = (float(np.cumsum(v.astype(np.float32), dtype=np.float32)[-1]),
                   float(np.cumsum((v * v).astype(np.float32), dtype=np.float32)[-1]))
    out["fp64"] = (float(np.cumsum(v)[-1]), float(np.cumsum(v * v)[-1]))
    ld = v.astype(np.longdouble)
    out["long double"] = (float(np.cumsum(ld)[-1]), float(np.cumsum(ld * ld)[-1]))

    def pairwise(a):
        while len(a) > 1:
            if len(a) % 2:
                a = np.append(a, 0.0)
            a = a[0::2] + a[1::2]
        return float(a[0])
    out["pairwise"] = (pairwise(v.copy()), pairwise(v * v))
    return out


def test_crafted_rows_separate_the_exact_sums_from_any_fixed_accumulation():
    """Row A: squares 2^80 + 2^26 + 2^26 + 2^-40 -- the exact sum lies just above the
    tie 2^80 + 2^27 and rounds up to 2^80 + 2^28; every rounded accumulation (fp32, fp64,
    x87 long double, pairwise) loses 2^-40 and rounds the tie to even, 2^80.
    Row B: 2^60 + 2^-20 - 2^60 = 2^-20 exactly; the others cancel to 0."""
    a = _bits([2.0 ** 40, 2.0 ** 13, 2.0 ** 13, 2.0 ** -20] + [0.0] * 4)
    b = _bits([2.0 ** 60, 2.0 ** -20, -(2.0 ** 60)] + [0.0] * 5)
    s1, s2 = oracle.norm_stats(np.stack([a, b]))
    assert s2[0] == 2.0 ** 80 + 2.0 ** 28 and s1[1] == 2.0 ** -20
    assert (s1[0], s2[0]) == _exact_sums(a) and (s1[1], s2[1]) == _exact_sums(b)
    for name, (t1, t2) in _alternatives(a).items():
        assert t2 == 2.0 ** 80, name
    for name, (t1, t2) in _alternatives(b).items():
        assert t1 == 0.0, name


def test_layernorm_output_sees_the_exact_mean():
    """LayerNorm of row B with gamma 1, beta 0: the mean is 2^-20 / 8 = 2^-23, not 0, so
    the zeros of the row normalize to -2^-23 * rstd32 (nonzero), and the whole stored
    row equals the definition's fp32 steps on the exact statistics."""
    row = _bits([2.0 ** 60, 2.0 ** -20, -(2.0 ** 60)] + [0.0] * 5)
    one = np.full(8, 0x3F80, np.uint16)
    zero = np.zeros(8, np.uint16)
    y = oracle.norm_row(row[None, :], one, zero, True, 0.0)[0]
    e1, e2 = _exact_sums(row)
    n = 8.0
    mean = e1 / n
    var = e2 / n - mean * mean
    rstd = 1.0 / np.sqrt(var)
    m32, r32 = np.float32(mean), np.float32(rstd)
    xf = oracle.bf16_to_f32(row)
    t = ((xf - m32) * r32) * np.float32(1.0) + np.float32(0.0)
    want = _bits_rne(t)
    assert m32 == np.float32(2.0 ** -23)
    assert np.array_equal(y, want)
    assert np.all(oracle.bf16_to_f32(y[3:]) != 0.0)


def _bits_rne(t):
    """fp32 -> bf16 bit patterns, nearest, ties to even (numpy, finite values)."""
    u = np.asarray(t, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("layer", [False, True])
def test_norm_rows_follow_the_exact_statistics(layer):
    """Whole rows (including a wide-range one) against the definition evaluated on the
    Fraction statistics: mean, E[x^2], var and rstd by correctly rounded fp64 operations,
    then the fp32 steps and bf16 rounding."""
    x = np.concatenate([synth.normal_bf16((3, 256), 46, 1.0),
                        _bits(np.concatenate([[2.0 ** 40, 2.0 ** 13, 2.0 ** 13, 2.0 ** -20],
                                              np.zeros(252)]))[None, :]])
    g = synth.normal_bf16((1, 256), 47, 1.0).reshape(256)
    b = synth.normal_bf16((1, 256), 48, 1.0).reshape(256)
    eps = 1e-5
    y = oracle.norm_row(x, g, b if layer else None, layer, eps)
    gf, bf = oracle.bf16_to_f32(g), oracle.bf16_to_f32(b)
    for r in range(x.shape[0]):
        e1, e2 = _exact_sums(x[r])
        n = float(x.shape[1])
        mean, ms = e1 / n, e2 / n
        var = ms - mean * mean if layer else ms
        rstd = 1.0 / np.sqrt(var + eps)
        xf = oracle.bf16_to_f32(x[r])
        if layer:
            t = (((xf - np.float32(mean)) * np.float32(rstd)) * gf) + bf
        else:
            t = (xf * np.float32(rstd)) * gf
        assert np.array_equal(y[r], _bits_rne(t)), r
