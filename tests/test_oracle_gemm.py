"""Pins of the oracle's fp64 GEMMs (CPU only).

References: exact integer arithmetic on the fp8 grid, numpy's float64 matmul,
and the reductions between the dense, grouped, blockwise and MX forms.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _codes(fmt, shape, rng):
    """Random finite codes of a format (no NaN / inf patterns)."""
    tab = pins.torch_decode_table(fmt)
    ok = np.nonzero(np.isfinite(tab))[0]
    return rng.choice(ok, size=shape).astype(np.uint8)


def _dec(fmt, q):
    return pins.torch_decode_table(fmt)[q]


@pytest.mark.parametrize("fa,fb", [("e4m3fn", "e4m3fn"), ("e5m2", "e4m3fn"), ("e4m3fnuz", "e4m3fnuz")])
def test_dense_exact_integer(fa, fb):
    rng = np.random.default_rng(1)
    M, N, K = 5, 6, 48
    a, b = _codes(fa, (M, K), rng), _codes(fb, (N, K), rng)
    sa = rng.uniform(0.5, 2, M).astype(np.float32)
    sb = rng.uniform(0.5, 2, N).astype(np.float32)
    out = oracle.scaled_mm(a, fa, b, fb, oracle.SCALE_ROW, sa, sb)
    da, db = _dec(fa, a), _dec(fb, b)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(da[m, k])) * Fraction(float(db[n, k])) for k in range(K))
            want = exact * Fraction(float(sa[m])) * Fraction(float(sb[n]))
            got = Fraction(out[m, n])
            assert abs(got - want) <= abs(want) * Fraction(1, 2 ** 51) + Fraction(1, 2 ** 1000)


def test_dense_matches_numpy_matmul():
    rng = np.random.default_rng(2)
    M, N, K = 33, 40, 256
    a, b = _codes("e4m3fn", (M, K), rng), _codes("e4m3fn", (N, K), rng)
    sa = rng.uniform(0.01, 3, M).astype(np.float32)
    sb = rng.uniform(0.01, 3, N).astype(np.float32)
    out = oracle.scaled_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_ROW, sa, sb)
    ref = (_dec("e4m3fn", a) @ _dec("e4m3fn", b).T) * sa[:, None].astype(np.float64) * sb[None, :]
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-300)
    # tensorwise: a single scale each
    out_t = oracle.scaled_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_TENSOR, sa[:1], sb[:1])
    ref_t = (_dec("e4m3fn", a) @ _dec("e4m3fn", b).T) * float(sa[0]) * float(sb[0])
    np.testing.assert_allclose(out_t, ref_t, rtol=1e-13)


def test_scale_direction_negative():
    # passing the quantize multipliers instead of their inverses is off by (s_a * s_b)^2
    rng = np.random.default_rng(3)
    a, b = _codes("e4m3fn", (4, 64), rng), _codes("e4m3fn", (5, 64), rng)
    s_a, s_b = np.float32(8.0), np.float32(0.25)
    good = oracle.scaled_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_TENSOR, [1 / s_a], [1 / s_b])
    bad = oracle.scaled_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_TENSOR, [s_a], [s_b])
    nz = good != 0
    np.testing.assert_allclose(bad[nz] / good[nz], (float(s_a) * float(s_b)) ** 2, rtol=1e-12)


def _offsets(counts):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return off


def test_grouped_reduces_to_dense():
    rng = np.random.default_rng(4)
    K, N = 128, 24
    counts = [7, 0, 13, 1, 0, 9]
    E = len(counts)
    off = _offsets(counts)
    Mtot = int(off[-1])
    a, b = _codes("e4m3fn", (Mtot, K), rng), _codes("e4m3fn", (E, N, K), rng)
    sa = rng.uniform(0.5, 2, Mtot).astype(np.float32)
    sb = rng.uniform(0.5, 2, (E, N)).astype(np.float32)
    out = oracle.grouped_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_ROW, sa, sb, off)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ref = oracle.scaled_mm(a[lo:hi], "e4m3fn", b[e], "e4m3fn", oracle.SCALE_ROW, sa[lo:hi], sb[e])
        assert np.array_equal(out[lo:hi], ref)
    # E = 1 grouped == dense
    out1 = oracle.grouped_mm(a, "e4m3fn", b[:1], "e4m3fn", oracle.SCALE_ROW, sa, sb[:1], np.array([0, Mtot], np.int32))
    assert np.array_equal(out1, oracle.scaled_mm(a, "e4m3fn", b[0], "e4m3fn", oracle.SCALE_ROW, sa, sb[0]))
    # sampled positions agree with the full product
    rows = rng.integers(0, Mtot, 50)
    cols = rng.integers(0, N, 50)
    smp = oracle.grouped_mm_sample(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_ROW, sa, sb, off, rows, cols)
    assert np.array_equal(smp, out[rows, cols])


def test_block_and_mx_reduce_to_uniform_scaling():
    rng = np.random.default_rng(5)
    E, N, K = 2, 256, 512
    off = _offsets([70, 58])
    Mtot = int(off[-1])
    a, b = _codes("e4m3fn", (Mtot, K), rng), _codes("e4m3fn", (E, N, K), rng)
    c_a, c_b = np.float32(0.375), np.float32(3.0)
    ref = oracle.grouped_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_ROW,
                            np.full(Mtot, c_a, np.float32), np.full((E, N), c_b, np.float32), off)
    blk = oracle.grouped_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_BLOCK128,
                            np.full((Mtot, K // 128), c_a, np.float32),
                            np.full((E, N // 128, K // 128), c_b, np.float32), off)
    np.testing.assert_allclose(blk, ref, rtol=1e-14, atol=1e-300)
    unscaled = oracle.grouped_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_ROW,
                                 np.ones(Mtot, np.float32), np.ones((E, N), np.float32), off)
    mx1 = oracle.grouped_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_MX32,
                            np.full((Mtot, K // 32), 127, np.uint8), np.full((E, N, K // 32), 127, np.uint8), off)
    np.testing.assert_allclose(mx1, unscaled, rtol=1e-14, atol=1e-300)
    # opposite exponents cancel
    ka = rng.integers(-6, 7, (Mtot, K // 32))
    mxa = (127 + ka).astype(np.uint8)
    # b's scales can only depend on (n, group); make a's exponent constant per group column
    ka_col = ka[0]
    mxa = np.broadcast_to((127 + ka_col).astype(np.uint8), (Mtot, K // 32)).copy()
    mxb = np.broadcast_to((127 - ka_col).astype(np.uint8), (E, N, K // 32)).copy()
    mx2 = oracle.grouped_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_MX32, mxa, mxb, off)
    np.testing.assert_allclose(mx2, unscaled, rtol=1e-14, atol=1e-300)
    # a non-uniform MX scale matches numpy on the dequantized operands
    sa = rng.integers(120, 134, (Mtot, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 134, (E, N, K // 32)).astype(np.uint8)
    mx3 = oracle.grouped_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_MX32, sa, sb, off)
    da = _dec("e4m3fn", a) * np.exp2(np.repeat(sa.astype(np.int64) - 127, 32, axis=1))
    for e in range(E):
        db = _dec("e4m3fn", b[e]) * np.exp2(np.repeat(sb[e].astype(np.int64) - 127, 32, axis=1))
        ref = da[off[e]:off[e + 1]] @ db.T
        np.testing.assert_allclose(mx3[off[e]:off[e + 1]], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # a non-uniform block scale matches numpy on the dequantized operands
    ia = rng.uniform(0.1, 4, (Mtot, K // 128)).astype(np.float32)
    ib = rng.uniform(0.1, 4, (E, N // 128, K // 128)).astype(np.float32)
    bl = oracle.grouped_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_BLOCK128, ia, ib, off)
    da = _dec("e4m3fn", a) * np.repeat(ia.astype(np.float64), 128, axis=1)
    for e in range(E):
        db = _dec("e4m3fn", b[e]) * np.repeat(np.repeat(ib[e].astype(np.float64), 128, axis=0), 128, axis=1)
        ref = da[off[e]:off[e + 1]] @ db.T
        np.testing.assert_allclose(bl[off[e]:off[e + 1]], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_wgrad_matches_numpy():
    rng = np.random.default_rng(6)
    M, N, K = 64, 24, 40
    g = (rng.standard_normal((M, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out = oracle.wgrad_bf16(g, x)
    gf = oracle.bf16_to_f32(g).astype(np.float64)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    np.testing.assert_allclose(out, gf.T @ xf, rtol=1e-12, atol=1e-12)
    ns, ks = rng.integers(0, N, 20), rng.integers(0, K, 20)
    assert np.array_equal(oracle.wgrad_bf16_sample(g, x, ns, ks), out[ns, ks])


def test_grouped_wgrad_matches_numpy_per_expert():
    """Each expert's slice of rows against numpy's fp64 g^T x over exactly those
    rows (a shifted boundary or a dropped expert fails); an empty expert is 0."""
    rng = np.random.default_rng(7)
    counts = [5, 0, 33, 1, 0, 9]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    Mt, N, K = int(off[-1]), 16, 24
    g = (rng.standard_normal((Mt, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = (rng.standard_normal((Mt, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out = oracle.grouped_wgrad_bf16(g, x, off)
    gf = oracle.bf16_to_f32(g).astype(np.float64)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    assert out.shape == (len(counts), N, K)
    for e in range(len(counts)):
        ref = gf[off[e]:off[e + 1]].T @ xf[off[e]:off[e + 1]]
        np.testing.assert_allclose(out[e], ref, rtol=1e-12, atol=1e-12)
    assert not out[1].any() and not out[4].any()
    S = oracle.grouped_wgrad_bf16(g, x, off, absolute=True)
    np.testing.assert_allclose(S[2], np.abs(gf[5:38]).T @ np.abs(xf[5:38]), rtol=1e-12)


def test_absolute_product_sums():
    """S = sum |a_k b_k| |scales|: equals numpy's |A| @ |B|^T, bounds |ref|, and equals ref
    when every product is non-negative."""
    rng = np.random.default_rng(8)
    M, N, K = 20, 24, 256
    a, b = _codes("e4m3fn", (M, K), rng), _codes("e4m3fn", (N, K), rng)
    sa = rng.uniform(0.5, 2, M).astype(np.float32)
    sb = rng.uniform(0.5, 2, N).astype(np.float32)
    ref = oracle.scaled_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_ROW, sa, sb)
    S = oracle.scaled_mm(a, "e4m3fn", b, "e4m3fn", oracle.SCALE_ROW, sa, sb, absolute=True)
    np.testing.assert_allclose(S, (np.abs(_dec("e4m3fn", a)) @ np.abs(_dec("e4m3fn", b)).T) * sa[:, None] * sb[None, :],
                               rtol=1e-13)
    assert np.all(S >= np.abs(ref) * (1 - 1e-15))
    pa, pb = a & 0x7F, b & 0x7F  # clear the sign bits: all products >= 0
    np.testing.assert_allclose(oracle.scaled_mm(pa, "e4m3fn", pb, "e4m3fn", oracle.SCALE_ROW, sa, sb, absolute=True),
                               oracle.scaled_mm(pa, "e4m3fn", pb, "e4m3fn", oracle.SCALE_ROW, sa, sb), rtol=1e-15)
    off = _offsets([7, 0, 13])
    ga = _codes("e4m3fn", (20, K), rng)
    gb = _codes("e4m3fn", (3, N, K), rng)
    ia = rng.uniform(0.5, 2, 20).astype(np.float32)
    ib = rng.uniform(0.5, 2, (3, N)).astype(np.float32)
    G = oracle.grouped_mm(ga, "e4m3fn", gb, "e4m3fn", oracle.SCALE_ROW, ia, ib, off, absolute=True)
    rows, cols = rng.integers(0, 20, 30), rng.integers(0, N, 30)
    assert np.array_equal(oracle.grouped_mm_sample(ga, "e4m3fn", gb, "e4m3fn", oracle.SCALE_ROW, ia, ib, off, rows,
                                                   cols, absolute=True), G[rows, cols])
    g = (rng.standard_normal((30, 8)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = (rng.standard_normal((30, 6)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    W = oracle.wgrad_bf16(g, x, absolute=True)
    np.testing.assert_allclose(W, np.abs(oracle.bf16_to_f32(g).astype(np.float64)).T
                               @ np.abs(oracle.bf16_to_f32(x).astype(np.float64)), rtol=1e-13)
