"""Pins of the oracle's quantization at every granularity (CPU only).

References: a brute-force chain in exact rational arithmetic on tiny shapes,
invariants the method guarantees at any size, and special cases where one
granularity reduces to another.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import oracle_pins as pins

FMTS = ["e4m3fn", "e4m3fnuz", "e5m2", "e5m2fnuz"]
EPS = 1e-12


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)
    synth.build(force=False)


def _rand_bits(shape, seed, sigma=1.0, spread=False):
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    rm = synth.log_uniform_row_mult(rows, seed + 99, -6, 6) if spread else None
    return synth.normal_bf16(shape, seed, sigma, row_mult=rm)


# ---- brute force on tiny shapes ------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 1), (3, 5), (8, 8), (2, 7)])
def test_row_bruteforce(fmt, shape):
    x = _rand_bits(shape, 17 + shape[0], spread=True)
    q, s, i = oracle.quant_row(x, fmt, EPS)
    fmax = oracle.fp8_max(fmt)
    for r in range(shape[0]):
        rq, rs, ri = pins.quant_chain_reference(fmt, x[r], EPS, fmax)
        assert np.array_equal(q[r], rq) and s[r] == rs and i[r] == ri


@pytest.mark.parametrize("fmt", FMTS)
def test_col_block_tensor_mx_bruteforce(fmt):
    fmax = oracle.fp8_max(fmt)
    x = _rand_bits((6, 8), 41, spread=True)
    qT, s, i = oracle.quant_col(x, fmt, EPS)
    for c in range(8):
        rq, rs, ri = pins.quant_chain_reference(fmt, x[:, c], EPS, fmax)
        assert np.array_equal(qT[c], rq) and s[c] == rs and i[c] == ri
    q, s, i = oracle.quant_block(x, 4, 3, fmt, EPS)  # ragged edge blocks on both axes
    for rb in range(2):
        for cb in range(3):
            win = x[rb * 4:(rb + 1) * 4, cb * 3:(cb + 1) * 3]
            rq, rs, ri = pins.quant_chain_reference(fmt, win, EPS, fmax)
            assert np.array_equal(q[rb * 4:(rb + 1) * 4, cb * 3:(cb + 1) * 3], rq)
            assert s[rb, cb] == rs and i[rb, cb] == ri
    q, s, i = oracle.quant_tensor(x, fmt, EPS)
    rq, rs, ri = pins.quant_chain_reference(fmt, x, EPS, fmax)
    assert np.array_equal(q, rq) and s[0] == rs and i[0] == ri


@pytest.mark.parametrize("gfmt,xfmt", [("e5m2", "e4m3fn"), ("e5m2fnuz", "e4m3fnuz")])
def test_dual_bruteforce(gfmt, xfmt):
    """The all-FP8 backward's operands against the brute-force chain, one
    tensor scale each: gqT[n][m] is the chain's code of gy[m][n] and xqT[k][m]
    that of x[m][k] (a transposed orientation or a swapped scale fails)."""
    gy = _rand_bits((5, 7), 43, spread=True)
    x = _rand_bits((5, 3), 44, spread=True)
    gq, gqT, gs, gi, xqT, xs, xi = oracle.quant_dual(gy, x, gfmt, xfmt, EPS)
    rg, rgs, rgi = pins.quant_chain_reference(gfmt, gy, EPS, oracle.fp8_max(gfmt))
    rx, rxs, rxi = pins.quant_chain_reference(xfmt, x, EPS, oracle.fp8_max(xfmt))
    assert gq.shape == (5, 7) and gqT.shape == (7, 5) and xqT.shape == (3, 5)
    for m in range(5):
        for n in range(7):
            assert gq[m, n] == rg[m, n] and gqT[n, m] == rg[m, n]
        for k in range(3):
            assert xqT[k, m] == rx[m, k]
    assert (gs[0], gi[0], xs[0], xi[0]) == (rgs, rgi, rxs, rxi)


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_mx_bruteforce(fmt):
    # MX mode 0: power-of-two scale = largest 2^k with amax * 2^k <= fmax
    x = _rand_bits((3, 64), 43, spread=True)
    q, e = oracle.quant_mx(x, fmt)
    fmax = oracle.fp8_max(fmt)
    xf = synth.bf16_bits_to_f32(x)
    for r in range(3):
        for g in range(2):
            grp = xf[r, g * 32:(g + 1) * 32].astype(np.float64)
            amax = np.abs(grp).max()
            k = int(np.floor(np.log2(fmax / amax)))
            while amax * 2.0 ** k > fmax:
                k -= 1
            while amax * 2.0 ** (k + 1) <= fmax:
                k += 1
            assert e[r, g] == 127 - k
            y = np.clip((grp * 2.0 ** k).astype(np.float32), -fmax, fmax)  # exact: power of two
            assert np.array_equal(q[r, g * 32:(g + 1) * 32], pins.nearest_encode(fmt, y))


# ---- invariants at larger sizes ---------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
def test_row_invariants(fmt):
    x = _rand_bits((64, 300), 51, spread=True)
    q, s, inv = oracle.quant_row(x, fmt, EPS)
    fmax = np.float32(oracle.fp8_max(fmt))
    xf = synth.bf16_bits_to_f32(x)
    maxcode = oracle.encode(fmt, [fmax])[0]
    dec = oracle.decode(fmt, q)
    y = np.clip(xf * s[:, None], -fmax, fmax)  # numpy fp32 product, IEEE
    for r in range(64):
        j = np.argmax(np.abs(xf[r]))
        assert (q[r, j] & 0x7F) == maxcode
    ulp = np.vectorize(lambda v: pins.fp8_ulp(fmt, v))(y)
    assert np.all(np.abs(dec - y) <= ulp / 2)
    # dequantized error bound
    err = np.abs(dec * inv[:, None].astype(np.float64) - xf)
    bound = (ulp / 2 + 2.0 ** -24 * np.abs(y)) * inv[:, None] + 2.0 ** -22 * np.abs(xf)
    assert np.all(err <= bound)


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_groups_and_negative_zero(fmt):
    x = _rand_bits((4, 64), 61)
    x[1] = 0x0000  # +0 row: the eps clamp
    x[2] = 0x8000  # -0 row
    q, s, i = oracle.quant_row(x, fmt, EPS)
    fmax = oracle.fp8_max(fmt)
    _, s_eps, i_eps = oracle.scale_from_amax(fmt, 0.0, EPS)
    assert s[1] == s_eps and s[2] == s_eps and i[1] == i_eps
    assert np.all(q[1] == 0)
    neg0 = 0x00 if "fnuz" in fmt else 0x80
    assert np.all(q[2] == neg0)
    assert s_eps == np.float32(fmax / EPS)


def test_special_case_equivalences():
    x = _rand_bits((2, 37, 130), 71, spread=True)
    for fmt in FMTS:
        q_r, s_r, i_r = oracle.quant_row(x, fmt, EPS)
        # col(x) == row(x^T) byte for byte
        xt = np.ascontiguousarray(np.swapaxes(x, 1, 2))
        q_c, s_c, i_c = oracle.quant_col(x, fmt, EPS)
        q_rt, s_rt, i_rt = oracle.quant_row(xt, fmt, EPS)
        assert np.array_equal(q_c, q_rt) and np.array_equal(s_c, s_rt) and np.array_equal(i_c, i_rt)
        # block(1 x cols) == row
        q_b, s_b, i_b = oracle.quant_block(x, 1, 130, fmt, EPS)
        assert np.array_equal(q_b, q_r) and np.array_equal(s_b[..., 0], s_r)
        # block(rows x cols) == tensor, per batch
        q_b, s_b, _ = oracle.quant_block(x, 37, 130, fmt, EPS)
        q_t, s_t, _ = oracle.quant_tensor(np.ascontiguousarray(x[1]), fmt, EPS)
        assert np.array_equal(q_b[1], q_t) and s_b[1, 0, 0] == s_t[0]
    # tensor == row when every row has the same amax
    y = _rand_bits((16, 64), 73)
    y[:, 5] = 0x4100  # 8.0 dominates every row
    for fmt in FMTS:
        q_t, s_t, _ = oracle.quant_tensor(y, fmt, EPS)
        q_r, s_r, _ = oracle.quant_row(y, fmt, EPS)
        assert np.array_equal(q_t, q_r) and np.all(s_r == s_t[0])


def test_mx_power_of_two_data_is_exact():
    # values that are fmax-scaled powers of two survive MX quantization exactly
    fmt = "e4m3fn"
    rng = np.random.default_rng(3)
    k = rng.integers(-5, 5, (4, 64))
    v = (2.0 ** k * rng.choice([-1, 1], k.shape)).astype(np.float32)
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    q, e = oracle.quant_mx(bits, fmt)
    dec = oracle.decode(fmt, q) * np.exp2(np.repeat(e.astype(np.int64) - 127, 32, axis=1))
    assert np.array_equal(dec, v.astype(np.float64))


def test_thread_count_does_not_change_results():
    x = _rand_bits((3, 50, 96), 81, spread=True)
    for f in (oracle.quant_row, oracle.quant_col):
        a = f(x, "e4m3fn", EPS, threads=1)
        b = f(x, "e4m3fn", EPS, threads=8)
        for u, v in zip(a, b):
            assert np.array_equal(u, v)


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
@pytest.mark.parametrize("mode", [0, 1])
def test_mx_exponent_range_at_the_smallest_eps(fmt, mode):
    """With eps = 2^-100, the smallest the library accepts, an all-zero group's E8M0
    byte is 127 - floor(log2(fmax / eps)) (mode 0) or 127 + floor(log2 eps) -
    floor(log2 fmax) (mode 1), inside [1, 254]; the largest bf16 amax stays inside too."""
    import math
    fmax = oracle.fp8_max(fmt)
    x = np.zeros((1, 32), np.uint16)
    _, e = oracle.quant_mx(x, fmt, mode, 2.0 ** -100)
    want = 127 - math.floor(math.log2(fmax) + 100) if mode == 0 else 127 - 100 - math.floor(math.log2(fmax))
    assert int(e[0, 0]) == want and 1 <= want <= 254
    big = np.full((1, 32), 0x7F7F, np.uint16)  # largest finite bf16, about 2^128
    _, e = oracle.quant_mx(big, fmt, mode, 2.0 ** -100)
    assert 1 <= int(e[0, 0]) <= 254
