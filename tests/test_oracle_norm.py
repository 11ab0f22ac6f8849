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
