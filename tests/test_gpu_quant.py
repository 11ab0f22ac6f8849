"""GPU parity of the quantization kernels: every byte and every scale must equal the
oracle's (bit-exact), on small ragged shapes that span several tiles and on the full
workload sizes."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (check_guard, empty_u8, gpu, have_gpu, lib, to_dev, to_dev_bf16, u8)

pytestmark = [gpu, pytest.mark.skipif(not have_gpu(), reason="needs an MI355X")]

EPS = 1e-12


@pytest.fixture(scope="module")
def f():
    oracle.build(force=False)
    synth.build(force=False)
    f = lib()
    e4, e5 = f.fp8_probe(0)
    print(f"probe: e4m3 native={e4} e5m2 native={e5}", flush=True)
    return f


def _natives(f):
    e4, e5 = f.fp8_probe(0)
    name = {0: "e4m3fn", 1: "e4m3fnuz", 2: "e5m2", 3: "e5m2fnuz"}
    return [(f.E4M3_NATIVE, name[e4]), (f.E5M2_NATIVE, name[e5])]


def _x(shape, seed, spread=True):
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    rm = synth.log_uniform_row_mult(rows, seed + 7, -8, 8) if spread else None
    return synth.normal_bf16(shape, seed, 1.0, row_mult=rm)


def test_probe_reports_ocp_on_gfx950(f):
    import torch
    e4, e5 = f.fp8_probe(0)
    print("device:", torch.cuda.get_device_properties(0).gcnArchName, "e4m3:", e4, "e5m2:", e5, flush=True)
    # the answer is whatever the hardware measured; it must be one consistent family
    assert (e4, e5) in [(f.E4M3FN, f.E5M2), (f.E4M3FNUZ, f.E5M2FNUZ)]
    assert f.fp8_format_max(f.E4M3_NATIVE) == (448.0 if e4 == f.E4M3FN else 240.0)


def test_hardware_convert_matches_oracle_encoder(f):
    """Every finite bf16 pattern times three scales, through the row kernel with a
    unit scale (amax = fmax), against the oracle's bit-level encoder."""
    import torch
    for fmt, name in _natives(f):
        fm = oracle.fp8_max(name)
        bits = np.arange(65536, dtype=np.uint32)
        v = (bits << 16).view(np.float32)
        v = v[np.isfinite(v) & (np.abs(v) <= fm)]
        # rows of 1024 values with the row max pinned to fmax -> scale 1 exactly
        n = (v.size + 1022) // 1023 * 1023
        pad = np.zeros(n - v.size, np.float32)
        body = np.concatenate([v, pad]).reshape(-1, 1023)
        rows = np.concatenate([body, np.full((body.shape[0], 1), fm, np.float32)], axis=1)
        xb = (rows.view(np.uint32) >> 16).astype(np.uint16)
        xd = to_dev_bf16(xb)
        q = torch.empty(xb.shape, dtype=torch.uint8, device="cuda:0")
        s = torch.empty(xb.shape[0], dtype=torch.float32, device="cuda:0")
        f.fp8_quant_row(xd, fmt, EPS, q, s)
        torch.cuda.synchronize()
        assert np.all(s.cpu().numpy() == 1.0)
        ref = oracle.encode(name, rows)
        got = u8(q)
        bad = np.nonzero(got != ref)
        assert bad[0].size == 0, (name, rows[bad][:8], got[bad][:8], ref[bad][:8])


def _run_row(f, fmt, name, x, guard=256):
    import torch
    b = 1 if x.ndim == 2 else x.shape[0]
    q, full = empty_u8(x.shape, guard)
    s = torch.empty(x.shape[:-1], dtype=torch.float32, device="cuda:0")
    i = torch.empty(x.shape[:-1], dtype=torch.float32, device="cuda:0")
    f.fp8_quant_row(to_dev_bf16(x), fmt, EPS, q, s, i)
    torch.cuda.synchronize()
    check_guard(full, guard)
    rq, rs, ri = oracle.quant_row(x, name, EPS)
    assert np.array_equal(u8(q), rq), name
    assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)
    return q


@pytest.mark.parametrize("shape", [(1, 8), (3, 8), (7, 4096), (5, 14336), (4, 16392), (33, 100), (2, 3, 2056),
                                   (257, 1016)])
def test_quant_row(f, shape):
    x = _x(shape, 100 + shape[-1])
    for fmt, name in _natives(f):
        print("row", shape, name, flush=True)
        _run_row(f, fmt, name, x)


def test_quant_row_zero_and_negative_zero(f):
    x = _x((6, 512), 5)
    x[1] = 0x0000
    x[2] = 0x8000
    x[3, :7] = 0x8000
    for fmt, name in _natives(f):
        _run_row(f, fmt, name, x)


def test_quant_row_deterministic(f):
    x = _x((64, 4096), 9)
    for fmt, name in _natives(f):
        a = u8(_run_row(f, fmt, name, x))
        b = u8(_run_row(f, fmt, name, x))
        assert np.array_equal(a, b)


def _run_col(f, fmt, name, x, guard=256):
    import torch
    bsz, R, C = (1,) + x.shape if x.ndim == 2 else x.shape
    shape_t = x.shape[:-2] + (C, R)
    q, full = empty_u8(shape_t, guard)
    s = torch.empty(x.shape[:-2] + (C,), dtype=torch.float32, device="cuda:0")
    i = torch.empty(x.shape[:-2] + (C,), dtype=torch.float32, device="cuda:0")
    wsb = f.fp8_quant_col_ws_bytes(bsz, R, C)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device="cuda:0")
    f.fp8_quant_col(to_dev_bf16(x), fmt, EPS, q, s, i, ws)
    torch.cuda.synchronize()
    check_guard(full, guard)
    rq, rs, ri = oracle.quant_col(x, name, EPS)
    got = u8(q)
    bad = np.nonzero(got != rq)
    assert bad[0].size == 0, (name, [b[:5] for b in bad])
    assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)


@pytest.mark.parametrize("shape", [(16, 8), (2048, 64), (2048, 72), (48, 200), (100, 24), (4096, 128),
                                   (3, 48, 40), (2, 2064, 64), (1024, 2064, 8), (64, 64, 512), (70, 32, 520),
                                   (9, 2048, 3648), (40, 2000, 840),
                                   (14336, 256), (16384, 200), (3, 8192, 136), (5008, 72), (16400, 72)])
def test_quant_col(f, shape):
    """Up to 2048 rows: one workgroup per strip in registers. More rows: the split
    form (amax pass over row chunks, then the cast pass), with ragged last strips,
    batches and row counts that are not a multiple of the 1024-row chunk."""
    x = _x(shape, 300 + shape[-1], spread=False)
    for fmt, name in _natives(f):
        print("col", shape, name, flush=True)
        _run_col(f, fmt, name, x)


def test_quant_col_zero_columns(f):
    x = synth.normal_bf16((4, 256, 136), 11, 0.02)
    synth.zero_columns(x, 2, 12)
    x[1][:, 5] = 0x8000
    for fmt, name in _natives(f):
        _run_col(f, fmt, name, x)


@pytest.mark.parametrize("n", [1, 7, 4096, 131072, 262144, 3_000_017])
def test_quant_tensor(f, n):
    import torch
    x = _x((n,), 400 + n % 97, spread=False)
    for fmt, name in _natives(f):
        print("tensor", n, name, flush=True)
        q, full = empty_u8((n,), 256)
        s = torch.empty(1, dtype=torch.float32, device="cuda:0")
        i = torch.empty(1, dtype=torch.float32, device="cuda:0")
        ws = torch.full((f.fp8_quant_tensor_ws_bytes(),), 0x5A, dtype=torch.uint8, device="cuda:0")
        xd = to_dev_bf16(x)
        f.fp8_quant_tensor(xd, fmt, EPS, q, s, i, ws)
        f.fp8_quant_tensor(xd, fmt, EPS, q, s, i, ws)  # the workspace content on entry does not matter
        torch.cuda.synchronize()
        check_guard(full, 256)
        rq, rs, ri = oracle.quant_tensor(x, name, EPS)
        assert np.array_equal(u8(q), rq) and s.item() == rs[0] and i.item() == ri[0]


@pytest.mark.parametrize("shape", [(5, 300), (3, 4096), (2, 3, 136)])
def test_quant_row_fnuz_interop(f, shape):
    """fnuz bytes written by the software encoder on an OCP device, against the
    oracle's fnuz encoder (rows with outliers, zeros and negative zeros)."""
    import torch
    e4, e5 = f.fp8_probe(0)
    if (e4, e5) != (f.E4M3FN, f.E5M2):
        pytest.skip("fnuz is this device's native encoding")
    x = _x(shape, 700 + shape[-1])
    flat = x.reshape(-1, shape[-1])
    flat[0, :5] = 0x8000
    flat[-1, :] = 0x0000
    for fmt, name in [(f.E4M3FNUZ, "e4m3fnuz"), (f.E5M2FNUZ, "e5m2fnuz")]:
        q, full = empty_u8(x.shape, 256)
        s = torch.empty(x.shape[:-1], dtype=torch.float32, device="cuda:0")
        i = torch.empty(x.shape[:-1], dtype=torch.float32, device="cuda:0")
        f.fp8_quant_row(to_dev_bf16(x), fmt, EPS, q, s, i)
        torch.cuda.synchronize()
        check_guard(full, 256)
        rq, rs, ri = oracle.quant_row(x, name, EPS)
        got = u8(q)
        bad = np.nonzero(got != rq)
        assert bad[0].size == 0, (name, [b[:5] for b in bad], got[bad][:8], rq[bad][:8])
        assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)
        assert not np.any(got == 0x80), "fnuz NaN code written"


@pytest.mark.parametrize("n", [7, 262144, 3_000_017])
def test_quant_tensor_fnuz_interop(f, n):
    import torch
    e4, e5 = f.fp8_probe(0)
    if (e4, e5) != (f.E4M3FN, f.E5M2):
        pytest.skip("fnuz is this device's native encoding")
    x = _x((n,), 710 + n % 97, spread=False)
    for fmt, name in [(f.E4M3FNUZ, "e4m3fnuz"), (f.E5M2FNUZ, "e5m2fnuz")]:
        q, full = empty_u8((n,), 256)
        s = torch.empty(1, dtype=torch.float32, device="cuda:0")
        i = torch.empty(1, dtype=torch.float32, device="cuda:0")
        ws = torch.empty((f.fp8_quant_tensor_ws_bytes(),), dtype=torch.uint8, device="cuda:0")
        f.fp8_quant_tensor(to_dev_bf16(x), fmt, EPS, q, s, i, ws)
        torch.cuda.synchronize()
        check_guard(full, 256)
        rq, rs, ri = oracle.quant_tensor(x, name, EPS)
        assert np.array_equal(u8(q), rq) and s.item() == rs[0] and i.item() == ri[0], name


def test_fnuz_every_representable_value(f):
    """Every bf16 pattern whose magnitude is within the fnuz range, through the
    row kernel with a unit scale (amax pinned to fnuz max): the software encoder
    against the oracle's, over the whole subnormal band, all binades and ties."""
    import torch
    e4, e5 = f.fp8_probe(0)
    if (e4, e5) != (f.E4M3FN, f.E5M2):
        pytest.skip("fnuz is this device's native encoding")
    for fmt, name in [(f.E4M3FNUZ, "e4m3fnuz"), (f.E5M2FNUZ, "e5m2fnuz")]:
        fm = oracle.fp8_max(name)
        bits = np.arange(65536, dtype=np.uint32)
        v = (bits << 16).view(np.float32)
        v = v[np.isfinite(v) & (np.abs(v) <= fm)]
        n = (v.size + 1022) // 1023 * 1023
        body = np.concatenate([v, np.zeros(n - v.size, np.float32)]).reshape(-1, 1023)
        rows = np.concatenate([body, np.full((body.shape[0], 1), fm, np.float32)], axis=1)
        xb = (rows.view(np.uint32) >> 16).astype(np.uint16)
        q = torch.empty(xb.shape, dtype=torch.uint8, device="cuda:0")
        s = torch.empty(xb.shape[0], dtype=torch.float32, device="cuda:0")
        f.fp8_quant_row(to_dev_bf16(xb), fmt, EPS, q, s)
        torch.cuda.synchronize()
        assert np.all(s.cpu().numpy() == 1.0)
        ref = oracle.encode(name, rows)
        got = u8(q)
        bad = np.nonzero(got != ref)
        assert bad[0].size == 0, (name, rows[bad][:8], got[bad][:8], ref[bad][:8])


def test_fnuz_rejected_where_no_encoder(f):
    """Only the rowwise and tensorwise calls write fnuz on an OCP device."""
    import torch
    e4, e5 = f.fp8_probe(0)
    if (e4, e5) != (f.E4M3FN, f.E5M2):
        pytest.skip("fnuz is this device's native encoding")
    x = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda:0")
    q = torch.empty((64, 16), dtype=torch.uint8, device="cuda:0")
    s = torch.empty(64, dtype=torch.float32, device="cuda:0")
    with pytest.raises(f.Fp8Error) as e:
        f.fp8_quant_col(x, f.E4M3FNUZ, EPS, q, s, None, None)
    assert e.value.status == f.ERR_UNSUPPORTED


def _gamma(cols, seed, layer):
    g = synth.normal_bf16((1, cols), seed, 0.1).reshape(cols)
    g = oracle.bf16_to_f32(g) + 1.0  # weights near 1, as trained norms hold
    gb = (g.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b = synth.normal_bf16((1, cols), seed + 1, 0.1).reshape(cols) if layer else None
    return gb, b


@pytest.mark.parametrize("shape", [(3, 8), (7, 1016), (5, 4096), (4, 7168), (2, 16384), (33, 2056)])
@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_norm_quant_row(f, shape, kind):
    """The fused normalization + rowwise quantization: the bf16 activation, the
    codes and the scales equal the oracle's (norm, then quant_row), bit for bit."""
    import torch
    rows, cols = shape
    layer = kind == "layer"
    x = _x(shape, 800 + cols)
    g, b = _gamma(cols, 810 + cols, layer)
    for fmt, name in _natives(f):
        y = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
        q, full = empty_u8(shape, 256)
        s = torch.empty(rows, dtype=torch.float32, device="cuda:0")
        i = torch.empty(rows, dtype=torch.float32, device="cuda:0")
        f.fp8_norm_quant_row(to_dev_bf16(x), to_dev_bf16(g), None if b is None else to_dev_bf16(b),
                             f.NORM_LAYER if layer else f.NORM_RMS, 1e-5, fmt, EPS, y, q, s, i)
        torch.cuda.synchronize()
        check_guard(full, 256)
        ry, rq, rs, ri = oracle.norm_quant_row(x, g, b, layer, 1e-5, name, EPS)
        gy = y.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(gy, ry), (kind, shape, np.nonzero(gy != ry)[0][:5])
        assert np.array_equal(u8(q), rq), (kind, shape, name)
        assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)


def _bits(values):
    f32 = np.asarray(values, np.float32)
    b = (f32.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f32(b), f32)
    return b


def _rstd_boundary_row(cols, norm_eps):
    """A row whose RMSNorm rstd lies within 2^-60 of an fp32 rounding midpoint (3/4 +
    2^-25): bf16 values chosen greedily so their squares sum to cols * (1/m^2 - eps),
    each the largest bf16 not above the square root of what is left."""
    import math
    from fractions import Fraction
    m = Fraction(3, 4) + Fraction(1, 2 ** 25)
    r = cols * (1 / (m * m) - Fraction(norm_eps))
    vals = []
    for _ in range(12):
        if r <= 0:
            break
        x = float((np.float32(math.sqrt(float(r))).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32))
        if x == 0.0:
            break
        vals.append(x)
        r -= Fraction(x) ** 2
    row = np.zeros(cols, np.float32)
    row[:len(vals)] = vals
    return _bits(row)


def _hard_rows(cols, seed):
    """Rows the kernel's fp64 sums cannot settle, so it takes its exact path:
    2^60 + 2^-20 - 2^60 (the exact mean is 2^-20 / cols), squares just above an fp64
    tie (2^80 + 2^27 + 2^-40), subnormals beside 1.0, rows of random sign, mantissa
    and exponent over 2^-67 .. 2^63, and a row whose RMSNorm rstd sits on an fp32
    rounding midpoint; plus an all-zero row."""
    rng = np.random.default_rng(seed)
    rows = [_rstd_boundary_row(cols, 1e-5)]
    r = np.zeros(cols, np.float32)
    r[[0, 5, 9]] = [2.0 ** 60, 2.0 ** -20, -(2.0 ** 60)]
    rows.append(_bits(r))
    r = np.zeros(cols, np.float32)
    r[[1, 2, 3, cols - 1]] = [2.0 ** 40, 2.0 ** 13, 2.0 ** 13, 2.0 ** -20]
    rows.append(_bits(r))
    r = np.ones(cols, np.float32)
    r[::7] = 2.0 ** -133
    r[3::11] = -(2.0 ** -126)
    rows.append(_bits(r))
    for _ in range(3):
        e = rng.integers(60, 191, cols)
        rows.append(((rng.integers(0, 2, cols) << 15) | (e << 7) | rng.integers(0, 128, cols)).astype(np.uint16))
    rows.append(np.zeros(cols, np.uint16))
    return np.stack(rows)


@pytest.mark.parametrize("cols", [1016, 4096, 7168])
@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_norm_quant_row_exact_sums(f, cols, kind):
    """Rows whose statistics need the exact sums (the kernel's LDS integer path),
    mixed with ordinary rows (the fp64 path): y, codes and scales bit-exact against
    the oracle, whose sums are exact by construction. One wavefront per row (1016,
    4096 columns) and one workgroup per row (7168)."""
    import torch
    layer = kind == "layer"
    x = np.concatenate([_x((5, cols), 850 + cols), _hard_rows(cols, 860 + cols), _x((3, cols), 870 + cols)])
    rows = x.shape[0]
    g, b = _gamma(cols, 880 + cols, layer)
    fmt, name = _natives(f)[0]
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda:0")
    q, full = empty_u8((rows, cols), 256)
    s = torch.empty(rows, dtype=torch.float32, device="cuda:0")
    i = torch.empty(rows, dtype=torch.float32, device="cuda:0")
    f.fp8_norm_quant_row(to_dev_bf16(x), to_dev_bf16(g), None if b is None else to_dev_bf16(b),
                         f.NORM_LAYER if layer else f.NORM_RMS, 1e-5, fmt, EPS, y, q, s, i)
    torch.cuda.synchronize()
    check_guard(full, 256)
    ry, rq, rs, ri = oracle.norm_quant_row(x, g, b, layer, 1e-5, name, EPS)
    gy = y.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.nonzero(np.any(gy != ry, axis=1))[0]
    assert bad.size == 0, (kind, cols, bad)
    assert np.array_equal(u8(q), rq), (kind, cols)
    assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)


def test_norm_quant_row_partial_outputs_and_errors(f):
    """y only, q only; bad shapes and arguments are refused."""
    import torch
    x = _x((6, 512), 830)
    g, _ = _gamma(512, 831, False)
    xd, gd = to_dev_bf16(x), to_dev_bf16(g)
    ry, rq, rs, _ = oracle.norm_quant_row(x, g, None, False, 1e-6, _natives(f)[0][1], EPS)
    y = torch.empty((6, 512), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_norm_quant_row(xd, gd, None, f.NORM_RMS, 1e-6, f.E4M3_NATIVE, EPS, y, None, None)
    q = torch.empty((6, 512), dtype=torch.uint8, device="cuda:0")
    s = torch.empty(6, dtype=torch.float32, device="cuda:0")
    f.fp8_norm_quant_row(xd, gd, None, f.NORM_RMS, 1e-6, f.E4M3_NATIVE, EPS, None, q, s)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ry)
    assert np.array_equal(u8(q), rq) and np.array_equal(s.cpu().numpy(), rs)
    bad = [((6, 500), {}, f.ERR_ALIGNMENT), ((2, 16392), {}, f.ERR_UNSUPPORTED),
           ((6, 512), {"beta": True}, f.ERR_INVALID_ARGUMENT)]
    for shape, kw, st in bad:
        xx = torch.zeros(shape, dtype=torch.bfloat16, device="cuda:0")
        gg = torch.zeros(shape[1], dtype=torch.bfloat16, device="cuda:0")
        qq = torch.empty(shape, dtype=torch.uint8, device="cuda:0")
        ss = torch.empty(shape[0], dtype=torch.float32, device="cuda:0")
        with pytest.raises(f.Fp8Error) as e:
            f.fp8_norm_quant_row(xx, gg, gg if kw.get("beta") else None, f.NORM_RMS, 1e-6, f.E4M3_NATIVE, EPS, None,
                                 qq, ss)
        assert e.value.status == st, (shape, kw, e.value.status)


def _run_dual(f, M, N, K, seed, with_row=True, zero_rows=False):
    """fp8_quant_dual against the oracle's quant_dual, byte for byte, with
    guard bands after every output."""
    import torch
    e4, e5 = f.fp8_probe(0)
    name = {0: "e4m3fn", 1: "e4m3fnuz", 2: "e5m2", 3: "e5m2fnuz"}
    gy = _x((M, N), seed, spread=False)
    x = _x((M, K), seed + 1, spread=True)
    if zero_rows:
        gy[:16] = 0x8000
        x[:, :8] = 0x0000
    gq, gq_full = empty_u8((M, N), 256) if with_row else (None, None)
    gqT, gqT_full = empty_u8((N, M), 256)
    xqT, xqT_full = empty_u8((K, M), 256)
    sc = [torch.empty(1, dtype=torch.float32, device="cuda:0") for _ in range(4)]
    ws = torch.full((f.fp8_quant_dual_ws_bytes(),), 0x5A, dtype=torch.uint8, device="cuda:0")
    f.fp8_quant_dual(to_dev_bf16(gy), to_dev_bf16(x), f.E5M2_NATIVE, f.E4M3_NATIVE, EPS, gq, gqT, sc[0], sc[1],
                     xqT, sc[2], sc[3], ws)
    torch.cuda.synchronize()
    for full in (gq_full, gqT_full, xqT_full):
        if full is not None:
            check_guard(full, 256)
    rgq, rgqT, rgs, rgi, rxqT, rxs, rxi = oracle.quant_dual(gy, x, name[e5], name[e4], EPS)
    if with_row:
        assert np.array_equal(u8(gq), rgq), "gq"
    assert np.array_equal(u8(gqT), rgqT), "gqT"
    assert np.array_equal(u8(xqT), rxqT), "xqT"
    got = [t.item() for t in sc]
    assert got == [rgs[0], rgi[0], rxs[0], rxi[0]], (got, rgs, rgi, rxs, rxi)


@pytest.mark.parametrize("M,N,K", [(16, 8, 8), (48, 264, 136), (1040, 520, 264), (2048, 1032, 64),
                                   (3088, 72, 4104)])
def test_quant_dual(f, M, N, K):
    """Several 1024-row chunks with a ragged last one, strips narrower than 64
    columns, and both outputs of gy from one read."""
    print("dual", M, N, K, flush=True)
    _run_dual(f, M, N, K, 600 + M % 97)


def test_quant_dual_without_row_output_and_zeros(f):
    _run_dual(f, 64, 128, 96, 611, with_row=False, zero_rows=True)


def test_quant_dual_rejects_bad_shapes(f):
    import torch
    z = lambda *s: torch.zeros(s, dtype=torch.uint8, device="cuda:0")
    one = torch.empty(1, dtype=torch.float32, device="cuda:0")
    ws = z(f.fp8_quant_dual_ws_bytes())
    for M, N, K, st in [(24, 16, 16, f.ERR_ALIGNMENT), (32, 12, 16, f.ERR_ALIGNMENT), (32, 16, 4, f.ERR_ALIGNMENT)]:
        gy = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda:0")
        x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda:0")
        with pytest.raises(f.Fp8Error) as e:
            f.fp8_quant_dual(gy, x, f.E5M2_NATIVE, f.E4M3_NATIVE, EPS, z(M, N), z(N, M), one, one, z(K, M), one, one,
                             ws)
        assert e.value.status == st, (M, N, K, e.value.status)
    gy = torch.zeros((32, 16), dtype=torch.bfloat16, device="cuda:0")
    x = torch.zeros((32, 16), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(f.Fp8Error) as e:
        f.fp8_quant_dual(gy, x, f.E5M2_NATIVE, f.E4M3_NATIVE, EPS, None, z(16, 32), one, None, z(16, 32), one, None,
                         None)
    assert e.value.status == f.ERR_WORKSPACE


@pytest.mark.parametrize("br,shape", [(1, (3, 300)), (1, (5, 1024)), (1, (2, 7, 640)), (128, (130, 260)),
                                      (128, (2, 256, 384)), (128, (300, 136)), (128, (300, 768)),
                                      (128, (3, 200, 512)), (128, (64, 256))])
def test_quant_block(f, br, shape):
    import torch
    x = _x(shape, 500 + shape[-1])
    b = 1 if len(shape) == 2 else shape[0]
    R, C = shape[-2], shape[-1]
    nbr, nbc = -(-R // br), -(-C // 128)
    for fmt, name in _natives(f):
        print("block", br, shape, name, flush=True)
        q, full = empty_u8(shape, 256)
        s = torch.empty(shape[:-2] + (nbr, nbc), dtype=torch.float32, device="cuda:0")
        i = torch.empty_like(s)
        f.fp8_quant_block(to_dev_bf16(x), br, 128, fmt, EPS, q, s, i)
        torch.cuda.synchronize()
        check_guard(full, 256)
        rq, rs, ri = oracle.quant_block(x, br, 128, name, EPS)
        assert np.array_equal(u8(q), rq)
        assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", [(4, 64), (3, 96), (2, 5, 160), (129, 5120)])
def test_quant_mx(f, mode, shape):
    import torch
    x = _x(shape, 600 + shape[-1])
    x.reshape(-1, shape[-1])[0, :32] = 0  # an all-zero group: the eps clamp
    for fmt, name in _natives(f):
        q, full = empty_u8(shape, 256)
        e, efull = empty_u8(shape[:-1] + (shape[-1] // 32,), 256)
        f.fp8_quant_mx(to_dev_bf16(x), fmt, mode, EPS, q, e)
        torch.cuda.synchronize()
        check_guard(full, 256)
        check_guard(efull, 256)
        rq, re = oracle.quant_mx(x, name, mode, EPS)
        assert np.array_equal(u8(e), re), name
        assert np.array_equal(u8(q), rq), name
