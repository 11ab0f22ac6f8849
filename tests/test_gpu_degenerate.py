"""GPU results at the degenerate sizes, against the oracle.

A group with no elements has amax 0 (the maximum of |x| over an empty set of
non-negative values), so it still gets a scale: the eps-clamped one. A GEMM with
no contraction terms (K = 0) and a weight gradient over no rows (M = 0) are the
empty sum, all zeros. Operands and scales that hold nothing are passed as empty
tensors or None, so a kernel that read them would fault or pick up garbage."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import gpu, have_gpu, lib, to_dev

pytestmark = [gpu, pytest.mark.skipif(not have_gpu(), reason="needs an MI355X")]

EPS = 1e-12


@pytest.fixture(scope="module")
def f():
    oracle.build(force=False)
    return lib()


def _natives(f):
    e4, e5 = f.fp8_probe(0)
    name = {0: "e4m3fn", 1: "e4m3fnuz", 2: "e5m2", 3: "e5m2fnuz"}
    return [(f.E4M3_NATIVE, name[e4]), (f.E5M2_NATIVE, name[e5])]


def _nan(shape):
    import torch
    return torch.full(shape if isinstance(shape, tuple) else (shape,), float("nan"), dtype=torch.float32,
                      device="cuda:0")


def _bf16(shape):
    import torch
    return torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")


def _u8(shape):
    import torch
    return torch.empty(shape, dtype=torch.uint8, device="cuda:0")


def _same(got, ref):
    got = got.cpu().numpy()
    assert got.shape == np.asarray(ref).shape and np.array_equal(got, np.asarray(ref, np.float32)), (got, ref)


def test_empty_tensor_gets_the_clamped_scale(f):
    import torch
    ws = torch.zeros(f.fp8_quant_tensor_ws_bytes(), dtype=torch.uint8, device="cuda:0")
    for fmt, name in _natives(f):
        s, i = _nan(1), _nan(1)
        f.fp8_quant_tensor(_bf16(0), fmt, EPS, _u8(0), s, i, ws)
        torch.cuda.synchronize()
        _, rs, ri = oracle.quant_tensor(np.zeros(0, np.uint16), name, EPS)
        _same(s, rs)
        _same(i, ri)


@pytest.mark.parametrize("shape", [(4, 0), (2, 3, 0)])
def test_empty_rows_get_the_clamped_scale(f, shape):
    import torch
    for fmt, name in _natives(f):
        s, i = _nan(shape[:-1]), _nan(shape[:-1])
        f.fp8_quant_row(_bf16(shape), fmt, EPS, _u8(shape), s, i)
        torch.cuda.synchronize()
        _, rs, ri = oracle.quant_row(np.zeros(shape, np.uint16), name, EPS)
        _same(s, rs)
        _same(i, ri)


def test_empty_rows_fnuz_output(f):
    """The fnuz outputs of the rowwise quantizer use their own fp8 max (240 for e4m3fnuz)."""
    import torch
    if f.fp8_probe(0)[0] != f.E4M3FN:
        pytest.skip("fnuz interop output is offered on OCP devices")
    s, i = _nan((3,)), _nan((3,))
    f.fp8_quant_row(_bf16((3, 0)), f.E4M3FNUZ, EPS, _u8((3, 0)), s, i)
    torch.cuda.synchronize()
    _, rs, ri = oracle.quant_row(np.zeros((3, 0), np.uint16), "e4m3fnuz", EPS)
    _same(s, rs)
    _same(i, ri)


@pytest.mark.parametrize("shape", [(0, 24), (2, 0, 16)])
def test_empty_columns_get_the_clamped_scale(f, shape):
    import torch
    b = shape[0] if len(shape) == 3 else 1
    c = shape[-1]
    for fmt, name in _natives(f):
        s, i = _nan((b, c) if len(shape) == 3 else (c,)), _nan((b, c) if len(shape) == 3 else (c,))
        qT = _u8(shape[:-2] + (c, 0))
        f.fp8_quant_col(_bf16(shape), fmt, EPS, qT, s, i, None)
        torch.cuda.synchronize()
        _, rs, ri = oracle.quant_col(np.zeros(shape, np.uint16), name, EPS)
        _same(s, rs)
        _same(i, ri)


def test_norm_of_empty_rows(f):
    import torch
    for fmt, name in _natives(f):
        s, i = _nan((3,)), _nan((3,))
        f.fp8_norm_quant_row(_bf16((3, 0)), _bf16(0), None, f.NORM_RMS, 1e-6, fmt, EPS, None, _u8((3, 0)), s, i)
        torch.cuda.synchronize()
        _, _, rs, ri = oracle.norm_quant_row(np.zeros((3, 0), np.uint16), np.zeros(0, np.uint16), None, False, 1e-6,
                                             name, EPS)
        _same(s, rs)
        _same(i, ri)


@pytest.mark.parametrize("M,N,K", [(32, 0, 24), (32, 16, 0), (0, 16, 24), (16, 0, 0)])
def test_dual_with_empty_operands(f, M, N, K):
    """The all-FP8 backward's quantization when grad_out or the input holds nothing:
    the other operand is still quantized, and each tensor still has its scale."""
    import torch
    import synth
    synth.build(force=False)
    e4, e5 = f.fp8_probe(0)
    name = {0: "e4m3fn", 1: "e4m3fnuz", 2: "e5m2", 3: "e5m2fnuz"}
    gy = synth.normal_bf16((M, N), 701, 1.0) if M * N else np.zeros((M, N), np.uint16)
    x = synth.normal_bf16((M, K), 702, 1.0) if M * K else np.zeros((M, K), np.uint16)

    def dev(a):
        if a.size == 0:
            return _bf16(a.shape)
        return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    gq, gqT, xqT = _u8((M, N)), _u8((N, M)), _u8((K, M))
    sc = [_nan((1,)) for _ in range(4)]
    ws = torch.zeros(f.fp8_quant_dual_ws_bytes(), dtype=torch.uint8, device="cuda:0")
    f.fp8_quant_dual(dev(gy), dev(x), f.E5M2_NATIVE, f.E4M3_NATIVE, EPS, gq, gqT, sc[0], sc[1], xqT, sc[2], sc[3], ws)
    torch.cuda.synchronize()
    rgq, rgqT, rgs, rgi, rxqT, rxs, rxi = oracle.quant_dual(gy, x, name[e5], name[e4], EPS)
    assert np.array_equal(gq.cpu().numpy(), rgq) and np.array_equal(gqT.cpu().numpy(), rgqT)
    assert np.array_equal(xqT.cpu().numpy(), rxqT)
    assert [t.item() for t in sc] == [rgs[0], rgi[0], rxs[0], rxi[0]]


@pytest.mark.parametrize("out_f32", [False, True])
def test_gemm_without_contraction_is_zero(f, out_f32):
    """K = 0: all zeros, and neither the (empty) operands nor the scales are read
    (the rowwise scales are passed as None)."""
    import torch
    M, N = 300, 264
    dt = torch.float32 if out_f32 else torch.bfloat16
    ot = f.OUT_F32 if out_f32 else f.OUT_BF16
    for scaling in (f.SCALE_TENSOR, f.SCALE_ROW):
        out = torch.full((M, N), float("nan"), dtype=dt, device="cuda:0")
        f.fp8_scaled_mm(_u8((M, 0)), f.E4M3_NATIVE, _u8((N, 0)), f.E4M3_NATIVE, scaling, None, None, ot, out)
        torch.cuda.synchronize()
        ref = oracle.scaled_mm(np.zeros((M, 0), np.uint8), "e4m3fn", np.zeros((N, 0), np.uint8), "e4m3fn",
                               oracle.SCALE_ROW, np.ones(M, np.float32), np.ones(N, np.float32))
        assert np.array_equal(out.float().cpu().numpy(), ref), scaling
    off = to_dev(np.array([0, 100, 100, 300], np.int32))
    for scaling in (f.SCALE_ROW, f.SCALE_BLOCK128, f.SCALE_MX32):
        out = torch.full((M, N if scaling != f.SCALE_BLOCK128 else 256), float("nan"), dtype=dt, device="cuda:0")
        n = out.shape[1]
        f.fp8_grouped_mm(_u8((M, 0)), f.E4M3_NATIVE, _u8((3, n, 0)), f.E4M3_NATIVE, scaling, None, None, off, ot,
                         out)
        torch.cuda.synchronize()
        assert np.array_equal(out.float().cpu().numpy(), np.zeros((M, n))), scaling


def test_wgrad_over_no_rows_is_zero(f):
    import torch
    N, K = 72, 136
    gw = torch.full((N, K), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_wgrad_bf16(_bf16((0, N)), _bf16((0, K)), gw)
    torch.cuda.synchronize()
    ref = oracle.wgrad_bf16(np.zeros((0, N), np.uint16), np.zeros((0, K), np.uint16))
    assert np.array_equal(gw.float().cpu().numpy(), ref)


@pytest.mark.parametrize("recipe", ["rowwise", "tensorwise"])
def test_linear_empty_sums(f, recipe):
    """The linear layer's empty sums: the forward with K = 0, the grad-weight over
    M = 0 rows and the grad-input over N = 0 outputs are zeros."""
    import torch
    R = f.RECIPE_ROWWISE_BF16_WGRAD if recipe == "rowwise" else f.RECIPE_TENSORWISE

    def ws(M, N, K):
        return torch.empty(max(1, f.fp8_linear_ws_bytes(M, N, K, R)), dtype=torch.uint8, device="cuda:0")

    def nan16(shape):
        return torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    y = nan16((48, 32))
    f.fp8_linear_fwd(_bf16((48, 0)), _bf16((32, 0)), R, EPS, f.OUT_BF16, y, ws(48, 32, 0))
    gw = nan16((32, 48))
    f.fp8_linear_bwd(_bf16((0, 32)), _bf16((0, 48)), _bf16((32, 48)), R, EPS, _bf16((0, 48)), gw, ws(0, 32, 48))
    gx = nan16((48, 32))
    f.fp8_linear_bwd(_bf16((48, 0)), _bf16((48, 32)), _bf16((0, 32)), R, EPS, gx, _bf16((0, 32)), ws(48, 0, 32))
    torch.cuda.synchronize()
    for name, t in (("y", y), ("grad-weight", gw), ("grad-input", gx)):
        assert np.array_equal(t.float().cpu().numpy(), np.zeros(t.shape)), name
