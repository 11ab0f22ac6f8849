"""Float8Linear through autograd on the GPU: output and both gradients against the
oracle's composition of the same steps (quantize, fp64 GEMMs), for both recipes,
with a batched input and a bias."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gemm, gpu, have_gpu, lib, to_dev_bf16

pytestmark = [gpu, pytest.mark.skipif(not have_gpu(), reason="needs an MI355X")]
EPS = 1e-12


@pytest.fixture(scope="module")
def f():
    oracle.build(force=False)
    synth.build(force=False)
    return lib()


def _names(f):
    e4, e5 = f.fp8_probe(0)
    name = {0: "e4m3fn", 1: "e4m3fnuz", 2: "e5m2", 3: "e5m2fnuz"}
    return name[e4], name[e5]


@pytest.mark.parametrize("recipe", ["rowwise", "tensorwise"])
def test_float8_linear_autograd(f, recipe):
    import torch
    from fp8_dynamic_scaling_amd.nn import Float8Linear
    e4, e5 = _names(f)
    B, T, K, N = 2, 104, 384, 272
    M = B * T
    x = synth.normal_bf16((M, K), 811, 1.0)
    wt = synth.normal_bf16((N, K), 812, 0.02)
    gy = synth.normal_bf16((M, N), 813, 1e-3)
    layer = Float8Linear(K, N, bias=True, recipe=recipe, device="cuda:0")
    with torch.no_grad():
        layer.weight.copy_(to_dev_bf16(wt))
        layer.bias.zero_()
    xd = to_dev_bf16(x).reshape(B, T, K).clone().requires_grad_(True)
    y = layer(xd)
    assert y.shape == (B, T, N) and y.dtype == torch.bfloat16
    y.backward(to_dev_bf16(gy).reshape(B, T, N))
    torch.cuda.synchronize()
    if recipe == "rowwise":
        qx, _, ix = oracle.quant_row(x, e4, EPS)
        qw, _, iw = oracle.quant_row(wt, e4, EPS)
        qg, _, ig = oracle.quant_row(gy, e5, EPS)
        qwt, _, iwc = oracle.quant_col(wt, e4, EPS)
        sk = oracle.SCALE_ROW
        ref_gw = oracle.wgrad_bf16(gy, x)
        S_gw = oracle.wgrad_bf16(gy, x, absolute=True)
    else:
        qx, _, ix = oracle.quant_tensor(x, e4, EPS)
        qw, _, iw = oracle.quant_tensor(wt, e4, EPS)
        qg, qgT, _, ig, qxT, _, ix2 = oracle.quant_dual(gy, x, e5, e4, EPS)
        qt, _, iwc = oracle.quant_tensor(wt, e4, EPS)
        qwt = np.ascontiguousarray(qt.T)
        sk = oracle.SCALE_TENSOR
        ref_gw = oracle.scaled_mm(qgT, e5, qxT, e4, sk, ig, ix2)
        S_gw = oracle.scaled_mm(qgT, e5, qxT, e4, sk, ig, ix2, absolute=True)
    ref_y = oracle.scaled_mm(qx, e4, qw, e4, sk, ix, iw)
    S_y = oracle.scaled_mm(qx, e4, qw, e4, sk, ix, iw, absolute=True)
    ref_gx = oracle.scaled_mm(qg, e5, qwt, e4, sk, ig, iwc)
    S_gx = oracle.scaled_mm(qg, e5, qwt, e4, sk, ig, iwc, absolute=True)
    # forward: fast accumulation; backward: full precision
    check_gemm(y.detach().reshape(M, N).float().cpu().numpy(), ref_y, S_y, True, f"{recipe} y")
    check_gemm(xd.grad.reshape(M, K).float().cpu().numpy(), ref_gx, S_gx, True, f"{recipe} grad x", exact=True)
    check_gemm(layer.weight.grad.float().cpu().numpy(), ref_gw, S_gw, True, f"{recipe} grad w", exact=True)
    # the bias gradient is the plain sum over rows (autograd's own add)
    np.testing.assert_allclose(layer.bias.grad.float().cpu().numpy(),
                               oracle.bf16_to_f32(gy).astype(np.float64).sum(0), rtol=2e-2, atol=1e-4)


def test_float8_linear_from_linear(f):
    import torch
    from fp8_dynamic_scaling_amd.nn import Float8Linear
    lin = torch.nn.Linear(256, 128, bias=False, device="cuda:0", dtype=torch.bfloat16)
    m = Float8Linear.from_linear(lin, recipe="rowwise")
    assert torch.equal(m.weight, lin.weight)
    x = torch.randn(64, 256, device="cuda:0").to(torch.bfloat16)
    y8, y16 = m(x).float(), lin(x).float()
    # FP8 rowwise against the bf16 matmul: within the e4m3 quantization error
    assert (y8 - y16).norm() / y16.norm() < 0.05
