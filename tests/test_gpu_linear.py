"""GPU parity of one Linear layer (forward and backward) against the oracle's
composition of the same steps: quantize (tensorwise or rowwise e4m3; e5m2 for the
gradient; per-column e4m3 for the transposed weight), then the fp64 GEMMs."""
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


def _ws(f, M, N, K, recipe):
    import torch
    return torch.empty(f.fp8_linear_ws_bytes(M, N, K, recipe), dtype=torch.uint8, device="cuda:0")


@pytest.mark.parametrize("fast", [True, False])
def test_linear_tensorwise_forward_fp32(f, fast):
    """256 x 512 input, 512 x 512 weight, one scale each, fp32 out; both accumulation
    modes (full precision meets the floored elementwise 2e-3 fp32 bar)."""
    import torch
    e4, _ = _names(f)
    w = synth.linear_tensorwise()
    x, wt = w.tensors["x"], w.tensors["w"]
    M, K, N = x.shape[0], x.shape[1], wt.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    f.fp8_linear_fwd(to_dev_bf16(x), to_dev_bf16(wt), f.RECIPE_TENSORWISE, EPS, f.OUT_F32, y,
                     _ws(f, M, N, K, f.RECIPE_TENSORWISE), use_fast_accum=fast)
    torch.cuda.synchronize()
    qx, _, ix = oracle.quant_tensor(x, e4, EPS)
    qw, _, iw = oracle.quant_tensor(wt, e4, EPS)
    ref = oracle.scaled_mm(qx, e4, qw, e4, oracle.SCALE_TENSOR, ix, iw)
    S = oracle.scaled_mm(qx, e4, qw, e4, oracle.SCALE_TENSOR, ix, iw, absolute=True)
    check_gemm(y.cpu().numpy(), ref, S, False, "tensorwise linear fwd (fp32 out)", exact=not fast)


@pytest.mark.parametrize("recipe,M,K,N", [(r, m, k, n) for r, m in (("rowwise", 200), ("rowwise", 201), ("tensorwise", 208))
                                           for k, n in ((384, 272), (256, 384))] +
                         [("rowwise", 2752, 384, 384), ("rowwise", 2753, 384, 272), ("tensorwise", 2752, 384, 384)])
def test_linear_small_fwd_bwd(f, recipe, M, K, N):
    """M about 200: outputs of at most 256 tiles of 64 x 64, so both GEMMs of the
    rowwise recipe take row-major weights (the small-output GEMM). M 2752 / 2753:
    more tiles, so the rowwise forward's weight goes k-packed (N % 16 == 0, K %
    128 == 0) and so does the backward's w^T when N % 128 == 0 (384; with 272 it
    stays row-major). Rowwise takes any M (201, 2753: odd, and the weight
    gradient's row count not a multiple of its 64-row pipeline step); the all-FP8
    tensorwise backward needs M % 16 == 0."""
    import torch
    e4, e5 = _names(f)
    x = synth.normal_bf16((M, K), 801, 1.0)
    synth.add_outliers(x, 802, 0.01, 50.0)
    wt = synth.normal_bf16((N, K), 803, 0.02)
    gy = synth.normal_bf16((M, N), 804, 1e-3)
    rc = f.RECIPE_ROWWISE_BF16_WGRAD if recipe == "rowwise" else f.RECIPE_TENSORWISE
    ws = _ws(f, M, N, K, rc)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    gx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    gw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda:0")
    xd, wd, gd = to_dev_bf16(x), to_dev_bf16(wt), to_dev_bf16(gy)
    f.fp8_linear_fwd(xd, wd, rc, EPS, f.OUT_BF16, y, ws)
    f.fp8_linear_bwd(gd, xd, wd, rc, EPS, gx, gw, ws)
    torch.cuda.synchronize()
    if recipe == "rowwise":
        qx, _, ix = oracle.quant_row(x, e4, EPS)
        qw, _, iw = oracle.quant_row(wt, e4, EPS)
        qg, _, ig = oracle.quant_row(gy, e5, EPS)
        qwt, _, iwc = oracle.quant_col(wt, e4, EPS)
        sk = oracle.SCALE_ROW
    else:
        qx, _, ix = oracle.quant_tensor(x, e4, EPS)
        qw, _, iw = oracle.quant_tensor(wt, e4, EPS)
        qg, _, ig = oracle.quant_tensor(gy, e5, EPS)
        qt, _, iwc = oracle.quant_tensor(wt, e4, EPS)
        qwt = np.ascontiguousarray(qt.T)
        sk = oracle.SCALE_TENSOR
    ref_y = oracle.scaled_mm(qx, e4, qw, e4, sk, ix, iw)
    S_y = oracle.scaled_mm(qx, e4, qw, e4, sk, ix, iw, absolute=True)
    ref_gx = oracle.scaled_mm(qg, e5, qwt, e4, sk, ig, iwc)
    S_gx = oracle.scaled_mm(qg, e5, qwt, e4, sk, ig, iwc, absolute=True)
    if recipe == "rowwise":
        ref_gw = oracle.wgrad_bf16(gy, x)
        S_gw = oracle.wgrad_bf16(gy, x, absolute=True)
    else:
        # all-FP8 grad-weight: (q(gy)^T * inv_g) (q(x)^T * inv_x)^T over m
        _, qgT, _, ig2, qxT, _, ix2 = oracle.quant_dual(gy, x, e5, e4, EPS)
        ref_gw = oracle.scaled_mm(qgT, e5, qxT, e4, sk, ig2, ix2)
        S_gw = oracle.scaled_mm(qgT, e5, qxT, e4, sk, ig2, ix2, absolute=True)
    # the forward runs the fast accumulation; both backward GEMMs full precision (the
    # BF16 grad-weight of the rowwise recipe sums at fp32 precision too)
    for name, got, ref, S, ex in (("y", y, ref_y, S_y, False), ("gx", gx, ref_gx, S_gx, True),
                                  ("gw", gw, ref_gw, S_gw, True)):
        check_gemm(got.float().cpu().numpy(), ref, S, True, f"{recipe} {name}", exact=ex)


@pytest.mark.parametrize("M,K,N,special", [(256, 512, 512, None), (2048, 1024, 1536, None),
                                           (8192, 4096, 1024, None), (48, 16, 8, None),
                                           (256, 512, 512, "zero_x"), (256, 512, 512, "inf_w"),
                                           (256, 512, 512, "nan_x")])
def test_linear_tensorwise_fwd_matches_separate_quantizers(f, M, K, N, special):
    """The tensorwise forward quantizes x and w in one amax launch (maxima per
    workgroup) and one cast launch; its output must equal, bit for bit, two
    fp8_quant_tensor calls (one atomic amax word each) followed by fp8_scaled_mm on
    the same shape: equal codes and inverse scales give the same GEMM. 8192 x 4096:
    x takes the full 2048 amax workgroups; 48 x 16 x 8: one workgroup each.
    Degenerate inputs: an all-zero x (amax 0: the eps-clamped scale), an infinity in
    w (scale 0, so inf * 0 codes and NaN outputs), NaNs in x (dropped by the amax,
    cast to NaN codes)."""
    import torch
    x = synth.normal_bf16((M, K), 811, 1.0)
    synth.add_outliers(x, 812, 0.001, 50.0)
    wt = synth.normal_bf16((N, K), 813, 0.02)
    xd, wd = to_dev_bf16(x), to_dev_bf16(wt)
    if special == "zero_x":
        xd.zero_()
    elif special == "inf_w":
        wd[3, 100] = float("inf")
    elif special == "nan_x":
        xd[7, 9] = float("nan")
        xd[200, 511] = float("nan")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_linear_fwd(xd, wd, f.RECIPE_TENSORWISE, EPS, f.OUT_BF16, y, _ws(f, M, N, K, f.RECIPE_TENSORWISE))
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda:0")
    qw = torch.empty((N, K), dtype=torch.uint8, device="cuda:0")
    sx, ix, sw, iw = (torch.empty(1, dtype=torch.float32, device="cuda:0") for _ in range(4))
    ws = torch.empty(f.fp8_quant_tensor_ws_bytes(), dtype=torch.uint8, device="cuda:0")
    f.fp8_quant_tensor(xd, f.E4M3_NATIVE, EPS, qx, sx, ix, ws)
    f.fp8_quant_tensor(wd, f.E4M3_NATIVE, EPS, qw, sw, iw, ws)
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_scaled_mm(qx, f.E4M3_NATIVE, qw, f.E4M3_NATIVE, f.SCALE_TENSOR, ix, iw, f.OUT_BF16, y2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_linear_tensorwise_bwd_needs_m_multiple_of_16(f):
    """The all-FP8 tensorwise backward contracts over m in FP8 (transposed
    operands of 16-row groups): M % 16 != 0 is refused before any launch."""
    import torch
    M, K, N = 200, 128, 64
    gy = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda:0")
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda:0")
    gx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    gw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(f.Fp8Error) as e:
        f.fp8_linear_bwd(gy, x, w, f.RECIPE_TENSORWISE, EPS, gx, gw, _ws(f, M, N, K, f.RECIPE_TENSORWISE))
    assert e.value.status == f.ERR_ALIGNMENT
