"""GPU parity of the packed-operand paths: fp8_quant_row_kpacked / fp8_quant_col_kpacked /
fp8_quant_mx_kpacked write the oracle's codes (bit-exact) permuted into 1 KB chunks of 16
rows x 64 columns, fp8_quant_row_kpaired / fp8_quant_mx_kpaired into pair-interleaved
rows, and the k-packed GEMMs on those give
the oracle's products (to the GEMM bar of tests/gpu_util.check_gemm) and the same bits
as the row-major GEMMs. The permutation (tests/gpu_util.kpack) is numpy reshapes of the layout
the header states; nothing of it is shared with the library."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (check_gemm, check_guard, empty_u8, gpu, have_gpu, kpack, lib, to_dev, to_dev_bf16,
                             u8)

pytestmark = [gpu, pytest.mark.skipif(not have_gpu(), reason="needs an MI355X")]

EPS = 1e-12


@pytest.fixture(scope="module")
def f():
    oracle.build(force=False)
    synth.build(force=False)
    return lib()


def _natives(f):
    e4, e5 = f.fp8_probe(0)
    name = {0: "e4m3fn", 1: "e4m3fnuz", 2: "e5m2", 3: "e5m2fnuz"}
    return [(f.E4M3_NATIVE, name[e4]), (f.E5M2_NATIVE, name[e5])]


@pytest.mark.parametrize("shape", [(16, 64), (48, 7168), (2, 32, 192), (3, 16, 2112), (64, 16384), (160, 512),
                                   (4, 48, 4160)])
def test_quant_row_kpacked(f, shape):
    import torch
    x = synth.normal_bf16(shape, 900 + shape[-1], 1.0)
    # an all-zero row (eps clamp) and a row with one large outlier
    x.reshape(-1, shape[-1])[3] = 0
    x.reshape(-1, shape[-1])[5, 7] = 0x4700  # 32768.0
    n = int(np.prod(shape))
    for fmt, name in _natives(f):
        print("row kpacked", shape, name, flush=True)
        q, full = empty_u8((n,), 256)
        s = torch.empty(shape[:-1], dtype=torch.float32, device="cuda:0")
        i = torch.empty_like(s)
        f.fp8_quant_row_kpacked(to_dev_bf16(x), fmt, EPS, q, s, i)
        torch.cuda.synchronize()
        check_guard(full, 256)
        rq, rs, ri = oracle.quant_row(x, name, EPS)
        assert np.array_equal(u8(q), kpack(rq))
        assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)


@pytest.mark.parametrize("g", [16, 2])
@pytest.mark.parametrize("shape", [(16, 64), (48, 5120), (2, 32, 192), (3, 16, 1088), (64, 7168), (2, 96, 4160)])
def test_quant_mx_packed(f, shape, g):
    """Codes and E8M0 bytes of fp8_quant_mx, the codes permuted into the packed layout:
    a column count that is not a multiple of a workgroup tile (128 or 1024 columns),
    batches, an all-zero group and a large outlier, both rounding modes of the scale."""
    import torch
    x = synth.normal_bf16(shape, 930 + shape[-1] + g, 1.0)
    x.reshape(-1, shape[-1])[3, 32:64] = 0   # an all-zero group (eps clamp)
    x.reshape(-1, shape[-1])[5, 7] = 0x4700  # 32768.0
    n = int(np.prod(shape))
    fn = f.fp8_quant_mx_kpacked if g == 16 else f.fp8_quant_mx_kpaired
    for mode in (f.MX_POW2_FLOOR, f.MX_OCP):
        for fmt, name in _natives(f):
            print("mx packed", g, shape, mode, name, flush=True)
            q, full = empty_u8((n,), 256)
            e = torch.empty(shape[:-1] + (shape[-1] // 32,), dtype=torch.uint8, device="cuda:0")
            fn(to_dev_bf16(x), fmt, mode, EPS, q, e)
            torch.cuda.synchronize()
            check_guard(full, 256)
            rq, re = oracle.quant_mx(x, name, mode, EPS)
            assert np.array_equal(u8(q), kpack(rq, g))
            assert np.array_equal(u8(e), re)


def _offsets(counts):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return off


def _codes(name, shape, rng):
    tab = oracle.decode(name, np.arange(256))
    ok = np.nonzero(np.isfinite(tab))[0]
    return rng.choice(ok, size=shape).astype(np.uint8)


@pytest.mark.parametrize("counts,N,K,scaling,out_f32", [
    ([37, 0, 300, 1, 0, 514], 272, 384, "row", False),   # N past a whole tile, empty experts, odd starts
    ([0, 0, 64], 128, 128, "row", False),                 # two stages
    ([300, 5, 0, 129], 320, 640, "row", True),            # fp32 out
    ([600, 0, 4], 512, 1152, "row", False),
    ([4096, 4096], 2304, 128, "row", False),              # more tiles than workgroups
    ([101, 0, 200, 7], 256, 384, "mx", False),            # dword scale loads, odd starts
    ([300, 5, 0, 129], 320, 1024, "mx", False),           # 16-byte scale loads
    ([1536, 1536], 6144, 512, "mx", False),
])
def test_grouped_mm_kpacked(f, counts, N, K, scaling, out_f32):
    import torch
    e4 = _natives(f)[0][1]
    rng = np.random.default_rng(17 + N + K)
    off = _offsets(counts)
    E, Mt = len(counts), int(off[-1])
    a, b = _codes(e4, (Mt, K), rng), _codes(e4, (E, N, K), rng)
    if scaling == "row":
        sk, osk = f.SCALE_ROW, oracle.SCALE_ROW
        sa = rng.uniform(0.1, 2, Mt).astype(np.float32)
        sb = rng.uniform(0.1, 2, (E, N)).astype(np.float32)
    else:
        sk, osk = f.SCALE_MX32, oracle.SCALE_MX32
        sa = rng.integers(117, 137, (Mt, K // 32)).astype(np.uint8)
        sb = rng.integers(117, 137, (E, N, K // 32)).astype(np.uint8)
    dt = torch.float32 if out_f32 else torch.bfloat16
    ot = f.OUT_F32 if out_f32 else f.OUT_BF16
    print("grouped kpacked", counts, N, K, scaling, flush=True)
    y_rm = torch.full((Mt, N), float("nan"), dtype=dt, device="cuda:0")
    y_pk = torch.full((Mt, N), float("nan"), dtype=dt, device="cuda:0")
    da, dsa, dsb, doff = to_dev(a), to_dev(sa), to_dev(sb), to_dev(off)
    f.fp8_grouped_mm(da, f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, sk, dsa, dsb, doff, ot, y_rm)
    bp = to_dev(kpack(b)).reshape(E, -1)
    ap = to_dev(kpack(a, 2)).reshape(Mt, K)
    f.fp8_grouped_mm_kpacked(ap, f.E4M3_NATIVE, bp, f.E4M3_NATIVE, sk, dsa, dsb, doff, ot, y_pk, N)
    torch.cuda.synchronize()
    got = y_pk.float().cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(got)), "rows left unwritten"
    # the same kernel arithmetic in the same order: identical bits
    assert torch.equal(y_pk.view(torch.int16 if not out_f32 else torch.int32),
                       y_rm.view(torch.int16 if not out_f32 else torch.int32))
    ref = oracle.grouped_mm(a, e4, b, e4, osk, sa, sb, off)
    S = oracle.grouped_mm(a, e4, b, e4, osk, sa, sb, off, absolute=True)
    check_gemm(got, ref, S, not out_f32, f"grouped kpacked {counts} {scaling}")


def test_quant_then_gemm_kpacked(f):
    """The MoE layer's path: rowwise e4m3 quantization of the activations into the
    pair-interleaved layout and of W [E][N][K] into the k-packed one, then the grouped
    GEMM on both."""
    import torch
    e4 = _natives(f)[0][1]
    counts = [200, 0, 77, 301]
    E, N, K = len(counts), 256, 512
    off = _offsets(counts)
    Mt = int(off[-1])
    w = synth.normal_bf16((E, N, K), 910, 0.02)
    xa = synth.normal_bf16((Mt, K), 911, 1.0)
    qa, sa, ia = oracle.quant_row(xa, e4, EPS)
    rq, rs, ri = oracle.quant_row(w, e4, EPS)
    qap = torch.empty((Mt, K), dtype=torch.uint8, device="cuda:0")
    sap, iap = (torch.empty(Mt, dtype=torch.float32, device="cuda:0") for _ in range(2))
    f.fp8_quant_row_kpaired(to_dev_bf16(xa), f.E4M3_NATIVE, EPS, qap, sap, iap)
    qw = torch.empty(E * N * K, dtype=torch.uint8, device="cuda:0").reshape(E, -1)
    sw = torch.empty((E, N), dtype=torch.float32, device="cuda:0")
    iw = torch.empty_like(sw)
    f.fp8_quant_row_kpacked(to_dev_bf16(w), f.E4M3_NATIVE, EPS, qw, sw, iw)
    y = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_grouped_mm_kpacked(qap, f.E4M3_NATIVE, qw, f.E4M3_NATIVE, f.SCALE_ROW, iap, iw, to_dev(off),
                             f.OUT_BF16, y, N)
    torch.cuda.synchronize()
    assert np.array_equal(u8(qap).reshape(-1), kpack(qa, 2)) and np.array_equal(iap.cpu().numpy(), ia)
    assert np.array_equal(u8(qw).reshape(-1), kpack(rq))
    assert np.array_equal(iw.cpu().numpy(), ri)
    ref = oracle.grouped_mm(qa, e4, rq, e4, oracle.SCALE_ROW, ia, ri, off)
    S = oracle.grouped_mm(qa, e4, rq, e4, oracle.SCALE_ROW, ia, ri, off, absolute=True)
    check_gemm(y.float().cpu().numpy().astype(np.float64), ref, S, True, "quant + grouped kpacked")


@pytest.mark.parametrize("shape", [(128, 64), (2, 256, 48), (2048, 144), (4096, 128), (2112, 64),
                                   (1024, 2112, 64), (14336, 128), (3, 8192, 80), (16448, 64)])
def test_quant_col_kpacked(f, shape):
    """The three column paths: up to 2048 rows in registers, the split form (column amax
    over row chunks, then the cast) and the fused two-read form (many strips)."""
    import torch
    x = synth.normal_bf16(shape, 920 + shape[-2], 0.02)
    x.reshape(-1, shape[-1])[:, 3] = 0  # an all-zero column
    b = 1 if len(shape) == 2 else shape[0]
    R, C = shape[-2], shape[-1]
    for fmt, name in _natives(f):
        print("col kpacked", shape, name, flush=True)
        q, full = empty_u8((b * R * C,), 256)
        s = torch.empty(shape[:-2] + (C,), dtype=torch.float32, device="cuda:0")
        i = torch.empty_like(s)
        ws = torch.empty(max(f.fp8_quant_col_ws_bytes(b, R, C), 4), dtype=torch.uint8, device="cuda:0")
        f.fp8_quant_col_kpacked(to_dev_bf16(x), fmt, EPS, q, s, i, ws)
        torch.cuda.synchronize()
        check_guard(full, 256)
        rq, rs, ri = oracle.quant_col(x, name, EPS)
        assert np.array_equal(u8(q), kpack(rq))
        assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)


@pytest.mark.parametrize("M,N,K,scaling,out_f32", [(256, 512, 512, "tensor", False), (256, 512, 512, "row", False),
                                                   (300, 208, 384, "row", True), (513, 272, 1152, "row", False),
                                                   (2100, 8192, 128, "row", False)])
def test_scaled_mm_kpacked(f, M, N, K, scaling, out_f32):
    import torch
    e4 = _natives(f)[0][1]
    rng = np.random.default_rng(M + N + K)
    a, b = _codes(e4, (M, K), rng), _codes(e4, (N, K), rng)
    if scaling == "tensor":
        sa, sb, sk, osk = np.float32([0.37]), np.float32([2.5]), f.SCALE_TENSOR, oracle.SCALE_TENSOR
    else:
        sa = rng.uniform(0.01, 3, M).astype(np.float32)
        sb = rng.uniform(0.01, 3, N).astype(np.float32)
        sk, osk = f.SCALE_ROW, oracle.SCALE_ROW
    dt = torch.float32 if out_f32 else torch.bfloat16
    ot = f.OUT_F32 if out_f32 else f.OUT_BF16
    print("scaled_mm kpacked", M, N, K, scaling, flush=True)
    y_rm = torch.full((M, N), float("nan"), dtype=dt, device="cuda:0")
    y_pk = torch.full((M, N), float("nan"), dtype=dt, device="cuda:0")
    da, dsa, dsb = to_dev(a), to_dev(sa), to_dev(sb)
    f.fp8_scaled_mm(da, f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, sk, dsa, dsb, ot, y_rm)
    f.fp8_scaled_mm_kpacked(da, f.E4M3_NATIVE, to_dev(kpack(b)), f.E4M3_NATIVE, sk, dsa, dsb, ot, y_pk, N)
    torch.cuda.synchronize()
    got = y_pk.float().cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(got))
    iv = torch.int32 if out_f32 else torch.int16
    assert torch.equal(y_pk.view(iv), y_rm.view(iv))
    ref = oracle.scaled_mm(a, e4, b, e4, osk, sa, sb)
    S = oracle.scaled_mm(a, e4, b, e4, osk, sa, sb, absolute=True)
    check_gemm(got, ref, S, not out_f32, f"scaled_mm kpacked {M}x{N}x{K} {scaling}")


@pytest.mark.parametrize("shape", [(2, 64), (98, 7168), (2, 6, 192), (64, 16384), (3, 10, 4160), (6, 2048),
                                   (2, 10, 4096), (3, 4, 576)])
def test_quant_row_kpaired(f, shape):
    """A wavefront per row up to 4096 columns (a pair's two rows in one workgroup; 6 rows:
    the last workgroup holds a single pair), a workgroup per row beyond."""
    import torch
    x = synth.normal_bf16(shape, 930 + shape[-1], 1.0)
    x.reshape(-1, shape[-1])[1] = 0
    n = int(np.prod(shape))
    for fmt, name in _natives(f):
        print("row kpaired", shape, name, flush=True)
        q, full = empty_u8((n,), 256)
        s = torch.empty(shape[:-1], dtype=torch.float32, device="cuda:0")
        i = torch.empty_like(s)
        f.fp8_quant_row_kpaired(to_dev_bf16(x), fmt, EPS, q, s, i)
        torch.cuda.synchronize()
        check_guard(full, 256)
        rq, rs, ri = oracle.quant_row(x, name, EPS)
        assert np.array_equal(u8(q), kpack(rq, 2))
        assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)
