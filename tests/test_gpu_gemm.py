"""GPU parity of the FP8 GEMMs (dense, grouped; tensor, row, block, MX scales) and of the
BF16 weight-gradient GEMM against the oracle's fp64 products of the same quantized
operands. Acceptance (tests/gpu_util.check_gemm): normwise max relative error at most
1e-2 for bf16 output and 2e-3 for fp32 output, and every element within the
componentwise accumulation bound 2^-9 * sum|products| plus the output rounding. The
operands here are random codes over a format's whole range, the hardest case for the
matrix cores' internal accumulation."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (check_gemm, gpu, have_gpu, lib, to_dev, to_dev_bf16)

pytestmark = [gpu, pytest.mark.skipif(not have_gpu(), reason="needs an MI355X")]


@pytest.fixture(scope="module")
def f():
    oracle.build(force=False)
    synth.build(force=False)
    return lib()


def _names(f):
    e4, e5 = f.fp8_probe(0)
    name = {0: "e4m3fn", 1: "e4m3fnuz", 2: "e5m2", 3: "e5m2fnuz"}
    return name[e4], name[e5]


def _codes(name, shape, rng, lo=None):
    """Random finite codes of a format."""
    tab = oracle.decode(name, np.arange(256))
    ok = np.nonzero(np.isfinite(tab))[0]
    return rng.choice(ok, size=shape).astype(np.uint8)


def _out(shape, f32):
    import torch
    return torch.empty(shape, dtype=torch.float32 if f32 else torch.bfloat16, device="cuda:0")


def _host(out):
    return out.float().cpu().numpy().astype(np.float64)


# Zero rows appended to A so that the output has more than 256 tiles of 64 x 64
# (the dense GEMM's small-output form takes up to one such tile per compute
# unit): the padded calls run the 256 x 256 ping-pong kernel, the unpadded ones
# the small-output form, and the tests below pin both.
PAD_ROWS = 64 * 257


def _pad_rows(a, pad):
    if not pad:
        return a
    return np.concatenate([a, np.zeros((PAD_ROWS, a.shape[1]), a.dtype)], axis=0)


@pytest.mark.parametrize("pad", [False, True])
@pytest.mark.parametrize("fast", [True, False])
def test_code_pair_product_table(f, fast, pad):
    """The exhaustive code-pair table through the matrix cores: row a of A holds code a
    at all 128 K positions, row b of B code b, so out[a][b] = 128 dec(a) dec(b), exactly
    (equal products need no alignment; the value fits fp32), for every pair of finite
    codes: A in e4m3 and in e5m2, B in e4m3. Both accumulation modes, both dense
    kernels (pad: zero rows after the table, which must come out zero)."""
    import torch
    e4, e5 = _names(f)
    tb = oracle.decode(e4, np.arange(256))
    fb = np.isfinite(tb)
    b = np.repeat(np.where(fb, np.arange(256), 0).astype(np.uint8)[:, None], 128, axis=1)
    one = torch.ones(1, dtype=torch.float32, device="cuda:0")
    for fa, name in ((f.E4M3_NATIVE, e4), (f.E5M2_NATIVE, e5)):
        ta = oracle.decode(name, np.arange(256))
        fa_ok = np.isfinite(ta)
        a = _pad_rows(np.repeat(np.where(fa_ok, np.arange(256), 0).astype(np.uint8)[:, None], 128, axis=1), pad)
        out = _out((a.shape[0], 256), True)
        f.fp8_scaled_mm(to_dev(a), fa, to_dev(b), f.E4M3_NATIVE, f.SCALE_TENSOR, one, one, f.OUT_F32, out,
                        use_fast_accum=fast)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        want = 128.0 * np.outer(np.where(fa_ok, ta, 0.0), np.where(fb, tb, 0.0))
        assert np.array_equal(got[:256], want), (name, fast, int(np.sum(got[:256] != want)))
        assert not np.any(got[256:])


@pytest.mark.parametrize("pad", [False, True])
@pytest.mark.parametrize("fast", [True, False])
def test_matrix_core_decodes_every_code(f, fast, pad):
    """A has code c at k = 0 of row c (zeros elsewhere); B row 0 holds the code of 1.0.
    out[c][0] must be exactly the oracle's value of code c, for all finite codes, both
    formats on the A side and the e4m3 format on the B side; both accumulation modes
    (the full-precision one decodes the codes to bf16 with gfx950's converts), both
    dense kernels (pad: zero rows after the codes)."""
    import torch
    e4, e5 = _names(f)
    one_b = oracle.encode(e4, [1.0])[0]
    for fa, name in ((f.E4M3_NATIVE, e4), (f.E5M2_NATIVE, e5)):
        tab = oracle.decode(name, np.arange(256))
        a = np.zeros((256, 128), np.uint8)
        a[:, 0] = np.arange(256)
        fin = np.isfinite(tab)
        a[~fin, 0] = 0
        a = _pad_rows(a, pad)
        b = np.zeros((16, 128), np.uint8)
        b[0, 0] = one_b
        out = _out((a.shape[0], 16), True)
        one = torch.ones(1, dtype=torch.float32, device="cuda:0")
        f.fp8_scaled_mm(to_dev(a), fa, to_dev(b), f.E4M3_NATIVE, f.SCALE_TENSOR, one, one, f.OUT_F32, out,
                        use_fast_accum=fast)
        torch.cuda.synchronize()
        got = out.cpu().numpy()[:256, 0].astype(np.float64)
        assert np.array_equal(got[fin], tab[fin]), name
        assert np.all(out.cpu().numpy()[:, 1:] == 0) and not np.any(out.cpu().numpy()[256:])
    # and e4m3 codes on the B side
    tab = oracle.decode(e4, np.arange(256))
    fin = np.isfinite(tab)
    b = np.zeros((256, 128), np.uint8)
    b[:, 0] = np.where(fin, np.arange(256), 0)
    a = _pad_rows(np.zeros((16, 128), np.uint8), pad)
    a[0, 0] = one_b
    out = _out((a.shape[0], 256), True)
    one = torch.ones(1, dtype=torch.float32, device="cuda:0")
    f.fp8_scaled_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, f.SCALE_TENSOR, one, one, f.OUT_F32, out,
                    use_fast_accum=fast)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy()[0].astype(np.float64)[fin], tab[fin])


def test_small_integer_products_are_exact(f):
    """Small-integer operands with unit scales: the fp32 result is exact."""
    import torch
    e4, _ = _names(f)
    rng = np.random.default_rng(1)
    M, N, K = 96, 80, 512
    av = rng.integers(-4, 5, (M, K)).astype(np.float32)
    bv = rng.integers(-4, 5, (N, K)).astype(np.float32)
    a, b = oracle.encode(e4, av), oracle.encode(e4, bv)
    out = _out((M, N), True)
    one = torch.ones(1, dtype=torch.float32, device="cuda:0")
    f.fp8_scaled_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, f.SCALE_TENSOR, one, one, f.OUT_F32, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), av.astype(np.float64) @ bv.T.astype(np.float64))


# up to 256 output tiles of 64 x 64: the small-output form; more: the ping-pong
# kernel where K % 128 == 0 (1100 x 1040: 306 tiles, ragged in both), else the
# generic 128 x 128 tiles (1100 x 1040 x 272)
@pytest.mark.parametrize("M,N,K", [(256, 512, 512), (1, 16, 16), (100, 72, 48), (300, 200, 384), (513, 260, 1040),
                                   (300, 520, 1152), (64, 64, 128), (200, 136, 256), (1024, 1024, 256),
                                   (1100, 1040, 384), (1100, 1040, 272), (2100, 8200, 128)])
@pytest.mark.parametrize("scaling", ["tensor", "row"])
@pytest.mark.parametrize("out_f32", [True, False])
@pytest.mark.parametrize("fast", [True, False])
def test_scaled_mm(f, M, N, K, scaling, out_f32, fast):
    import torch
    e4, _ = _names(f)
    rng = np.random.default_rng(M * 7 + N)
    a, b = _codes(e4, (M, K), rng), _codes(e4, (N, K), rng)
    if scaling == "tensor":
        sa, sb, sk = np.float32([0.37]), np.float32([2.5]), f.SCALE_TENSOR
    else:
        sa = rng.uniform(0.01, 3, M).astype(np.float32)
        sb = rng.uniform(0.01, 3, N).astype(np.float32)
        sk = f.SCALE_ROW
    out = _out((M, N), out_f32)
    f.fp8_scaled_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, sk, to_dev(sa), to_dev(sb),
                    f.OUT_F32 if out_f32 else f.OUT_BF16, out, use_fast_accum=fast)
    torch.cuda.synchronize()
    osk = oracle.SCALE_TENSOR if scaling == "tensor" else oracle.SCALE_ROW
    ref = oracle.scaled_mm(a, e4, b, e4, osk, sa, sb)
    S = oracle.scaled_mm(a, e4, b, e4, osk, sa, sb, absolute=True)
    check_gemm(_host(out), ref, S, not out_f32, f"scaled_mm {M}x{N}x{K} {scaling}", exact=not fast)


def test_scaled_mm_e5m2_a(f):
    """Grad-input shape: e5m2 A (a gradient) x e4m3 B."""
    import torch
    e4, e5 = _names(f)
    rng = np.random.default_rng(3)
    M, N, K = 192, 320, 640
    a, b = _codes(e5, (M, K), rng), _codes(e4, (N, K), rng)
    # keep magnitudes moderate so fp32 accumulation stays well inside range
    a = np.where(np.abs(oracle.decode(e5, a)) > 1024, 0, a).astype(np.uint8)
    sa = rng.uniform(0.5, 2, M).astype(np.float32)
    sb = rng.uniform(0.5, 2, N).astype(np.float32)
    out = _out((M, N), False)
    f.fp8_scaled_mm(to_dev(a), f.E5M2_NATIVE, to_dev(b), f.E4M3_NATIVE, f.SCALE_ROW, to_dev(sa), to_dev(sb),
                    f.OUT_BF16, out)
    torch.cuda.synchronize()
    ref = oracle.scaled_mm(a, e5, b, e4, oracle.SCALE_ROW, sa, sb)
    S = oracle.scaled_mm(a, e5, b, e4, oracle.SCALE_ROW, sa, sb, absolute=True)
    check_gemm(_host(out), ref, S, True, "e5m2 x e4m3")


def test_scale_direction_negative(f):
    """Passing the quantize multipliers instead of their inverses is off by (s_a s_b)^2."""
    import torch
    e4, _ = _names(f)
    rng = np.random.default_rng(4)
    a, b = _codes(e4, (64, 128), rng), _codes(e4, (32, 128), rng)
    good, bad = _out((64, 32), True), _out((64, 32), True)
    inv_a, inv_b = torch.tensor([0.125], device="cuda:0"), torch.tensor([4.0], device="cuda:0")
    f.fp8_scaled_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, f.SCALE_TENSOR, inv_a, inv_b, f.OUT_F32, good)
    f.fp8_scaled_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, f.SCALE_TENSOR, 1 / inv_a, 1 / inv_b,
                    f.OUT_F32, bad)
    torch.cuda.synchronize()
    g, w = good.cpu().numpy(), bad.cpu().numpy()
    nz = g != 0
    np.testing.assert_allclose(w[nz] / g[nz], (8.0 * 0.25) ** 2, rtol=1e-6)


def _offsets(counts):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return off


@pytest.mark.parametrize("counts,N,K", [([37, 0, 300, 1, 0, 513], 272, 384), ([0, 0, 64], 128, 128),
                                         ([256], 256, 256), ([5] * 40, 64, 512), ([300, 5, 0, 129], 320, 640),
                                         ([17], 64, 128), ([600, 0, 3], 512, 1152)])
@pytest.mark.parametrize("fast", [True, False])
def test_grouped_row(f, counts, N, K, fast):
    import torch
    e4, _ = _names(f)
    rng = np.random.default_rng(sum(counts) + N)
    off = _offsets(counts)
    E, Mt = len(counts), int(off[-1])
    a, b = _codes(e4, (Mt, K), rng), _codes(e4, (E, N, K), rng)
    sa = rng.uniform(0.1, 2, Mt).astype(np.float32)
    sb = rng.uniform(0.1, 2, (E, N)).astype(np.float32)
    out = torch.full((Mt, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_grouped_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, f.SCALE_ROW, to_dev(sa), to_dev(sb),
                     to_dev(off), f.OUT_BF16, out, use_fast_accum=fast)
    torch.cuda.synchronize()
    ref = oracle.grouped_mm(a, e4, b, e4, oracle.SCALE_ROW, sa, sb, off)
    S = oracle.grouped_mm(a, e4, b, e4, oracle.SCALE_ROW, sa, sb, off, absolute=True)
    got = _host(out)
    assert not np.any(np.isnan(got)), "rows left unwritten"
    check_gemm(got, ref, S, True, f"grouped row {counts}", exact=not fast)


@pytest.mark.parametrize("counts,N,K,out_f32,shift", [([100, 0, 200, 7], 256, 384, False, 0),
                                                       ([512, 512], 128, 256, False, 0),
                                                       ([64], 128, 128, False, 0),
                                                       ([300, 5, 0, 129], 384, 640, True, 0),
                                                       ([4096, 4096], 2304, 128, False, 0),
                                                       ([64], 256, 512, False, 0),
                                                       ([300, 5, 0, 129], 384, 1024, False, 0),
                                                       ([600, 0, 3], 512, 2048, True, 0),
                                                       ([1000, 24], 640, 1536, False, 0),
                                                       ([300, 5, 0, 129], 384, 1024, False, 4),
                                                       ([600, 0, 3], 512, 1152, False, 0)])
@pytest.mark.parametrize("fast", [True, False])
def test_grouped_block(f, counts, N, K, out_f32, shift, fast):
    """One K block (no prefetch), an odd number of K blocks, a partial B tile and fp32
    output, and more tiles than workgroups (each walks several, reusing its LDS slots).
    K % 512 == 0 with 16-byte aligned scales takes the kernel's loads of four K blocks'
    scales at a time; other K, or scales at a 4-byte offset (shift), one K block's."""
    import torch
    e4, _ = _names(f)
    rng = np.random.default_rng(11)
    off = _offsets(counts)
    E, Mt = len(counts), int(off[-1])
    a, b = _codes(e4, (Mt, K), rng), _codes(e4, (E, N, K), rng)
    sa = rng.uniform(0.01, 4, (Mt, K // 128)).astype(np.float32)
    sb = rng.uniform(0.01, 4, (E, N // 128, K // 128)).astype(np.float32)
    out = _out((Mt, N), out_f32)

    def shifted(x):
        # the same floats at a device address `shift` bytes past a 256-byte boundary
        buf = torch.zeros(x.size + 64, dtype=torch.float32, device="cuda:0")
        v = buf[shift // 4:shift // 4 + x.size]
        v.copy_(torch.from_numpy(x.reshape(-1)).to("cuda:0"))
        return v
    f.fp8_grouped_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, f.SCALE_BLOCK128, shifted(sa), shifted(sb),
                     to_dev(off), f.OUT_F32 if out_f32 else f.OUT_BF16, out, use_fast_accum=fast)
    torch.cuda.synchronize()
    ref = oracle.grouped_mm(a, e4, b, e4, oracle.SCALE_BLOCK128, sa, sb, off)
    S = oracle.grouped_mm(a, e4, b, e4, oracle.SCALE_BLOCK128, sa, sb, off, absolute=True)
    check_gemm(_host(out), ref, S, not out_f32, f"grouped block {counts} K={K}", exact=not fast)


@pytest.mark.parametrize("counts,N,K,shift", [([100, 0, 200, 7], 256, 384, 0), ([512, 512], 128, 256, 0),
                                               ([33], 48, 96, 0), ([300, 5, 0, 129], 320, 640, 0),
                                               ([64], 192, 128, 0), ([600, 0, 3], 512, 1152, 0),
                                               ([300, 5, 0, 129], 320, 1024, 0), ([64], 192, 512, 0),
                                               ([600, 0, 3], 512, 2048, 0), ([300, 5, 0, 129], 320, 1024, 4),
                                               ([1536, 1536], 6144, 512, 0)])
@pytest.mark.parametrize("fast", [True, False])
def test_grouped_mx(f, counts, N, K, shift, fast):
    """K % 512 == 0 with 16-byte aligned scales takes the kernel's 16-bytes-per-row
    scale loads; other K, or scales at a 4-byte offset (shift), the dword loads."""
    import torch
    e4, _ = _names(f)
    rng = np.random.default_rng(13)
    off = _offsets(counts)
    E, Mt = len(counts), int(off[-1])
    a, b = _codes(e4, (Mt, K), rng), _codes(e4, (E, N, K), rng)
    sa = rng.integers(117, 137, (Mt, K // 32)).astype(np.uint8)
    sb = rng.integers(117, 137, (E, N, K // 32)).astype(np.uint8)
    out = _out((Mt, N), False)

    def shifted(x):
        # the same bytes at a device address `shift` bytes past a 256-byte boundary
        buf = torch.zeros(x.size + 256, dtype=torch.uint8, device="cuda:0")
        v = buf[shift:shift + x.size]
        v.copy_(to_dev(x).reshape(-1))
        return v
    f.fp8_grouped_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, f.SCALE_MX32, shifted(sa), shifted(sb),
                     to_dev(off), f.OUT_BF16, out, use_fast_accum=fast)
    torch.cuda.synchronize()
    ref = oracle.grouped_mm(a, e4, b, e4, oracle.SCALE_MX32, sa, sb, off)
    S = oracle.grouped_mm(a, e4, b, e4, oracle.SCALE_MX32, sa, sb, off, absolute=True)
    check_gemm(_host(out), ref, S, True, f"grouped mx {counts}", exact=not fast)


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (100, 264, 136), (1000, 512, 256), (7, 16, 8), (128, 264, 136),
                                   (640, 520, 264), (1024, 256, 256)])
def test_wgrad_bf16(f, M, N, K):
    import torch
    g = synth.normal_bf16((M, N), 700 + M, 1e-3)
    x = synth.normal_bf16((M, K), 701 + M, 1.0)
    gw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_wgrad_bf16(to_dev_bf16(g), to_dev_bf16(x), gw)
    torch.cuda.synchronize()
    ref = oracle.wgrad_bf16(g, x)
    S = oracle.wgrad_bf16(g, x, absolute=True)
    check_gemm(_host(gw), ref, S, True, f"wgrad {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(64, 16632, 904), (128, 22784, 1024)])
def test_wgrad_bf16_leftover_half_tiles(f, M, N, K):
    """More 256 x 256 tiles than workgroups with at most half a round left over
    (260 tiles with ragged last row and column tiles, and 356 tiles, on 256 CUs):
    the leftover tiles run as 128-column halves in a second launch."""
    import torch
    g = synth.normal_bf16((M, N), 720 + M, 1e-3)
    x = synth.normal_bf16((M, K), 721 + M, 1.0)
    gw = torch.full((N, K), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_wgrad_bf16(to_dev_bf16(g), to_dev_bf16(x), gw)
    torch.cuda.synchronize()
    ref = oracle.wgrad_bf16(g, x)
    S = oracle.wgrad_bf16(g, x, absolute=True)
    check_gemm(_host(gw), ref, S, True, f"wgrad halves {M}x{N}x{K}")


@pytest.mark.parametrize("counts,N,K", [([37, 0, 300, 1, 0, 513], 264, 136), ([64], 256, 256), ([0, 0], 64, 64),
                                         ([5] * 40, 64, 512), ([600, 0, 3], 520, 264),
                                         ([32, 31, 33, 95, 96, 97, 128], 128, 136)])
def test_grouped_wgrad_bf16(f, counts, N, K):
    """Expert row ranges shorter than one 32-row stage, on stage boundaries and
    ragged; empty experts must come out exactly zero."""
    import torch
    off = _offsets(counts)
    E, Mt = len(counts), int(off[-1])
    g = synth.normal_bf16((max(Mt, 1), N), 900 + E, 1e-3)[:Mt]
    x = synth.normal_bf16((max(Mt, 1), K), 901 + E, 1.0)[:Mt]
    gw = torch.full((E, N, K), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    gd = to_dev_bf16(np.ascontiguousarray(g)) if Mt else torch.empty((0, N), dtype=torch.bfloat16, device="cuda:0")
    xd = to_dev_bf16(np.ascontiguousarray(x)) if Mt else torch.empty((0, K), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_grouped_wgrad_bf16(gd, xd, to_dev(off), gw)
    torch.cuda.synchronize()
    got = gw.float().cpu().numpy()
    ref = oracle.grouped_wgrad_bf16(g, x, off)
    S = oracle.grouped_wgrad_bf16(g, x, off, absolute=True)
    for e, c in enumerate(counts):
        if c == 0:
            assert np.all(got[e] == 0.0), f"expert {e} (empty) not zero"
        else:
            check_gemm(got[e], ref[e], S[e], True, f"grouped wgrad expert {e} ({c} rows)")
