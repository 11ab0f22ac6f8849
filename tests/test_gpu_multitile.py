"""GPU parity of the FP8 GEMMs where every workgroup of the persistent grid takes several
output tiles: more 256 x 256 tiles than the 256 workgroups, ragged last row and column
tiles, ragged experts (one empty, one of a single row), and K of 19 to 24 64-deep stages
(deep enough that the tiles' stage rings wrap many times). Every output element is
compared with the oracle, so a tile written to the wrong place, a tile lost, or a stale
accumulator or scale carried from one tile into the next shows. Row-major and packed
operands; rowwise, tensorwise and MX scales; dense and grouped."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gemm, gpu, have_gpu, kpack, lib, to_dev

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


def _codes(name, shape, rng):
    tab = oracle.decode(name, np.arange(256))
    ok = np.nonzero(np.isfinite(tab))[0]
    return rng.choice(ok, size=shape).astype(np.uint8)


def _offsets(counts):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return off


def _nan_out(shape):
    import torch
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")


@pytest.mark.parametrize("M,N,K,scaling", [(6104, 8184, 1280, "row"), (4100, 4360, 1344, "tensor"),
                                           (2312, 28680, 1216, "row")])
def test_dense_multi_tile(f, M, N, K, scaling):
    """768 tiles (3 per workgroup) at 20 stages; 306 tiles at 21; 1130 tiles at 19."""
    import torch
    e4, _ = _names(f)
    rng = np.random.default_rng(M + K)
    a, b = _codes(e4, (M, K), rng), _codes(e4, (N, K), rng)
    if scaling == "tensor":
        sa, sb, sk, osk = np.float32([0.37]), np.float32([2.5]), f.SCALE_TENSOR, oracle.SCALE_TENSOR
    else:
        sa = rng.uniform(0.01, 3, M).astype(np.float32)
        sb = rng.uniform(0.01, 3, N).astype(np.float32)
        sk, osk = f.SCALE_ROW, oracle.SCALE_ROW
    print("dense multi-tile", M, N, K, scaling, flush=True)
    out = _nan_out((M, N))
    f.fp8_scaled_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, sk, to_dev(sa), to_dev(sb), f.OUT_BF16, out)
    torch.cuda.synchronize()
    ref = oracle.scaled_mm(a, e4, b, e4, osk, sa, sb)
    S = oracle.scaled_mm(a, e4, b, e4, osk, sa, sb, absolute=True)
    check_gemm(out.float().cpu().numpy().astype(np.float64), ref, S, True, f"dense multi-tile {M}x{N}x{K}")


COUNTS = [2999, 0, 4101, 257, 6000, 1, 3333, 511, 2200]  # 19402 rows, 81 row tiles


@pytest.mark.parametrize("K,packed", [(1280, False), (1536, True), (1280, True)])
def test_grouped_multi_tile_rowwise(f, K, packed):
    """Ragged experts (one empty, one of a single row), 81 x 8 row-by-column tiles over
    256 workgroups; row-major operands, and the packed ones (pair-interleaved A,
    k-packed B) of the MoE layer's forward."""
    import torch
    e4, _ = _names(f)
    rng = np.random.default_rng(K + packed)
    off = _offsets(COUNTS)
    E, Mt, N = len(COUNTS), int(off[-1]), 2048
    a, b = _codes(e4, (Mt, K), rng), _codes(e4, (E, N, K), rng)
    sa = rng.uniform(0.1, 2, Mt).astype(np.float32)
    sb = rng.uniform(0.1, 2, (E, N)).astype(np.float32)
    print("grouped multi-tile", K, packed, flush=True)
    out = _nan_out((Mt, N))
    if packed:
        f.fp8_grouped_mm_kpacked(to_dev(kpack(a, 2)).reshape(Mt, K), f.E4M3_NATIVE, to_dev(kpack(b)).reshape(E, -1),
                                 f.E4M3_NATIVE, f.SCALE_ROW, to_dev(sa), to_dev(sb), to_dev(off), f.OUT_BF16, out, N)
    else:
        f.fp8_grouped_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, f.SCALE_ROW, to_dev(sa), to_dev(sb),
                         to_dev(off), f.OUT_BF16, out)
    torch.cuda.synchronize()
    ref = oracle.grouped_mm(a, e4, b, e4, oracle.SCALE_ROW, sa, sb, off)
    S = oracle.grouped_mm(a, e4, b, e4, oracle.SCALE_ROW, sa, sb, off, absolute=True)
    check_gemm(out.float().cpu().numpy().astype(np.float64), ref, S, True, f"grouped multi-tile K {K} packed {packed}")


@pytest.mark.parametrize("K", [1536, 1280])
def test_grouped_multi_tile_mx(f, K):
    """MX scales: K = 1536 loads a row's E8M0 bytes 16 at a time, K = 1280 (not a
    multiple of 512) a dword per stage pair."""
    import torch
    e4, _ = _names(f)
    rng = np.random.default_rng(K + 7)
    off = _offsets(COUNTS)
    E, Mt, N = len(COUNTS), int(off[-1]), 2048
    a, b = _codes(e4, (Mt, K), rng), _codes(e4, (E, N, K), rng)
    sa = rng.integers(117, 137, (Mt, K // 32)).astype(np.uint8)
    sb = rng.integers(117, 137, (E, N, K // 32)).astype(np.uint8)
    print("grouped multi-tile mx", K, flush=True)
    out = _nan_out((Mt, N))
    f.fp8_grouped_mm(to_dev(a), f.E4M3_NATIVE, to_dev(b), f.E4M3_NATIVE, f.SCALE_MX32, to_dev(sa), to_dev(sb),
                     to_dev(off), f.OUT_BF16, out)
    torch.cuda.synchronize()
    ref = oracle.grouped_mm(a, e4, b, e4, oracle.SCALE_MX32, sa, sb, off)
    S = oracle.grouped_mm(a, e4, b, e4, oracle.SCALE_MX32, sa, sb, off, absolute=True)
    check_gemm(out.float().cpu().numpy().astype(np.float64), ref, S, True, f"grouped multi-tile mx K {K}")
