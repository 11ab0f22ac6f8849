"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times: every quantized byte and scale against the oracle (bit-exact), GEMM outputs on
sampled positions the oracle computes one by one. The samples cover every 256 x 256
output tile of every expert (two random positions and two corners per tile) plus
seeded random positions. Each FP8 GEMM runs in both accumulation modes: the full
precision one is held to the floored elementwise bar, the fast one to the hardware's
componentwise bound (check_gemm)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gemm, gpu, have_gpu, kpack, lib, to_dev, to_dev_bf16, u8

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


def _samples(M, N, seed, n=2048, offsets=None, tile=256):
    """Output positions to check: in every tile x tile output tile of every expert (the
    kernels' tiles start at each expert's first row), two seeded random positions and
    its first and last corner; then n seeded random positions over the whole output."""
    rng = np.random.default_rng(seed)
    off = np.asarray(offsets if offsets is not None else [0, M], np.int64)
    rows, cols = [], []
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        for m0 in range(lo, hi, tile):
            m1 = min(m0 + tile, hi)
            for n0 in range(0, N, tile):
                n1 = min(n0 + tile, N)
                rows += list(rng.integers(m0, m1, 2)) + [m0, m1 - 1]
                cols += list(rng.integers(n0, n1, 2)) + [n0, n1 - 1]
    rows += list(rng.integers(0, M, n))
    cols += list(rng.integers(0, N, n))
    return np.array(rows, np.int64), np.array(cols, np.int64)


def _gather(t, rows, cols):
    import torch
    r = torch.from_numpy(rows).to(t.device)
    c = torch.from_numpy(cols).to(t.device)
    return t[r, c].float().cpu().numpy().astype(np.float64)


def _log(*a):
    print(*a, flush=True)


def test_linear_rowwise_llama3_8b_mlp(f):
    """X [8192,4096] (0.1% outliers x50), W [14336,4096], grad_out [8192,14336]."""
    import torch
    e4, e5 = _names(f)
    wl = synth.linear_rowwise()
    x, wt, gy = wl.tensors["x"], wl.tensors["w"], wl.tensors["gy"]
    M, K, N = x.shape[0], x.shape[1], wt.shape[0]
    _log("linear_rowwise generated", wl.meta["outliers"], "outliers")
    xd, wd, gd = to_dev_bf16(x), to_dev_bf16(wt), to_dev_bf16(gy)
    # quantization steps, bit-exact, with the same calls the Linear layer makes
    qx = torch.empty((M, K), dtype=torch.uint8, device="cuda:0")
    sx = torch.empty(M, dtype=torch.float32, device="cuda:0")
    ix = torch.empty_like(sx)
    f.fp8_quant_row(xd, f.E4M3_NATIVE, EPS, qx, sx, ix)
    qw = torch.empty((N, K), dtype=torch.uint8, device="cuda:0")
    sw = torch.empty(N, dtype=torch.float32, device="cuda:0")
    iw = torch.empty_like(sw)
    f.fp8_quant_row(wd, f.E4M3_NATIVE, EPS, qw, sw, iw)
    qg = torch.empty((M, N), dtype=torch.uint8, device="cuda:0")
    sg = torch.empty(M, dtype=torch.float32, device="cuda:0")
    ig = torch.empty_like(sg)
    f.fp8_quant_row(gd, f.E5M2_NATIVE, EPS, qg, sg, ig)
    qwt = torch.empty((K, N), dtype=torch.uint8, device="cuda:0")
    swc = torch.empty(K, dtype=torch.float32, device="cuda:0")
    iwc = torch.empty_like(swc)
    ws = torch.empty(max(f.fp8_quant_col_ws_bytes(1, N, K), 4), dtype=torch.uint8, device="cuda:0")
    f.fp8_quant_col(wd, f.E4M3_NATIVE, EPS, qwt, swc, iwc, ws)
    torch.cuda.synchronize()
    r_qx, r_sx, r_ix = oracle.quant_row(x, e4, EPS)
    assert np.array_equal(u8(qx), r_qx) and np.array_equal(ix.cpu().numpy(), r_ix)
    r_qw, r_sw, r_iw = oracle.quant_row(wt, e4, EPS)
    assert np.array_equal(u8(qw), r_qw) and np.array_equal(iw.cpu().numpy(), r_iw)
    r_qg, r_sg, r_ig = oracle.quant_row(gy, e5, EPS)
    assert np.array_equal(u8(qg), r_qg) and np.array_equal(ig.cpu().numpy(), r_ig)
    r_qwt, r_swc, r_iwc = oracle.quant_col(wt, e4, EPS)
    assert np.array_equal(u8(qwt), r_qwt) and np.array_equal(iwc.cpu().numpy(), r_iwc)
    _log("linear_rowwise quantization bit-exact")

    # the k-packed weight path the benchmark times for the forward and grad-input
    # GEMMs: the same codes permuted, and the same output bits as row-major B
    qwp = torch.empty(N * K, dtype=torch.uint8, device="cuda:0")
    qwtp = torch.empty(N * K, dtype=torch.uint8, device="cuda:0")
    swp, iwp, swcp, iwcp = (torch.empty_like(t) for t in (sw, iw, swc, iwc))
    f.fp8_quant_row_kpacked(wd, f.E4M3_NATIVE, EPS, qwp, swp, iwp)
    f.fp8_quant_col_kpacked(wd, f.E4M3_NATIVE, EPS, qwtp, swcp, iwcp, ws)
    pair = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0") for _ in range(2)]
    f.fp8_scaled_mm(qx, f.E4M3_NATIVE, qw, f.E4M3_NATIVE, f.SCALE_ROW, ix, iw, f.OUT_BF16, pair[0])
    f.fp8_scaled_mm_kpacked(qx, f.E4M3_NATIVE, qwp, f.E4M3_NATIVE, f.SCALE_ROW, ix, iwp, f.OUT_BF16, pair[1], N)
    gpair = [torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0") for _ in range(2)]
    f.fp8_scaled_mm(qg, f.E5M2_NATIVE, qwt, f.E4M3_NATIVE, f.SCALE_ROW, ig, iwc, f.OUT_BF16, gpair[0])
    f.fp8_scaled_mm_kpacked(qg, f.E5M2_NATIVE, qwtp, f.E4M3_NATIVE, f.SCALE_ROW, ig, iwcp, f.OUT_BF16, gpair[1], K)
    torch.cuda.synchronize()
    assert np.array_equal(u8(qwp), kpack(r_qw)) and np.array_equal(u8(qwtp), kpack(r_qwt))
    assert torch.equal(iwp, iw) and torch.equal(iwcp, iwc)
    assert torch.equal(pair[1].view(torch.int16), pair[0].view(torch.int16)), "k-packed forward differs"
    assert torch.equal(gpair[1].view(torch.int16), gpair[0].view(torch.int16)), "k-packed grad-input differs"
    # full precision: the same bits from the k-packed and the row-major weights too
    y_ex = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0") for _ in range(2)]
    f.fp8_scaled_mm(qx, f.E4M3_NATIVE, qw, f.E4M3_NATIVE, f.SCALE_ROW, ix, iw, f.OUT_BF16, y_ex[0],
                    use_fast_accum=False)
    f.fp8_scaled_mm_kpacked(qx, f.E4M3_NATIVE, qwp, f.E4M3_NATIVE, f.SCALE_ROW, ix, iwp, f.OUT_BF16, y_ex[1], N,
                            use_fast_accum=False)
    torch.cuda.synchronize()
    assert torch.equal(y_ex[1].view(torch.int16), y_ex[0].view(torch.int16)), "k-packed exact forward differs"
    y_exact, gx_fast, y_fast_rm = y_ex[0], gpair[0], pair[0]
    del qwp, qwtp, pair, gpair, y_ex
    _log("linear_rowwise k-packed weights and GEMMs bit-identical (both accumulation modes)")

    rc = f.RECIPE_ROWWISE_BF16_WGRAD
    lws = torch.empty(f.fp8_linear_ws_bytes(M, N, K, rc), dtype=torch.uint8, device="cuda:0")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    gx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    gw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_linear_fwd(xd, wd, rc, EPS, f.OUT_BF16, y, lws)
    f.fp8_linear_bwd(gd, xd, wd, rc, EPS, gx, gw, lws)
    torch.cuda.synchronize()
    # the Linear call's forward is the fast accumulation (k-packed weight): the same
    # bits as the row-major fast GEMM above
    assert torch.equal(y.view(torch.int16), y_fast_rm.view(torch.int16)), "fp8_linear_fwd differs"
    r, c = _samples(M, N, 1)
    ref = oracle.scaled_mm_sample(r_qx, e4, r_qw, e4, oracle.SCALE_ROW, r_ix, r_iw, r, c)
    S = oracle.scaled_mm_sample(r_qx, e4, r_qw, e4, oracle.SCALE_ROW, r_ix, r_iw, r, c, absolute=True)
    check_gemm(_gather(y, r, c), ref, S, True, "linear_rowwise forward (sampled)")
    check_gemm(_gather(y_exact, r, c), ref, S, True, "linear_rowwise forward (sampled)", exact=True)
    r, c = _samples(M, K, 2)
    ref = oracle.scaled_mm_sample(r_qg, e5, r_qwt, e4, oracle.SCALE_ROW, r_ig, r_iwc, r, c)
    S = oracle.scaled_mm_sample(r_qg, e5, r_qwt, e4, oracle.SCALE_ROW, r_ig, r_iwc, r, c, absolute=True)
    check_gemm(_gather(gx, r, c), ref, S, True, "linear_rowwise grad-input (sampled)", exact=True)
    check_gemm(_gather(gx_fast, r, c), ref, S, True, "linear_rowwise grad-input (sampled)")
    r, c = _samples(N, K, 3)
    ref = oracle.wgrad_bf16_sample(gy, x, r, c)
    S = oracle.wgrad_bf16_sample(gy, x, r, c, absolute=True)
    check_gemm(_gather(gw, r, c), ref, S, True, "linear_rowwise grad-weight bf16 (sampled)", exact=True)


def test_fused_rmsnorm_quant_llama3_8b_activation(f):
    """RMSNorm fused with the rowwise e4m3 quantization on the Llama3-8B MLP input
    X [8192,4096] (0.1% outliers x50; weights 1 + N(0,0.1)): the stored bf16
    activation and every code and scale equal the oracle's, over the whole tensor."""
    import torch
    e4, _ = _names(f)
    wl = synth.linear_rowwise()
    x = wl.tensors["x"]
    M, K = x.shape
    g32 = oracle.bf16_to_f32(synth.normal_bf16((1, K), 2004, 0.1).reshape(K)) + 1.0
    g = (g32.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda:0")
    s = torch.empty(M, dtype=torch.float32, device="cuda:0")
    i = torch.empty_like(s)
    f.fp8_norm_quant_row(to_dev_bf16(x), to_dev_bf16(g), None, f.NORM_RMS, 1e-5, f.E4M3_NATIVE, EPS, y, q, s, i)
    torch.cuda.synchronize()
    ry, rq, rs, ri = oracle.norm_quant_row(x, g, None, False, 1e-5, e4, EPS)
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ry)
    assert np.array_equal(u8(q), rq)
    assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)


def test_linear_tensorwise_all_fp8_backward_llama3_8b_mlp(f):
    """The all-FP8 tensorwise backward on the Llama3-8B MLP shapes (the same
    X, W and grad_out as the rowwise workload): the dual quantization's three
    outputs bit-exact over the whole tensors, then grad-input and the FP8
    grad-weight GEMM of the whole fp8_linear_bwd call on sampled positions."""
    import torch
    e4, e5 = _names(f)
    wl = synth.linear_rowwise()
    x, wt, gy = wl.tensors["x"], wl.tensors["w"], wl.tensors["gy"]
    M, K, N = x.shape[0], x.shape[1], wt.shape[0]
    xd, wd, gd = to_dev_bf16(x), to_dev_bf16(wt), to_dev_bf16(gy)
    u8d = dict(dtype=torch.uint8, device="cuda:0")
    gq, gqT, xqT = torch.empty((M, N), **u8d), torch.empty((N, M), **u8d), torch.empty((K, M), **u8d)
    sc = [torch.empty(1, dtype=torch.float32, device="cuda:0") for _ in range(4)]
    ws = torch.empty(f.fp8_quant_dual_ws_bytes(), **u8d)
    f.fp8_quant_dual(gd, xd, f.E5M2_NATIVE, f.E4M3_NATIVE, EPS, gq, gqT, sc[0], sc[1], xqT, sc[2], sc[3], ws)
    torch.cuda.synchronize()
    r_gq, r_gqT, r_gs, r_gi, r_xqT, r_xs, r_xi = oracle.quant_dual(gy, x, e5, e4, EPS)
    assert np.array_equal(u8(gq), r_gq) and np.array_equal(u8(gqT), r_gqT) and np.array_equal(u8(xqT), r_xqT)
    assert [t.item() for t in sc] == [r_gs[0], r_gi[0], r_xs[0], r_xi[0]]
    del gq, gqT, xqT
    _log("dual quantization bit-exact")

    rc = f.RECIPE_TENSORWISE
    lws = torch.empty(f.fp8_linear_ws_bytes(M, N, K, rc), **u8d)
    gx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    gw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_linear_bwd(gd, xd, wd, rc, EPS, gx, gw, lws)
    torch.cuda.synchronize()
    r_qw, _, r_iw = oracle.quant_tensor(wt, e4, EPS)
    r_qwt = np.ascontiguousarray(r_qw.T)
    r, c = _samples(M, K, 4)
    ref = oracle.scaled_mm_sample(r_gq, e5, r_qwt, e4, oracle.SCALE_TENSOR, r_gi, r_iw, r, c)
    S = oracle.scaled_mm_sample(r_gq, e5, r_qwt, e4, oracle.SCALE_TENSOR, r_gi, r_iw, r, c, absolute=True)
    check_gemm(_gather(gx, r, c), ref, S, True, "tensorwise grad-input (sampled)", exact=True)
    r, c = _samples(N, K, 5)
    ref = oracle.scaled_mm_sample(r_gqT, e5, r_xqT, e4, oracle.SCALE_TENSOR, r_gi, r_xi, r, c)
    S = oracle.scaled_mm_sample(r_gqT, e5, r_xqT, e4, oracle.SCALE_TENSOR, r_gi, r_xi, r, c, absolute=True)
    check_gemm(_gather(gw, r, c), ref, S, True, "tensorwise FP8 grad-weight (sampled)", exact=True)


def test_expert_colwise(f):
    """32 experts x [2048,7168] with 2 zero columns each -> transposed codes + column scales."""
    import torch
    e4, _ = _names(f)
    wl = synth.expert_colwise()
    w = wl.tensors["w"]
    E, R, C = w.shape
    wd = to_dev_bf16(w)
    qt = torch.empty((E, C, R), dtype=torch.uint8, device="cuda:0")
    s = torch.empty((E, C), dtype=torch.float32, device="cuda:0")
    i = torch.empty_like(s)
    f.fp8_quant_col(wd, f.E4M3_NATIVE, EPS, qt, s, i, None)
    torch.cuda.synchronize()
    rq, rs, ri = oracle.quant_col(w, e4, EPS)
    assert np.array_equal(u8(qt), rq)
    assert np.array_equal(s.cpu().numpy(), rs) and np.array_equal(i.cpu().numpy(), ri)
    # the zero columns took the eps clamp
    zc = wl.meta["zero_cols"]
    assert np.all(rs[np.arange(E)[:, None], zc] == np.float32(oracle.fp8_max(e4) / EPS))


def test_moe_grouped_forward(f):
    """16384 tokens x top-8 over 32 experts (Zipf 1.1, 2 empty) -> A [131072,7168] rowwise,
    W [32][2048][7168] per-expert-column scales, bf16 [131072,2048]."""
    import torch
    e4, _ = _names(f)
    wl = synth.moe_grouped()
    a, w, off = wl.tensors["a"], wl.tensors["w"], wl.meta["offsets"]
    Mt, K = a.shape
    E, N, _ = w.shape
    _log("moe_grouped generated; counts", list(wl.meta["counts"]))
    ad, wd = to_dev_bf16(a), to_dev_bf16(w)
    qa = torch.empty((Mt, K), dtype=torch.uint8, device="cuda:0")
    sa = torch.empty(Mt, dtype=torch.float32, device="cuda:0")
    ia = torch.empty_like(sa)
    f.fp8_quant_row(ad, f.E4M3_NATIVE, EPS, qa, sa, ia)
    qw = torch.empty((E, N, K), dtype=torch.uint8, device="cuda:0")
    sw = torch.empty((E, N), dtype=torch.float32, device="cuda:0")
    iw = torch.empty_like(sw)
    f.fp8_quant_row(wd, f.E4M3_NATIVE, EPS, qw, sw, iw)
    out = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_grouped_mm(qa, f.E4M3_NATIVE, qw, f.E4M3_NATIVE, f.SCALE_ROW, ia, iw, to_dev(off), f.OUT_BF16, out)
    # the packed path the benchmark times: the weights quantized into 1 KB
    # chunks of 16 rows x 64 K, the activations into pair-interleaved rows,
    # then the grouped GEMM reading both
    qwp = torch.empty((E, N * K), dtype=torch.uint8, device="cuda:0")
    swp, iwp = torch.empty_like(sw), torch.empty_like(iw)
    f.fp8_quant_row_kpacked(wd, f.E4M3_NATIVE, EPS, qwp, swp, iwp)
    qap = torch.empty((Mt, K), dtype=torch.uint8, device="cuda:0")
    sap, iap = torch.empty_like(sa), torch.empty_like(ia)
    f.fp8_quant_row_kpaired(ad, f.E4M3_NATIVE, EPS, qap, sap, iap)
    outp = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_grouped_mm_kpacked(qap, f.E4M3_NATIVE, qwp, f.E4M3_NATIVE, f.SCALE_ROW, iap, iwp, to_dev(off), f.OUT_BF16,
                             outp, N)
    torch.cuda.synchronize()
    del ad, wd
    assert torch.equal(outp.view(torch.int16), out.view(torch.int16)), "k-packed GEMM differs from row-major"
    assert torch.equal(iwp, iw) and torch.equal(swp, sw) and torch.equal(iap, ia) and torch.equal(sap, sa)
    # full precision, row-major and packed: the same bits
    out_x = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_grouped_mm(qa, f.E4M3_NATIVE, qw, f.E4M3_NATIVE, f.SCALE_ROW, ia, iw, to_dev(off), f.OUT_BF16, out_x,
                     use_fast_accum=False)
    f.fp8_grouped_mm_kpacked(qap, f.E4M3_NATIVE, qwp, f.E4M3_NATIVE, f.SCALE_ROW, iap, iwp, to_dev(off), f.OUT_BF16,
                             outp, N, use_fast_accum=False)
    torch.cuda.synchronize()
    assert torch.equal(outp.view(torch.int16), out_x.view(torch.int16)), "k-packed exact GEMM differs"
    del outp
    r_qa, _, r_ia = oracle.quant_row(a, e4, EPS)
    assert np.array_equal(u8(qa), r_qa) and np.array_equal(ia.cpu().numpy(), r_ia)
    assert np.array_equal(u8(qap).reshape(-1), kpack(r_qa, 2))
    del qap
    del a
    r_qw, _, r_iw = oracle.quant_row(w, e4, EPS)
    assert np.array_equal(u8(qw), r_qw) and np.array_equal(iw.cpu().numpy(), r_iw)
    assert np.array_equal(u8(qwp).reshape(-1), kpack(r_qw))
    _log("moe_grouped quantization bit-exact (row-major and k-packed)")
    r, c = _samples(Mt, N, 4, offsets=off)
    ref = oracle.grouped_mm_sample(r_qa, e4, r_qw, e4, oracle.SCALE_ROW, r_ia, r_iw, off, r, c)
    S = oracle.grouped_mm_sample(r_qa, e4, r_qw, e4, oracle.SCALE_ROW, r_ia, r_iw, off, r, c, absolute=True)
    check_gemm(_gather(out, r, c), ref, S, True, "moe_grouped gemm (sampled)")
    check_gemm(_gather(out_x, r, c), ref, S, True, "moe_grouped gemm (sampled)", exact=True)


def test_moe_backward(f):
    """The MoE layer's backward on the same routing and weights: grad_out
    [131072,2048] ~N(0,1e-3) quantized per row (e5m2); grouped grad-input
    against the per-expert-column transposed weights (the column kernel on W
    [32][2048][7168] -> [32][7168][2048]); grouped BF16 grad-weight over the
    offsets -> [32][2048][7168] (the two empty experts exactly zero)."""
    import torch
    e4, e5 = _names(f)
    wl = synth.moe_grouped()
    a, w, off = wl.tensors["a"], wl.tensors["w"], wl.meta["offsets"]
    Mt, K = a.shape
    E, N, _ = w.shape
    go = synth.normal_bf16((Mt, N), 4003, 1e-3)
    ad, wd, gd = to_dev_bf16(a), to_dev_bf16(w), to_dev_bf16(go)
    offd = to_dev(off)
    qg = torch.empty((Mt, N), dtype=torch.uint8, device="cuda:0")
    sg = torch.empty(Mt, dtype=torch.float32, device="cuda:0")
    ig = torch.empty_like(sg)
    f.fp8_quant_row(gd, f.E5M2_NATIVE, EPS, qg, sg, ig)
    qT = torch.empty((E, K, N), dtype=torch.uint8, device="cuda:0")
    sT = torch.empty((E, K), dtype=torch.float32, device="cuda:0")
    iT = torch.empty_like(sT)
    f.fp8_quant_col(wd, f.E4M3_NATIVE, EPS, qT, sT, iT, None)
    gx = torch.empty((Mt, K), dtype=torch.bfloat16, device="cuda:0")
    gx_fast = torch.empty((Mt, K), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_grouped_mm(qg, f.E5M2_NATIVE, qT, f.E4M3_NATIVE, f.SCALE_ROW, ig, iT, offd, f.OUT_BF16, gx,
                     use_fast_accum=False)
    f.fp8_grouped_mm(qg, f.E5M2_NATIVE, qT, f.E4M3_NATIVE, f.SCALE_ROW, ig, iT, offd, f.OUT_BF16, gx_fast)
    gw = torch.full((E, N, K), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_grouped_wgrad_bf16(gd, ad, offd, gw)
    # the packed path the benchmark times: grad_out pair-interleaved, the transposed
    # weights k-packed, the k-packed grouped GEMM giving the row-major GEMM's bits
    qgp, qTp = torch.empty_like(qg), torch.empty_like(qT)
    sgp, igp, sTp, iTp = torch.empty_like(sg), torch.empty_like(ig), torch.empty_like(sT), torch.empty_like(iT)
    f.fp8_quant_row_kpaired(gd, f.E5M2_NATIVE, EPS, qgp, sgp, igp)
    f.fp8_quant_col_kpacked(wd, f.E4M3_NATIVE, EPS, qTp, sTp, iTp, None)
    gxp = torch.empty_like(gx)
    gxp_fast = torch.empty_like(gx)
    f.fp8_grouped_mm_kpacked(qgp, f.E5M2_NATIVE, qTp.reshape(E, -1), f.E4M3_NATIVE, f.SCALE_ROW, igp, iTp, offd,
                             f.OUT_BF16, gxp, K, use_fast_accum=False)
    f.fp8_grouped_mm_kpacked(qgp, f.E5M2_NATIVE, qTp.reshape(E, -1), f.E4M3_NATIVE, f.SCALE_ROW, igp, iTp, offd,
                             f.OUT_BF16, gxp_fast, K)
    torch.cuda.synchronize()
    assert torch.equal(igp, ig) and torch.equal(iTp, iT)
    assert torch.equal(gxp.view(torch.int16), gx.view(torch.int16))
    assert torch.equal(gxp_fast.view(torch.int16), gx_fast.view(torch.int16))
    del ad, wd, gd
    r_qg, _, r_ig = oracle.quant_row(go, e5, EPS)
    assert np.array_equal(u8(qg), r_qg) and np.array_equal(ig.cpu().numpy(), r_ig)
    assert np.array_equal(u8(qgp).reshape(-1), kpack(r_qg, 2))
    r_qT, _, r_iT = oracle.quant_col(w, e4, EPS)
    assert np.array_equal(u8(qT), r_qT) and np.array_equal(iT.cpu().numpy(), r_iT)
    assert np.array_equal(u8(qTp).reshape(-1), kpack(r_qT, 16))
    _log("moe backward quantization bit-exact (row-major and packed)")
    r, c = _samples(Mt, K, 6, offsets=off)
    ref = oracle.grouped_mm_sample(r_qg, e5, r_qT, e4, oracle.SCALE_ROW, r_ig, r_iT, off, r, c)
    S = oracle.grouped_mm_sample(r_qg, e5, r_qT, e4, oracle.SCALE_ROW, r_ig, r_iT, off, r, c, absolute=True)
    check_gemm(_gather(gx, r, c), ref, S, True, "moe grouped grad-input (sampled)", exact=True)
    check_gemm(_gather(gx_fast, r, c), ref, S, True, "moe grouped grad-input (sampled)")
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            assert torch.count_nonzero(gw[e]).item() == 0, f"empty expert {e}"
            continue
        # every 256 x 256 tile of the expert's [N][K] gradient, and 64 random positions
        ns, ks = _samples(N, K, 700 + e, n=64)
        gs, xs = np.ascontiguousarray(go[lo:hi]), np.ascontiguousarray(a[lo:hi])
        ref = oracle.wgrad_bf16_sample(gs, xs, ns, ks)
        S = oracle.wgrad_bf16_sample(gs, xs, ns, ks, absolute=True)
        got = gw[e][torch.from_numpy(ns).cuda(), torch.from_numpy(ks).cuda()].float().cpu().numpy()
        check_gemm(got.astype(np.float64), ref, S, True, f"moe grouped grad-weight expert {e} (sampled)", exact=True)


def test_moe_block_and_mx(f):
    """16 experts, K 5120, N 8192, 8192 rows (512 per expert), per-row magnitude spread
    2^-8..2^8: 1x128 / 128x128 blockwise and 32-element MX quantization and GEMMs."""
    import torch
    e4, _ = _names(f)
    wl = synth.moe_block_mx()
    a, w, off = wl.tensors["a"], wl.tensors["w"], wl.meta["offsets"]
    Mt, K = a.shape
    E, N, _ = w.shape
    ad, wd, offd = to_dev_bf16(a), to_dev_bf16(w), to_dev(off)
    # blockwise
    qa = torch.empty((Mt, K), dtype=torch.uint8, device="cuda:0")
    sa = torch.empty((Mt, K // 128), dtype=torch.float32, device="cuda:0")
    ia = torch.empty_like(sa)
    f.fp8_quant_block(ad, 1, 128, f.E4M3_NATIVE, EPS, qa, sa, ia)
    qw = torch.empty((E, N, K), dtype=torch.uint8, device="cuda:0")
    sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device="cuda:0")
    iw = torch.empty_like(sw)
    f.fp8_quant_block(wd, 128, 128, f.E4M3_NATIVE, EPS, qw, sw, iw)
    out = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda:0")
    out_x = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda:0")
    f.fp8_grouped_mm(qa, f.E4M3_NATIVE, qw, f.E4M3_NATIVE, f.SCALE_BLOCK128, ia, iw, offd, f.OUT_BF16, out)
    f.fp8_grouped_mm(qa, f.E4M3_NATIVE, qw, f.E4M3_NATIVE, f.SCALE_BLOCK128, ia, iw, offd, f.OUT_BF16, out_x,
                     use_fast_accum=False)
    torch.cuda.synchronize()
    r_qa, _, r_ia = oracle.quant_block(a, 1, 128, e4, EPS)
    assert np.array_equal(u8(qa), r_qa) and np.array_equal(ia.cpu().numpy(), r_ia)
    r_qw, _, r_iw = oracle.quant_block(w, 128, 128, e4, EPS)
    assert np.array_equal(u8(qw), r_qw) and np.array_equal(iw.cpu().numpy(), r_iw)
    r, c = _samples(Mt, N, 5, offsets=off)
    ref = oracle.grouped_mm_sample(r_qa, e4, r_qw, e4, oracle.SCALE_BLOCK128, r_ia, r_iw, off, r, c)
    S = oracle.grouped_mm_sample(r_qa, e4, r_qw, e4, oracle.SCALE_BLOCK128, r_ia, r_iw, off, r, c, absolute=True)
    check_gemm(_gather(out, r, c), ref, S, True, "moe blockwise gemm (sampled)")
    check_gemm(_gather(out_x, r, c), ref, S, True, "moe blockwise gemm (sampled)", exact=True)
    del r_qw
    # MX
    ea = torch.empty((Mt, K // 32), dtype=torch.uint8, device="cuda:0")
    f.fp8_quant_mx(ad, f.E4M3_NATIVE, f.MX_POW2_FLOOR, EPS, qa, ea)
    ew = torch.empty((E, N, K // 32), dtype=torch.uint8, device="cuda:0")
    f.fp8_quant_mx(wd, f.E4M3_NATIVE, f.MX_POW2_FLOOR, EPS, qw, ew)
    f.fp8_grouped_mm(qa, f.E4M3_NATIVE, qw, f.E4M3_NATIVE, f.SCALE_MX32, ea, ew, offd, f.OUT_BF16, out)
    f.fp8_grouped_mm(qa, f.E4M3_NATIVE, qw, f.E4M3_NATIVE, f.SCALE_MX32, ea, ew, offd, f.OUT_BF16, out_x,
                     use_fast_accum=False)
    torch.cuda.synchronize()
    r_qa, r_ea = oracle.quant_mx(a, e4, oracle.MX_POW2_FLOOR, EPS)
    assert np.array_equal(u8(qa), r_qa) and np.array_equal(u8(ea), r_ea)
    r_qw, r_ew = oracle.quant_mx(w, e4, oracle.MX_POW2_FLOOR, EPS)
    assert np.array_equal(u8(qw), r_qw) and np.array_equal(u8(ew), r_ew)
    ref = oracle.grouped_mm_sample(r_qa, e4, r_qw, e4, oracle.SCALE_MX32, r_ea, r_ew, off, r, c)
    S = oracle.grouped_mm_sample(r_qa, e4, r_qw, e4, oracle.SCALE_MX32, r_ea, r_ew, off, r, c, absolute=True)
    check_gemm(_gather(out, r, c), ref, S, True, "moe MX gemm (sampled)")
    check_gemm(_gather(out_x, r, c), ref, S, True, "moe MX gemm (sampled)", exact=True)
    # the packed path the benchmark times: the MX quantizers writing pair-interleaved A
    # and k-packed W give the oracle's codes permuted and the same E8M0 bytes, and the
    # k-packed grouped GEMM on them gives the row-major GEMM's bits
    qap, qwp = torch.empty_like(qa), torch.empty_like(qw)
    eap, ewp = torch.empty_like(ea), torch.empty_like(ew)
    f.fp8_quant_mx_kpaired(ad, f.E4M3_NATIVE, f.MX_POW2_FLOOR, EPS, qap, eap)
    f.fp8_quant_mx_kpacked(wd, f.E4M3_NATIVE, f.MX_POW2_FLOOR, EPS, qwp, ewp)
    out_p = torch.empty_like(out)
    f.fp8_grouped_mm_kpacked(qap, f.E4M3_NATIVE, qwp.reshape(E, -1), f.E4M3_NATIVE, f.SCALE_MX32, eap, ewp, offd,
                             f.OUT_BF16, out_p, N)
    torch.cuda.synchronize()
    assert torch.equal(eap, ea) and torch.equal(ewp, ew)
    assert np.array_equal(u8(qap).reshape(-1), kpack(r_qa, 2))
    assert np.array_equal(u8(qwp).reshape(-1), kpack(r_qw, 16))
    assert torch.equal(out_p.view(torch.int16), out.view(torch.int16))
