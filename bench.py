"""Benchmark of the dynamic-FP8 hot path on one MI355X.

One step runs every step of the path over the five synthetic workloads, inputs
already resident in HBM:
  linear_tensorwise  fp8_linear_fwd, X [256,512] W [512,512], one scale each, fp32 out
  linear_rowwise     Llama3-8B MLP (tokens 8192, K 4096, N 14336): rowwise quant of X, W
                     (e4m3) and grad_out (e5m2), per-column transposed quant of W (both
                     W codes k-packed), FP8 forward and grad-input GEMMs, BF16
                     weight-gradient GEMM; beside it
                     (reported per row, outside the aggregates) the all-FP8 tensorwise
                     backward of the same layer: the dual quantization of grad_out and X,
                     the FP8 weight-gradient GEMM and the whole fp8_linear_bwd call
  expert_colwise     per-expert column scales + transposed cast, 32 x [2048,7168]
  moe_grouped        rowwise quant of A [131072,7168] and of W [32][2048][7168] (per
                     expert column; W's codes k-packed, 1 KB chunks of 16 rows x 64 K,
                     A's pair-interleaved),
                     FP8 grouped GEMM over int32[33] offsets -> bf16; beside
                     it (per row, outside the aggregates) the layer's backward: grad_out
                     [131072,2048] per-row e5m2, the grouped grad-input GEMM against
                     expert_colwise's transposed per-column weights, the grouped BF16
                     grad-weight GEMM over the same offsets
  moe_block_mx       1x128 / 128x128 blockwise and MX quant, 16 experts, K 5120, N 8192,
                     and the blockwise and MX grouped GEMMs
Every launch is bracketed by HIP events on the stream it runs on. The steps run
twice: back to back (warm; the wall-clock timed region of ms_per_step) and with a
512 MiB read before each call, outside its events (cold: nothing left in the L2 or
the Infinity Cache, and no dirty lines whose write-back would fall inside the call).
The JSON line reports, from the cold pass, the fused-quantization
throughput (algorithmic bytes of all quantization calls / their summed event time,
3 B per element + 8 B per fp32 scale group or 1 B per E8M0 group) as `value`, the
grouped-GEMM throughput (2*M*N*K / event time) of the moe_grouped GEMM as
`gemm_value`, per-call avg/median/p10/p90 (cold and warm) under `rows`, the roofline
of the dominant kernel, the shader and memory clocks sampled during the run, and the
oracle's CPU throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0
EPS = 1e-12

METRIC = "fused FP8 quant GB/s (% HBM peak); FP8 grouped-GEMM TFLOP/s (% MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Step:
    """A list of named calls; each call is timed with a pair of HIP events."""

    def __init__(self, torch):
        self.torch = torch
        self.calls = []  # (name, kind, work, fn); kind: quant (bytes) / gemm8 / gemm16 (flops) / latency

    def add(self, name, kind, work, fn):
        self.calls.append((name, kind, float(work), fn))

    def run(self, stream, record=None, flush=None):
        """One pass over the calls. record: per-call lists receiving (start, end) events.
        flush: a device buffer read in full before each call, outside its events,
        so that the call finds neither its inputs nor its outputs in the L2 or the
        256 MB Infinity Cache (the cold measurement). It is read, not written: a
        written flush leaves its own dirty lines in the caches, and their write-back
        to HBM then runs inside the next call's events (measured on MI355X: the
        Llama3-8B weight's column quantization 81 us after a 512 MiB write, 59 us
        after a 512 MiB read)."""
        torch = self.torch
        for i, (name, kind, work, fn) in enumerate(self.calls):
            if flush is not None:
                torch.amax(flush)
            if record is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                record[i].append((e0, e1))
            else:
                fn()


# sha256 (first 16 hex digits) of the host inputs that build_step draws beside
# the workloads' own tensors, filled in as it draws them
EXTRA_INPUT_SHA = {}


def input_digests(wls):
    """sha256 of every generated host input: each workload's tensors and
    offsets, then the extra inputs the step draws."""
    import numpy as np
    import synth
    d = {}
    for n, w in wls.items():
        if w is None:
            continue
        for k, v in w.tensors.items():
            d[f"{n}.{k}"] = synth.sha256(v)
        if "offsets" in w.meta:
            d[f"{n}.offsets"] = synth.sha256(np.asarray(w.meta["offsets"]))
    d.update(EXTRA_INPUT_SHA)
    return d


def build_step(f, torch, dev, wls, dev_of):
    """Allocates outputs and returns a Step whose calls cover every step of the path."""
    st = Step(torch)
    E4, E5 = f.E4M3_NATIVE, f.E5M2_NATIVE
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)

    # ---- linear_tensorwise: the whole fp8_linear_fwd call (latency-bound) ----
    w1 = wls["linear_tensorwise"]
    x1, wt1 = dev_of(w1.tensors["x"]), dev_of(w1.tensors["w"])
    M1, K1, N1 = x1.shape[0], x1.shape[1], wt1.shape[0]
    ws1 = torch.empty(f.fp8_linear_ws_bytes(M1, N1, K1, f.RECIPE_TENSORWISE), **u8)
    y1 = torch.empty((M1, N1), **f32)
    st.add("linear_tensorwise.fwd", "latency", 2.0 * M1 * N1 * K1,
           lambda: f.fp8_linear_fwd(x1, wt1, f.RECIPE_TENSORWISE, EPS, f.OUT_F32, y1, ws1))

    # ---- linear_rowwise: forward and backward of the Llama3-8B MLP projection ----
    w2 = wls["linear_rowwise"]
    x2, wt2, g2 = dev_of(w2.tensors["x"]), dev_of(w2.tensors["w"]), dev_of(w2.tensors["gy"])
    M, K = x2.shape
    N = wt2.shape[0]
    qx, sx, ix = torch.empty((M, K), **u8), torch.empty(M, **f32), torch.empty(M, **f32)
    qw, sw, iw = torch.empty((N, K), **u8), torch.empty(N, **f32), torch.empty(N, **f32)
    qg, sg, ig = torch.empty((M, N), **u8), torch.empty(M, **f32), torch.empty(M, **f32)
    qwt, swc, iwc = torch.empty((K, N), **u8), torch.empty(K, **f32), torch.empty(K, **f32)
    colws = torch.empty(max(f.fp8_quant_col_ws_bytes(1, N, K), 4), **u8)
    y2 = torch.empty((M, N), **bf)
    gx2 = torch.empty((M, K), **bf)
    gw2 = torch.empty((N, K), **bf)
    st.add("linear_rowwise.quant_row_x", "quant", 3 * M * K + 8 * M,
           lambda: f.fp8_quant_row(x2, E4, EPS, qx, sx, ix))
    # W's codes k-packed by both of its quantizations (1 KB chunks of 16 rows
    # x 64 K of the GEMM's B operand): the forward's and the grad-input's
    st.add("linear_rowwise.quant_row_w", "quant", 3 * N * K + 8 * N,
           lambda: f.fp8_quant_row_kpacked(wt2, E4, EPS, qw, sw, iw))
    st.add("linear_rowwise.gemm_fwd", "gemm8", 2.0 * M * N * K,
           lambda: f.fp8_scaled_mm_kpacked(qx, E4, qw, E4, f.SCALE_ROW, ix, iw, f.OUT_BF16, y2, N))
    st.add("linear_rowwise.quant_row_gy_e5m2", "quant", 3 * M * N + 8 * M,
           lambda: f.fp8_quant_row(g2, E5, EPS, qg, sg, ig))
    st.add("linear_rowwise.quant_col_w", "quant", 3 * N * K + 8 * K,
           lambda: f.fp8_quant_col_kpacked(wt2, E4, EPS, qwt, swc, iwc, colws))
    st.add("linear_rowwise.gemm_dgrad", "gemm8", 2.0 * M * N * K,
           lambda: f.fp8_scaled_mm_kpacked(qg, E5, qwt, E4, f.SCALE_ROW, ig, iwc, f.OUT_BF16, gx2, K))
    st.add("linear_rowwise.wgrad_bf16", "gemm16", 2.0 * M * N * K,
           lambda: f.fp8_wgrad_bf16(g2, x2, gw2))
    # the grad-input GEMM at full precision (codes decoded to bf16, BF16 matrix
    # cores), as fp8_linear_bwd runs it; and the two whole Linear calls, each the
    # sum of its launches above (forward: quant_row_x + quant_row_w + gemm_fwd;
    # backward: quant_row_gy_e5m2 + quant_col_w + gemm_dgrad_exact + wgrad_bf16)
    gx2x = torch.empty((M, K), **bf)
    st.add("linear_rowwise.gemm_dgrad_exact", "gemm8x_next", 2.0 * M * N * K,
           lambda: f.fp8_scaled_mm_kpacked(qg, E5, qwt, E4, f.SCALE_ROW, ig, iwc, f.OUT_BF16, gx2x, K,
                                           use_fast_accum=False))
    lws_r = torch.empty(f.fp8_linear_ws_bytes(M, N, K, f.RECIPE_ROWWISE_BF16_WGRAD), **u8)
    y2l, gx2l, gw2l = torch.empty((M, N), **bf), torch.empty((M, K), **bf), torch.empty((N, K), **bf)
    st.add("linear_rowwise.linear_fwd", "latency", 2.0 * M * N * K,
           lambda: f.fp8_linear_fwd(x2, wt2, f.RECIPE_ROWWISE_BF16_WGRAD, EPS, f.OUT_BF16, y2l, lws_r))
    st.add("linear_rowwise.linear_bwd", "latency", 4.0 * M * N * K,
           lambda: f.fp8_linear_bwd(g2, x2, wt2, f.RECIPE_ROWWISE_BF16_WGRAD, EPS, gx2l, gw2l, lws_r))

    # ---- the norm that produces X, fused with its rowwise quantization,
    # against the unfused pair (outside the aggregates) ----
    import numpy as np
    import synth as _synth
    # RMSNorm weights 1 + N(0, 0.1), truncated to bf16
    gn = _synth.normal_bf16((1, K), 2004, 0.1).reshape(K)
    EXTRA_INPUT_SHA["linear_rowwise.norm_weight_delta"] = _synth.sha256(gn)
    gn32 = (gn.astype(np.uint32) << 16).view(np.float32) + np.float32(1.0)
    gnd = dev_of((gn32.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    yn = torch.empty((M, K), **bf)
    qn, sn, in_ = torch.empty((M, K), **u8), torch.empty(M, **f32), torch.empty(M, **f32)
    st.add("norm_quant.unfused_rmsnorm", "quant_next", 4 * M * K,
           lambda: f.fp8_norm_quant_row(x2, gnd, None, f.NORM_RMS, 1e-5, E4, EPS, yn, None, None))
    st.add("norm_quant.unfused_quant_row", "quant_next", 3 * M * K + 8 * M,
           lambda: f.fp8_quant_row(yn, E4, EPS, qn, sn, in_))
    st.add("norm_quant.fused_y_and_q", "quant_next", 5 * M * K + 8 * M,
           lambda: f.fp8_norm_quant_row(x2, gnd, None, f.NORM_RMS, 1e-5, E4, EPS, yn, qn, sn, in_))
    st.add("norm_quant.fused_q_only", "quant_next", 3 * M * K + 8 * M,
           lambda: f.fp8_norm_quant_row(x2, gnd, None, f.NORM_RMS, 1e-5, E4, EPS, None, qn, sn, in_))

    # ---- the all-FP8 tensorwise backward of the same layer (beside the
    # rowwise recipe; not part of the aggregate figures) ----
    gqb, gqTb, xqTb = torch.empty((M, N), **u8), torch.empty((N, M), **u8), torch.empty((K, M), **u8)
    dsc = [torch.empty(1, **f32) for _ in range(4)]
    dws = torch.empty(f.fp8_quant_dual_ws_bytes(), **u8)
    gwf = torch.empty((N, K), **bf)
    gxt, gwt = torch.empty((M, K), **bf), torch.empty((N, K), **bf)
    lws2 = torch.empty(f.fp8_linear_ws_bytes(M, N, K, f.RECIPE_TENSORWISE), **u8)
    st.add("linear_tensorwise_fp8_bwd.quant_dual_gy_x", "quant_next",
           2 * (M * N + M * K) + 2 * M * N + M * K + 16,
           lambda: f.fp8_quant_dual(g2, x2, E5, E4, EPS, gqb, gqTb, dsc[0], dsc[1], xqTb, dsc[2], dsc[3], dws))
    st.add("linear_tensorwise_fp8_bwd.gemm_wgrad_fp8", "gemm8_next", 2.0 * M * N * K,
           lambda: f.fp8_scaled_mm(gqTb, E5, xqTb, E4, f.SCALE_TENSOR, dsc[1], dsc[3], f.OUT_BF16, gwf))
    st.add("linear_tensorwise_fp8_bwd.gemm_wgrad_fp8_exact", "gemm8x_next", 2.0 * M * N * K,
           lambda: f.fp8_scaled_mm(gqTb, E5, xqTb, E4, f.SCALE_TENSOR, dsc[1], dsc[3], f.OUT_BF16, gwf,
                                   use_fast_accum=False))
    st.add("linear_tensorwise_fp8_bwd.linear_bwd", "latency", 4.0 * M * N * K,
           lambda: f.fp8_linear_bwd(g2, x2, wt2, f.RECIPE_TENSORWISE, EPS, gxt, gwt, lws2))

    # ---- expert_colwise ----
    w3 = wls["expert_colwise"]
    we3 = dev_of(w3.tensors["w"])
    E3, R3, C3 = we3.shape
    qt3 = torch.empty((E3, C3, R3), **u8)
    s3, i3 = torch.empty((E3, C3), **f32), torch.empty((E3, C3), **f32)
    # the transposed codes k-packed (the MoE backward's grouped grad-input GEMM
    # loads B from that layout in whole lines)
    st.add("expert_colwise.quant_col", "quant", 3 * E3 * R3 * C3 + 8 * E3 * C3,
           lambda: f.fp8_quant_col_kpacked(we3, E4, EPS, qt3, s3, i3, None))

    # ---- moe_grouped ----
    w4 = wls["moe_grouped"]
    a4, we4 = dev_of(w4.tensors["a"]), dev_of(w4.tensors["w"])
    off4 = torch.from_numpy(w4.meta["offsets"]).to(dev)
    Mt, K4 = a4.shape
    E4n, N4, _ = we4.shape
    qa4, sa4, ia4 = torch.empty((Mt, K4), **u8), torch.empty(Mt, **f32), torch.empty(Mt, **f32)
    qw4, sw4, iw4 = torch.empty((E4n, N4, K4), **u8), torch.empty((E4n, N4), **f32), torch.empty((E4n, N4), **f32)
    out4 = torch.empty((Mt, N4), **bf)
    # the activations' codes pair-interleaved (rows 2i, 2i + 1 share each
    # 128-byte line), the A layout of the k-packed grouped GEMM
    st.add("moe_grouped.quant_row_a", "quant", 3 * Mt * K4 + 8 * Mt,
           lambda: f.fp8_quant_row_kpaired(a4, E4, EPS, qa4, sa4, ia4))
    # the weights' codes k-packed (1 KB chunks of 16 rows x 64 K) by their
    # quantization, the layout the grouped GEMM loads B from in whole lines
    st.add("moe_grouped.quant_expert_cols_w", "quant", 3 * E4n * N4 * K4 + 8 * E4n * N4,
           lambda: f.fp8_quant_row_kpacked(we4, E4, EPS, qw4, sw4, iw4))
    st.add("moe_grouped.grouped_gemm", "gemm8", 2.0 * Mt * N4 * K4,
           lambda: f.fp8_grouped_mm_kpacked(qa4, E4, qw4, E4, f.SCALE_ROW, ia4, iw4, off4, f.OUT_BF16, out4, N4))

    # ---- the MoE layer's backward on the same routing (outside the
    # aggregates): grad_out quantized per row (e5m2); grouped grad-input
    # against the per-expert-column transposed weights expert_colwise wrote
    # (its W has the layer's [32][2048][7168] shape); grouped BF16
    # grad-weight over the offsets ----
    import synth as _synth
    go4_h = _synth.normal_bf16((Mt, N4), 4003, 1e-3)
    EXTRA_INPUT_SHA["moe_grouped.grad_out"] = _synth.sha256(go4_h)
    go4 = dev_of(go4_h)
    qgo4, sgo4, igo4 = torch.empty((Mt, N4), **u8), torch.empty(Mt, **f32), torch.empty(Mt, **f32)
    gx4 = torch.empty((Mt, K4), **bf)
    gw4 = torch.empty((E4n, N4, K4), **bf)
    # grad_out pair-interleaved and the transposed weights k-packed: the k-packed
    # grouped GEMM (same bits as the row-major one)
    st.add("moe_backward.quant_row_go_e5m2", "quant_next", 3 * Mt * N4 + 8 * Mt,
           lambda: f.fp8_quant_row_kpaired(go4, E5, EPS, qgo4, sgo4, igo4))
    st.add("moe_backward.grouped_dgrad", "gemm8_next", 2.0 * Mt * N4 * K4,
           lambda: f.fp8_grouped_mm_kpacked(qgo4, E5, qt3.reshape(E3, -1), E4, f.SCALE_ROW, igo4, i3, off4, f.OUT_BF16,
                                            gx4, C3))
    st.add("moe_backward.grouped_dgrad_exact", "gemm8x_next", 2.0 * Mt * N4 * K4,
           lambda: f.fp8_grouped_mm_kpacked(qgo4, E5, qt3.reshape(E3, -1), E4, f.SCALE_ROW, igo4, i3, off4, f.OUT_BF16,
                                            gx4, C3, use_fast_accum=False))
    st.add("moe_backward.grouped_wgrad_bf16", "gemm16_next", 2.0 * Mt * N4 * K4,
           lambda: f.fp8_grouped_wgrad_bf16(go4, a4, off4, gw4))

    # ---- moe_block_mx ----
    w5 = wls["moe_block_mx"]
    a5, we5 = dev_of(w5.tensors["a"]), dev_of(w5.tensors["w"])
    off5 = torch.from_numpy(w5.meta["offsets"]).to(dev)
    M5, K5 = a5.shape
    E5n, N5, _ = we5.shape
    qa5, qw5 = torch.empty((M5, K5), **u8), torch.empty((E5n, N5, K5), **u8)
    sa5, ia5 = torch.empty((M5, K5 // 128), **f32), torch.empty((M5, K5 // 128), **f32)
    sw5, iw5 = torch.empty((E5n, N5 // 128, K5 // 128), **f32), torch.empty((E5n, N5 // 128, K5 // 128), **f32)
    ea5, ew5 = torch.empty((M5, K5 // 32), **u8), torch.empty((E5n, N5, K5 // 32), **u8)
    qa5m, qw5m = torch.empty((M5, K5), **u8), torch.empty((E5n, N5, K5), **u8)
    out5 = torch.empty((M5, N5), **bf)
    out5m = torch.empty((M5, N5), **bf)
    st.add("moe_block_mx.quant_block_a_1x128", "quant", 3 * M5 * K5 + 8 * M5 * (K5 // 128),
           lambda: f.fp8_quant_block(a5, 1, 128, E4, EPS, qa5, sa5, ia5))
    st.add("moe_block_mx.quant_block_w_128x128", "quant", 3 * E5n * N5 * K5 + 8 * E5n * (N5 // 128) * (K5 // 128),
           lambda: f.fp8_quant_block(we5, 128, 128, E4, EPS, qw5, sw5, iw5))
    st.add("moe_block_mx.grouped_gemm_block", "gemm8", 2.0 * M5 * N5 * K5,
           lambda: f.fp8_grouped_mm(qa5, E4, qw5, E4, f.SCALE_BLOCK128, ia5, iw5, off5, f.OUT_BF16, out5))
    # MX codes written in the k-packed grouped GEMM's operand layouts by the
    # quantizers themselves (A pair-interleaved, W k-packed), as for moe_grouped
    st.add("moe_block_mx.quant_mx_a", "quant", 3 * M5 * K5 + M5 * (K5 // 32),
           lambda: f.fp8_quant_mx_kpaired(a5, E4, f.MX_POW2_FLOOR, EPS, qa5m, ea5))
    st.add("moe_block_mx.quant_mx_w", "quant", 3 * E5n * N5 * K5 + E5n * N5 * (K5 // 32),
           lambda: f.fp8_quant_mx_kpacked(we5, E4, f.MX_POW2_FLOOR, EPS, qw5m, ew5))
    st.add("moe_block_mx.grouped_gemm_mx", "gemm8", 2.0 * M5 * N5 * K5,
           lambda: f.fp8_grouped_mm_kpacked(qa5m, E4, qw5m.reshape(E5n, -1), E4, f.SCALE_MX32, ea5, ew5, off5,
                                            f.OUT_BF16, out5m, N5))
    return st


# Source files whose kernels each kind of bench row runs: a stored HBM-traffic
# figure is used only while these files are byte-identical to the ones profiled.
KERNEL_SOURCES = {
    "quant": ["quant.hip", "common.hpp"],
    "gemm8": ["gemm_fp8_fast.hip", "gemm_fp8.hip", "gemm_common.hpp", "common.hpp"],
    "gemm16": ["gemm_bf16.hip", "gemm_common.hpp", "common.hpp"],
}
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def sources_digest(kind):
    import hashlib
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES.get(kind, []):
        with open(os.path.join(ROOT, "fp8_dynamic_scaling_amd", "csrc", fn), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(name, kind):
    """HBM bytes per launch of bench row `name` from the committed counter table
    (FETCH_SIZE + WRITE_SIZE, each scaled by the plain-copy calibration), or None
    when there is no entry or the kernel's sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_TABLE):
        return None
    digest = sources_digest(kind)
    with open(TRAFFIC_TABLE) as fh:
        for line in fh:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 4 and cells[0] == name and cells[1] == digest:
                try:
                    return int(cells[-1])
                except ValueError:
                    return None
    return None


def calibration_copy(torch, dev, nbytes):
    """A plain device-to-device copy of nbytes (read nbytes, write nbytes), run
    outside the timed region so that counter runs can scale FETCH_SIZE and
    WRITE_SIZE to bytes."""
    src = torch.full((nbytes,), 7, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline(wls, budget_s=20.0):
    """The oracle as it stands, on a bounded sample of the moe_grouped workload:
    rowwise quantization of the activation rows, then fp64 grouped-GEMM outputs
    for a sample of rows, until about budget_s seconds are spent."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    threads = oracle.threads_used(0)
    w = wls["moe_grouped"]
    a, wt, off = w.tensors["a"], w.tensors["w"], w.meta["offsets"]
    Mt, K = a.shape
    E, N, _ = wt.shape
    # quantization: whole row blocks of A until a quarter of the budget is used
    rows_done, t_q = 0, 0.0
    chunk = 8192
    while t_q < budget_s * 0.25 and rows_done < Mt:
        blk = np.ascontiguousarray(a[rows_done:rows_done + chunk])
        t0 = time.perf_counter()
        oracle.quant_row(blk, "e4m3fn", EPS, threads=threads)
        t_q += time.perf_counter() - t0
        rows_done += blk.shape[0]
    q_bytes = rows_done * (3 * K + 8)
    # GEMM: output rows of the grouped product (all N columns) on a row sample
    qa, _, ia = oracle.quant_row(np.ascontiguousarray(a[:16384]), "e4m3fn", EPS, threads=threads)
    qw, _, iw = oracle.quant_row(wt, "e4m3fn", EPS, threads=threads)
    sub_off = np.minimum(off, 16384).astype(np.int32)
    n_rows, t_g = 0, 0.0
    rng = np.random.default_rng(0)
    while t_g < budget_s * 0.75 and n_rows < 16384:
        rows = rng.integers(0, 16384, 16)
        rr = np.repeat(rows, N)
        cc = np.tile(np.arange(N), rows.size)
        t0 = time.perf_counter()
        oracle.grouped_mm_sample(qa, "e4m3fn", qw, "e4m3fn", oracle.SCALE_ROW, ia, iw, sub_off, rr, cc)
        t_g += time.perf_counter() - t0
        n_rows += rows.size
    flops = 2.0 * n_rows * N * K
    return {
        "value": round(q_bytes / t_q / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"moe_grouped: rowwise quantization of the first {rows_done} activation rows "
                   f"({q_bytes / 1e9:.2f} GB algorithmic) in {t_q:.1f} s; fp64 grouped GEMM of "
                   f"{n_rows} sampled output rows x {N} columns x K {K} in {t_g:.1f} s"),
        "gemm_value": round(flops / t_g / 1e12, 6), "gemm_unit": "TFLOP/s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--only", default="", help="comma-separated workload names (profiling runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run a plain copy of this many MiB first (counter calibration runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the path has no multi-GPU part).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_dynamic_scaling_amd as f
    import synth

    f.load()
    synth.build(force=False)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    e4, e5 = f.fp8_probe(0)
    if args.calib_copy_mib > 0:
        calibration_copy(torch, dev, args.calib_copy_mib << 20)
    t0 = time.perf_counter()
    names = ["linear_tensorwise", "linear_rowwise", "expert_colwise", "moe_grouped", "moe_block_mx"]
    if args.only:
        names = [n for n in names if n in args.only.split(",")]
    gens = {"linear_tensorwise": synth.linear_tensorwise, "linear_rowwise": synth.linear_rowwise,
            "expert_colwise": synth.expert_colwise, "moe_grouped": synth.moe_grouped,
            "moe_block_mx": synth.moe_block_mx}
    wls = {n: gens[n]() for n in names}
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev_of(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    # build the step (only the selected workloads)
    full = {n: wls.get(n) for n in names}
    st = build_step_subset(f, torch, dev, full, dev_of)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        st.run(stream)
    torch.cuda.synchronize()
    log("warmup done")
    clocks = ClockSampler()
    clocks.start()
    # warm: the steps back to back, as a training step runs them (the timed region)
    warm = [[] for _ in st.calls]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        st.run(stream, warm)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    log(f"warm steps done ({ms_per_step:.2f} ms per step)")
    # cold: the same steps with a 512 MiB read before every call (outside its
    # events), twice the 256 MB Infinity Cache, so no call reads data an earlier
    # call left in the caches, and no earlier call's dirty lines are written
    # back inside it; the reported figures are these
    flush = torch.zeros(128 << 20, dtype=torch.int32, device=dev)
    cold = [[] for _ in st.calls]
    for _ in range(args.steps):
        st.run(stream, cold, flush=flush)
    torch.cuda.synchronize()
    del flush
    clocks.stop()
    log("cold steps done")

    def times(rec_i):
        return np.array([e0.elapsed_time(e1) for e0, e1 in rec_i]) * 1e-3  # seconds

    rows = {}
    q_bytes = q_time = 0.0
    dom = None
    for i, (name, kind, work, _) in enumerate(st.calls):
        ts, tw = times(cold[i]), times(warm[i])
        avg = float(ts.mean())
        r = {"avg_us": round(avg * 1e6, 2), "median_us": round(float(np.median(ts)) * 1e6, 2),
             "p10_us": round(float(np.percentile(ts, 10)) * 1e6, 2),
             "p90_us": round(float(np.percentile(ts, 90)) * 1e6, 2),
             "warm_avg_us": round(float(tw.mean()) * 1e6, 2),
             "warm_p10_us": round(float(np.percentile(tw, 10)) * 1e6, 2),
             "warm_p90_us": round(float(np.percentile(tw, 90)) * 1e6, 2)}
        if kind == "quant":
            r.update(gbs=round(work / avg / 1e9, 1), frac_hbm=round(work / avg / 1e9 / HBM_PEAK_GBS, 4),
                     bytes=int(work))
            q_bytes += work
            q_time += avg
        elif kind == "quant_next":
            r.update(gbs=round(work / avg / 1e9, 1), frac_hbm=round(work / avg / 1e9 / HBM_PEAK_GBS, 4),
                     bytes=int(work))
        elif kind in ("gemm8", "gemm16", "gemm8_next", "gemm16_next", "gemm8x_next"):
            # full-precision FP8 GEMMs (gemm8x) run on the BF16 matrix cores
            peak = BF16_PEAK_TFLOPS if kind.startswith(("gemm16", "gemm8x")) else FP8_PEAK_TFLOPS
            r.update(tflops=round(work / avg / 1e12, 1), frac_mfma=round(work / avg / 1e12 / peak, 4),
                     flops=work, peak_tflops=peak)
        rows[name] = r
        if kind in ("quant", "gemm8", "gemm16") and (dom is None or avg > dom[2]):
            dom = (name, kind, avg, work)

    out = {"metric": METRIC}
    out["value"] = round(q_bytes / q_time / 1e9, 1) if q_time > 0 else None
    out["unit"] = "GB/s"
    out["n_gpus"] = 1
    out["steps"] = args.steps
    out["warmup"] = args.warmup
    out["ms_per_step"] = round(ms_per_step, 3)
    out["higher_is_better"] = True
    out["scaling"] = "weak"
    out["vs_baseline"] = None
    out["dtype"] = "fp8-e4m3/e5m2 (fp32 accumulate, bf16 in/out)"
    out["data"] = "synthetic (seeded; shapes and distributions of the pages' workloads)"
    out["config"] = {"workload": "+".join(names), "parallelism": "none (1 GPU)",
                     "e4m3": {0: "e4m3fn", 1: "e4m3fnuz"}.get(e4, e4), "e5m2": {2: "e5m2", 3: "e5m2fnuz"}.get(e5, e5)}
    out["frac_hbm"] = round(out["value"] / HBM_PEAK_GBS, 4) if out["value"] else None
    g = rows.get("moe_grouped.grouped_gemm")
    if g:
        out["gemm_value"] = g["tflops"]
        out["gemm_unit"] = "TFLOP/s"
        out["gemm_frac_mfma"] = g["frac_mfma"]
    if dom is not None:
        name, kind, avg, work = dom
        traffic = stored_traffic(name, kind)
        if kind == "quant":
            out["roofline"] = {"kernel": name, "bound": "hbm", "achieved": round(work / avg / 1e9, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(work / avg / 1e9 / HBM_PEAK_GBS, 4), "traffic": traffic}
        else:
            peak = FP8_PEAK_TFLOPS if kind == "gemm8" else BF16_PEAK_TFLOPS
            out["roofline"] = {"kernel": name, "bound": "mfma", "achieved": round(work / avg / 1e12, 1),
                               "peak": peak, "unit": "TFLOP/s", "frac": round(work / avg / 1e12 / peak, 4),
                               "traffic": traffic}
        out["roofline"]["traffic_unit"] = "bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
        out["roofline"]["sources"] = sources_digest(kind)
    out["timing"] = ("per row: HIP events on the launch stream; avg/median/p10/p90 with a 512 MiB read "
                     "between calls (cold: caches hold neither inputs nor dirty lines; value, gemm_value and "
                     "roofline use these), warm_* back to back")
    out["clocks"] = clocks.summary()
    out["rows"] = rows
    out["inputs_sha256"] = input_digests(wls)
    if not args.no_cpu_baseline and "moe_grouped" in wls:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline(wls, args.cpu_budget)
    print(json.dumps(out), flush=True)


class ClockSampler:
    """Samples the GPU's shader and memory clocks while the timed steps run: the
    current DPM level of card*/device/pp_dpm_sclk and pp_dpm_mclk (the line marked
    '*'), or rocm-smi's JSON where sysfs does not show them."""

    def __init__(self, period_s=0.02):
        import glob
        import threading
        self.period = period_s
        self.samples = {"sclk": [], "mclk": []}
        self.files = {}
        for k in ("sclk", "mclk"):
            fs = sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{k}"))
            if fs:
                self.files[k] = fs
        self.source = "sysfs pp_dpm_*" if self.files else "rocm-smi --showclocks"
        if not self.files:
            self.period = 0.25
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._loop, daemon=True)

    @staticmethod
    def _mhz(text):
        import re
        m = re.search(r"(\d+)\s*[Mm][Hh]z", text)
        return int(m.group(1)) if m else None

    def _read(self):
        if self.files:
            for k, fs in self.files.items():
                for fn in fs:
                    try:
                        with open(fn) as fh:
                            for line in fh:
                                if "*" in line:
                                    v = self._mhz(line)
                                    if v:
                                        self.samples[k].append(v)
                    except OSError:
                        pass
            return
        import subprocess
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=5)
            d = json.loads(r.stdout) if r.returncode == 0 else {}
        except (OSError, ValueError, subprocess.TimeoutExpired):
            return
        for card in d.values():
            if not isinstance(card, dict):
                continue
            for key, val in card.items():
                kl = key.lower()
                v = self._mhz(str(val)) if isinstance(val, str) else None
                if v and kl.startswith("sclk"):
                    self.samples["sclk"].append(v)
                elif v and kl.startswith("mclk"):
                    self.samples["mclk"].append(v)

    def _loop(self):
        while not self._stop.is_set():
            self._read()
            self._stop.wait(self.period)

    def start(self):
        self._t.start()

    def stop(self):
        self._stop.set()
        self._t.join(timeout=10)

    def summary(self):
        import numpy as np
        out = {"source": self.source}
        for k, v in self.samples.items():
            if v:
                a = np.array(v)
                out[k + "_mhz"] = {"min": int(a.min()), "median": int(np.median(a)), "max": int(a.max()),
                                   "samples": int(a.size)}
            else:
                out[k + "_mhz"] = None
        return out


def build_step_subset(f, torch, dev, wls, dev_of):
    """build_step restricted to the workloads present in wls (for profiling runs):
    absent workloads get tiny stand-ins whose calls are then dropped."""
    import synth
    full_names = ["linear_tensorwise", "linear_rowwise", "expert_colwise", "moe_grouped", "moe_block_mx"]
    if set(wls) == set(full_names):
        return build_step(f, torch, dev, wls, dev_of)
    small = {
        "linear_tensorwise": synth.linear_tensorwise,
        "linear_rowwise": lambda: synth.linear_rowwise(M=64, K=128, N=128),
        "expert_colwise": lambda: synth.expert_colwise(E=1, R=64, C=64),
        "moe_grouped": lambda: synth.moe_grouped(tokens=64, topk=2, E=4, N=64, K=128, n_empty=0),
        "moe_block_mx": lambda: synth.moe_block_mx(E=2, K=256, N=256, rows=64),
    }
    allw = {n: (wls[n] if n in wls else small[n]()) for n in full_names}
    st = build_step(f, torch, dev, allw, dev_of)
    st.calls = [c for c in st.calls if c[0].split(".")[0] in wls]
    return st


if __name__ == "__main__":
    main()
