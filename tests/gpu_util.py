"""Helpers for the GPU parity tests: host <-> device marshalling and the error metric.

These helpers never compute an expected value: expected values come from the
oracle package only.
"""
from __future__ import annotations

import numpy as np
import pytest

try:
    import torch
except Exception:  # pragma: no cover
    torch = None


def have_gpu() -> bool:
    return torch is not None and torch.cuda.is_available()


def lib():
    import fp8_dynamic_scaling_amd as f
    f.load()
    return f


def to_dev_bf16(x_bits: np.ndarray):
    """numpy uint16 bf16 bit patterns -> torch.bfloat16 tensor on cuda:0 (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16))
    return t.to("cuda:0").view(torch.bfloat16)


def to_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def u8(t) -> np.ndarray:
    return t.view(torch.uint8).cpu().numpy()


def f32(t) -> np.ndarray:
    return t.float().cpu().numpy()


def empty_u8(shape, guard: int = 0):
    """uint8 device buffer; with guard > 0, padded by `guard` canary bytes on each side
    (returns (view, full_buffer))."""
    n = int(np.prod(shape))
    full = torch.full((n + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda:0")
    if guard:
        # keep the view 16-byte aligned
        assert guard % 256 == 0
    return full[guard:guard + n].view(shape), full


def check_guard(full, guard: int):
    if guard:
        h = full.cpu().numpy()
        assert np.all(h[:guard] == 0xA5) and np.all(h[-guard:] == 0xA5), "write outside the output buffer"


def rel_err(y: np.ndarray, r: np.ndarray) -> float:
    """max_i |y_i - r_i| / max(|r_i|, 1e-3 * max_j |r_j|)."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    peak = np.abs(r).max()
    den = np.maximum(np.abs(r), 1e-3 * peak)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(y - r) / den))


TOL_BF16 = 1e-2
TOL_F32 = 2e-3

# Componentwise bound. The gfx950 FP8 (and BF16) matrix-core instructions do not
# accumulate at full fp32 precision inside one instruction: measured on MI355X, the
# error of one 128-product FP8 instruction reaches 2^-12 of its largest product
# (the older 32-deep FP8 instruction behaves the same). Summed over K, the
# accumulation error of an output is below 2^-12 * S, S = sum_k |a_k b_k| |scales|
# (componentwise dot-product error analysis), so each element must satisfy
#   |y - r| <= C_ACC * S + C_OUT * |r|
# with C_ACC = 2^-9 (8x margin) and C_OUT the output rounding (bf16 half-ulp with
# margin, or a few fp32 ulps for the scale multiplies and fp32 output).
C_ACC = 2.0 ** -9
C_OUT_BF16 = 2.0 ** -8
C_OUT_F32 = 2.0 ** -21


def norm_err(y, r) -> float:
    """max_i |y_i - r_i| / max_j |r_j| (relative error in the max norm)."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    peak = np.abs(r).max() if r.size else 0.0
    return float(np.abs(y - r).max() / peak) if peak > 0 else float(np.abs(y - r).max())


def check_gemm(y, r, S, out_bf16: bool, label: str = "", exact: bool = False):
    """The GEMM acceptance test against the oracle's fp64 result r.

    exact=True (full-precision accumulation, use_fast_accum off): the floored
    elementwise error max|y - r| / max(|r|, 1e-3 max|r|) and the normwise error
    max|y - r| / max|r| are both within 1e-2 (bf16 out) or 2e-3 (fp32 out).

    exact=False (the FP8 matrix-core instructions): the normwise error within the same
    tolerance, and every element within the componentwise bound of the hardware's
    per-instruction product alignment (C_ACC above). The floored elementwise error is
    printed: on outputs near the floor that alignment exceeds it.
    Returns (normwise error, worst componentwise ratio, floored elementwise error)."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    S = np.asarray(S, np.float64)
    assert np.all(np.isfinite(y)), f"{label}: non-finite output"
    tol = TOL_BF16 if out_bf16 else TOL_F32
    ne = norm_err(y, r)
    bound = C_ACC * S + (C_OUT_BF16 if out_bf16 else C_OUT_F32) * np.abs(r) + 1e-30
    ratio = float(np.max(np.abs(y - r) / bound)) if r.size else 0.0
    fe = rel_err(y, r)
    mode = "exact" if exact else "fast"
    print(f"{label} [{mode}]: normwise {ne:.3e}  componentwise/bound {ratio:.3f}  floored-elementwise {fe:.3e}",
          flush=True)
    assert ne <= tol, (label, mode, ne)
    if exact:
        assert fe <= tol, (label, mode, fe)
    else:
        assert ratio <= 1.0, (label, mode, ratio)
    return ne, ratio, fe

gpu = pytest.mark.gpu


def kpack(q, g: int = 16):
    """[..., R, C] row-major codes -> the flat k-packed bytes: per batch slice, chunk
    (r // g, c // 64) of g x 64 bytes at ((r // g) * (C // 64) + c // 64) * 64 g, row
    r % g at 64 (r % g) in it. g = 16: fp8_quant_row_kpacked / fp8_quant_col_kpacked;
    g = 2: fp8_quant_row_kpaired's pair-interleaved rows."""
    *lead, R, C = q.shape
    B = int(np.prod(lead)) if lead else 1
    return np.ascontiguousarray(q.reshape(B, R // g, g, C // 64, 64).transpose(0, 1, 3, 2, 4)).reshape(-1)
