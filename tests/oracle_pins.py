"""Independent references used to pin the oracle (no GPU, no HIP library).

Nothing here re-types the oracle's C code: the FP8 value tables come from
torch's own float8 dtypes, rounding to fp32 is done on exact rationals, and
the encoder reference is a nearest-value search over the table.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

TORCH_DTYPES = {
    "e4m3fn": torch.float8_e4m3fn,
    "e4m3fnuz": torch.float8_e4m3fnuz,
    "e5m2": torch.float8_e5m2,
    "e5m2fnuz": torch.float8_e5m2fnuz,
}
FNUZ = {"e4m3fn": False, "e4m3fnuz": True, "e5m2": False, "e5m2fnuz": True}


def torch_decode_table(fmt: str) -> np.ndarray:
    """Value of each of the 256 codes, as torch's float8 dtype defines it."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(TORCH_DTYPES[fmt]).to(torch.float64).numpy()


def torch_encode(fmt: str, y: np.ndarray) -> np.ndarray:
    """torch's CPU fp32 -> float8 conversion (round to nearest even; not saturating,
    so only meaningful for |y| <= max)."""
    t = torch.from_numpy(np.ascontiguousarray(y, np.float32))
    return t.to(TORCH_DTYPES[fmt]).view(torch.uint8).numpy()


def positive_grid(fmt: str):
    """(codes, values) of the finite non-negative codes in increasing order."""
    tab = torch_decode_table(fmt)
    codes = np.arange(128)
    vals = tab[:128]
    ok = np.isfinite(vals)
    return codes[ok], vals[ok]


def nearest_encode(fmt: str, y: np.ndarray) -> np.ndarray:
    """Brute-force saturating round-to-nearest-even encoder: search the sorted value
    grid for the two neighbours of |y|, take the nearer, on a tie the even code."""
    codes, vals = positive_grid(fmt)
    y = np.asarray(y, np.float32)
    a = np.abs(y.astype(np.float64))
    vmax = vals[-1]
    idx = np.searchsorted(vals, np.minimum(a, vmax), side="left")
    idx = np.clip(idx, 0, len(vals) - 1)
    lo = np.clip(idx - 1, 0, len(vals) - 1)
    dhi = vals[idx] - a
    dlo = a - vals[lo]
    pick = idx.copy()
    take_lo = (dlo < dhi) | ((dlo == dhi) & (codes[lo] % 2 == 0) & (lo != idx))
    pick[take_lo] = lo[take_lo]
    exact = vals[idx] == a
    pick[exact] = idx[exact]
    pick[a >= vmax] = len(vals) - 1
    code = codes[pick].astype(np.uint8)
    neg = np.signbit(y)
    if FNUZ[fmt]:
        out = np.where(code == 0, 0, code | (neg.astype(np.uint8) << 7))
    else:
        out = code | (neg.astype(np.uint8) << 7)
    return out.astype(np.uint8)


def rn32(fr: Fraction) -> np.float32:
    """Exact rational -> nearest fp32, ties to even (normal range)."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]

    def key(c):
        return (abs(Fraction(float(c)) - fr), int(np.array(c, np.float32).view(np.uint32)) & 1)

    return min(cands, key=key)


def exact_f32_product(x: float, s: float) -> np.float32:
    return rn32(Fraction(float(x)) * Fraction(float(s)))


def fp8_ulp(fmt: str, y: float) -> float:
    """Spacing of the fp8 grid at |y| (the subnormal quantum below the smallest normal)."""
    _, vals = positive_grid(fmt)
    a = abs(float(y))
    i = int(np.searchsorted(vals, a, side="right"))
    i = min(max(i, 1), len(vals) - 1)
    return float(vals[i] - vals[i - 1])


def quant_chain_reference(fmt: str, x_bits: np.ndarray, eps: float, fmax: float):
    """The quantization chain on one group, in exact rational arithmetic plus the
    brute-force encoder: amax, fp64 scale, fp32 product, clamp, nearest-even cast."""
    xf = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    amax = max(abs(v) for v in xf.ravel()) if xf.size else 0.0
    d = max(Fraction(float(amax)), Fraction(eps))
    s64 = float(Fraction(fmax) / d)  # the fp64 quotient, correctly rounded
    scale = rn32(Fraction(s64))
    inv = rn32(1 / Fraction(s64)) if s64 != 0 else np.float32(np.inf)
    y = np.array([exact_f32_product(v, float(scale)) for v in xf.ravel()], np.float32)
    y = np.clip(y, -np.float32(fmax), np.float32(fmax))
    q = nearest_encode(fmt, y).reshape(x_bits.shape)
    return q, np.float32(scale), np.float32(inv)
