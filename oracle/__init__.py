"""Plain, slow CPU oracle for dynamic FP8 quantization and scaled FP8 GEMMs.

TEST INFRASTRUCTURE ONLY: the library never imports this package. Only the
tests, the smoke check and the benchmark's CPU-baseline leg may use it. The C
sources next to this file (codec.c, quant.c, gemm.c) hold all the arithmetic;
this module only marshals numpy arrays through ctypes. It shares no code with
the HIP path.

Citations for each function are in fp8_oracle.h and the C sources.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SOURCES = ["codec.c", "quant.c", "gemm.c", "norm.c"]

E4M3FN, E4M3FNUZ, E5M2, E5M2FNUZ = 0, 1, 2, 3
FORMATS = {"e4m3fn": E4M3FN, "e4m3fnuz": E4M3FNUZ, "e5m2": E5M2, "e5m2fnuz": E5M2FNUZ}
MX_POW2_FLOOR, MX_OCP = 0, 1
SCALE_TENSOR, SCALE_ROW, SCALE_BLOCK128, SCALE_MX32 = 0, 1, 2, 3

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (IEEE arithmetic: no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    srcs = [os.path.join(_HERE, s) for s in _SOURCES]
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wno-unknown-pragmas",
           "-o", tmp] + srcs + ["-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, D, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_float
    I = ctypes.c_int
    U8 = ctypes.c_uint8
    sig = {
        "orc_fp8_max": (D, [I]),
        "orc_fp8_decode": (D, [I, U8]),
        "orc_fp8_encode": (U8, [I, F]),
        "orc_bf16_to_f32": (F, [ctypes.c_uint16]),
        "orc_decode_array": (None, [I, P, I64, P]),
        "orc_encode_array": (None, [I, P, I64, P]),
        "orc_scale_from_amax": (D, [I, F, D, P, P]),
        "orc_mx_scale_from_amax": (U8, [I, I, F, D, P, P]),
        "orc_quant_elem": (U8, [I, ctypes.c_uint16, F]),
        "orc_quant_tensor": (None, [P, I64, I, D, P, P, P, P]),
        "orc_quant_row": (None, [P, I64, I64, I64, I, D, P, P, P, I]),
        "orc_norm_row": (None, [P, P, P, I64, I64, I, D, P]),
        "orc_norm_stats": (None, [P, I64, I64, P, P]),
        "orc_norm_quant_row": (None, [P, P, P, I64, I64, I, D, I, D, P, P, P, P]),
        "orc_quant_col": (None, [P, I64, I64, I64, I, D, P, P, P, I]),
        "orc_quant_block": (None, [P, I64, I64, I64, I64, I64, I, D, P, P, P, I]),
        "orc_quant_mx": (None, [P, I64, I64, I64, I, I, D, P, P, I]),
        "orc_scaled_mm": (None, [P, I, P, I, I, P, P, I64, I64, I64, P, I]),
        "orc_scaled_mm_sample": (None, [P, I, P, I, I, P, P, I64, I64, I64, P, P, I64, P]),
        "orc_grouped_mm": (None, [P, I, P, I, I, P, P, P, I32, I64, I64, I64, P, I]),
        "orc_grouped_mm_sample": (None, [P, I, P, I, I, P, P, P, I32, I64, I64, I64, P, P, I64, P]),
        "orc_wgrad_bf16": (None, [P, P, I64, I64, I64, P, I]),
        "orc_wgrad_bf16_sample": (None, [P, P, I64, I64, I64, P, P, I64, P]),
        "orc_scaled_mm_abs": (None, [P, I, P, I, I, P, P, I64, I64, I64, P, I]),
        "orc_scaled_mm_abs_sample": (None, [P, I, P, I, I, P, P, I64, I64, I64, P, P, I64, P]),
        "orc_grouped_mm_abs": (None, [P, I, P, I, I, P, P, P, I32, I64, I64, I64, P, I]),
        "orc_grouped_mm_abs_sample": (None, [P, I, P, I, I, P, P, P, I32, I64, I64, I64, P, P, I64, P]),
        "orc_wgrad_bf16_abs": (None, [P, P, I64, I64, I64, P, I]),
        "orc_wgrad_bf16_abs_sample": (None, [P, P, I64, I64, I64, P, P, I64, P]),
        "orc_threads_used": (I, [I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _fmt(f) -> int:
    return FORMATS[f] if isinstance(f, str) else int(f)


def _u16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, "bf16 inputs are passed as uint16 bit patterns"
    return x


# ---- codec -------------------------------------------------------------------

def fp8_max(fmt) -> float:
    return _load().orc_fp8_max(_fmt(fmt))


def decode(fmt, codes) -> np.ndarray:
    q = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(q.shape, dtype=np.float64)
    _load().orc_decode_array(_fmt(fmt), _p(q), q.size, _p(out))
    return out


def encode(fmt, y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    _load().orc_encode_array(_fmt(fmt), _p(y), y.size, _p(out))
    return out


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def scale_from_amax(fmt, amax: float, eps: float = 1e-12):
    """Returns (scale64, scale32, inv32)."""
    s = ctypes.c_float()
    i = ctypes.c_float()
    s64 = _load().orc_scale_from_amax(_fmt(fmt), float(amax), float(eps), ctypes.byref(s), ctypes.byref(i))
    return s64, np.float32(s.value), np.float32(i.value)


def mx_scale_from_amax(fmt, amax: float, mode: int = MX_POW2_FLOOR, eps: float = 1e-12):
    """Returns (e8m0, scale32, inv32)."""
    s = ctypes.c_float()
    i = ctypes.c_float()
    e = _load().orc_mx_scale_from_amax(_fmt(fmt), int(mode), float(amax), float(eps), ctypes.byref(s), ctypes.byref(i))
    return int(e), np.float32(s.value), np.float32(i.value)


def quant_elem(fmt, x_bf16: int, scale: float) -> int:
    return int(_load().orc_quant_elem(_fmt(fmt), int(x_bf16), float(scale)))


# ---- quantization ------------------------------------------------------------

def quant_tensor(x, fmt, eps=1e-12):
    x = _u16(x)
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.empty(1, np.float32)
    i = np.empty(1, np.float32)
    a = np.empty(1, np.float32)
    _load().orc_quant_tensor(_p(x), x.size, _fmt(fmt), float(eps), _p(q), _p(s), _p(i), _p(a))
    return q, s, i


def norm_row(x, gamma, beta=None, layer=False, norm_eps=1e-6):
    """RMSNorm (layer=False) or LayerNorm of each row of x, stored as bf16
    (see norm.c for the steps). x [rows][cols], gamma/beta [cols] bf16 bits."""
    x, g = _u16(x), _u16(gamma)
    b = _u16(beta) if beta is not None else None
    rows, cols = x.shape
    y = np.empty((rows, cols), np.uint16)
    _load().orc_norm_row(_p(x), _p(g), _p(b), rows, cols, int(bool(layer)), float(norm_eps), _p(y))
    return y


def norm_stats(x):
    """(s1, s2) per row of x [rows][cols] bf16 bits: the exact sums of x and x^2,
    each rounded once to fp64 (norm.c, step 1)."""
    x = _u16(x)
    rows, cols = x.shape
    s1 = np.empty(rows, np.float64)
    s2 = np.empty(rows, np.float64)
    _load().orc_norm_stats(_p(x), rows, cols, _p(s1), _p(s2))
    return s1, s2


def norm_quant_row(x, gamma, beta=None, layer=False, norm_eps=1e-6, fmt="e4m3fn", eps=1e-12):
    """The normalization, then quant_row of its bf16 output ("FP8 Training:
    Quantization, Autograd, Torchao", section 8: the norm's output write and
    the next layer's amax pass are one memory pass when fused).
    Returns (y, q, scale, inv)."""
    y = norm_row(x, gamma, beta, layer, norm_eps)
    q, s, i = quant_row(y, fmt, eps)
    return y, q, s, i


def quant_dual(gy, x, g_fmt, x_fmt, eps=1e-12):
    """The operands of the all-FP8 Linear backward ("FP8 Training:
    Quantization, Autograd, Torchao", section 4: grad_output row-major for the
    grad-input GEMM and transposed for the grad-weight GEMM, the input
    column-major): quant_tensor of gy and of x, laid out as
    gq = q(gy) [M][N], gqT = q(gy)^T [N][M] and xqT = q(x)^T [K][M].
    Quantization is elementwise under one scale per tensor, so a transposed
    output is exactly the transpose of the row-major one.
    Returns (gq, gqT, g_scale, g_inv, xqT, x_scale, x_inv)."""
    gq, gs, gi = quant_tensor(gy, g_fmt, eps)
    xq, xs, xi = quant_tensor(x, x_fmt, eps)
    return gq, np.ascontiguousarray(gq.T), gs, gi, np.ascontiguousarray(xq.T), xs, xi


def _brc(x):
    if x.ndim == 2:
        return 1, x.shape[0], x.shape[1]
    assert x.ndim == 3
    return x.shape


def quant_row(x, fmt, eps=1e-12, threads=0):
    x = _u16(x)
    b, r, c = _brc(x)
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.empty(x.shape[:-1], np.float32)
    i = np.empty(x.shape[:-1], np.float32)
    _load().orc_quant_row(_p(x), b, r, c, _fmt(fmt), float(eps), _p(q), _p(s), _p(i), int(threads))
    return q, s, i


def quant_col(x, fmt, eps=1e-12, threads=0):
    """Column groups; returns the transposed codes qT [..., cols, rows]."""
    x = _u16(x)
    b, r, c = _brc(x)
    shape_t = x.shape[:-2] + (c, r)
    q = np.empty(shape_t, dtype=np.uint8)
    s = np.empty(x.shape[:-2] + (c,), np.float32)
    i = np.empty(x.shape[:-2] + (c,), np.float32)
    _load().orc_quant_col(_p(x), b, r, c, _fmt(fmt), float(eps), _p(q), _p(s), _p(i), int(threads))
    return q, s, i


def quant_block(x, br, bc, fmt, eps=1e-12, threads=0):
    x = _u16(x)
    b, r, c = _brc(x)
    nbr, nbc = -(-r // br), -(-c // bc)
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.empty(x.shape[:-2] + (nbr, nbc), np.float32)
    i = np.empty(x.shape[:-2] + (nbr, nbc), np.float32)
    _load().orc_quant_block(_p(x), b, r, c, int(br), int(bc), _fmt(fmt), float(eps), _p(q), _p(s), _p(i), int(threads))
    return q, s, i


def quant_mx(x, fmt, mode=MX_POW2_FLOOR, eps=1e-12, threads=0):
    x = _u16(x)
    b, r, c = _brc(x)
    assert c % 32 == 0
    q = np.empty(x.shape, dtype=np.uint8)
    e = np.empty(x.shape[:-1] + (c // 32,), np.uint8)
    _load().orc_quant_mx(_p(x), b, r, c, _fmt(fmt), int(mode), float(eps), _p(q), _p(e), int(threads))
    return q, e


# ---- GEMMs -------------------------------------------------------------------

def scaled_mm(a, fa, b, fb, scaling, a_inv, b_inv, threads=0, absolute=False):
    """a [M,K] codes, b [N,K] codes -> fp64 [M,N]. absolute=True: sum of |products| x |scales|."""
    a = np.ascontiguousarray(a, np.uint8)
    b = np.ascontiguousarray(b, np.uint8)
    M, K = a.shape
    N = b.shape[0]
    a_inv = np.ascontiguousarray(a_inv, np.float32)
    b_inv = np.ascontiguousarray(b_inv, np.float32)
    out = np.empty((M, N), np.float64)
    fn = _load().orc_scaled_mm_abs if absolute else _load().orc_scaled_mm
    fn(_p(a), _fmt(fa), _p(b), _fmt(fb), int(scaling), _p(a_inv), _p(b_inv), M, N, K, _p(out), int(threads))
    return out


def scaled_mm_sample(a, fa, b, fb, scaling, a_inv, b_inv, rows, cols, absolute=False):
    a = np.ascontiguousarray(a, np.uint8)
    b = np.ascontiguousarray(b, np.uint8)
    M, K = a.shape
    N = b.shape[0]
    rows = np.ascontiguousarray(rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    a_inv = np.ascontiguousarray(a_inv, np.float32)
    b_inv = np.ascontiguousarray(b_inv, np.float32)
    out = np.empty(rows.shape, np.float64)
    fn = _load().orc_scaled_mm_abs_sample if absolute else _load().orc_scaled_mm_sample
    fn(_p(a), _fmt(fa), _p(b), _fmt(fb), int(scaling), _p(a_inv), _p(b_inv), M, N, K, _p(rows), _p(cols),
       rows.size, _p(out))
    return out


def _scale_arr(s, scaling):
    return np.ascontiguousarray(s, np.uint8 if scaling == SCALE_MX32 else np.float32)


def grouped_mm(a, fa, b, fb, scaling, a_scale, b_scale, offsets, threads=0, absolute=False):
    """a [Mtot,K], b [E,N,K], offsets int32 [E+1] (host) -> fp64 [Mtot,N]."""
    a = np.ascontiguousarray(a, np.uint8)
    b = np.ascontiguousarray(b, np.uint8)
    Mtot, K = a.shape
    E, N, _ = b.shape
    off = np.ascontiguousarray(offsets, np.int32)
    sa, sb = _scale_arr(a_scale, scaling), _scale_arr(b_scale, scaling)
    out = np.empty((Mtot, N), np.float64)
    fn = _load().orc_grouped_mm_abs if absolute else _load().orc_grouped_mm
    fn(_p(a), _fmt(fa), _p(b), _fmt(fb), int(scaling), _p(sa), _p(sb), _p(off), E, Mtot, N, K, _p(out), int(threads))
    return out


def grouped_mm_sample(a, fa, b, fb, scaling, a_scale, b_scale, offsets, rows, cols, absolute=False):
    a = np.ascontiguousarray(a, np.uint8)
    b = np.ascontiguousarray(b, np.uint8)
    Mtot, K = a.shape
    E, N, _ = b.shape
    off = np.ascontiguousarray(offsets, np.int32)
    sa, sb = _scale_arr(a_scale, scaling), _scale_arr(b_scale, scaling)
    rows = np.ascontiguousarray(rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    out = np.empty(rows.shape, np.float64)
    fn = _load().orc_grouped_mm_abs_sample if absolute else _load().orc_grouped_mm_sample
    fn(_p(a), _fmt(fa), _p(b), _fmt(fb), int(scaling), _p(sa), _p(sb), _p(off), E, Mtot, N, K, _p(rows), _p(cols),
       rows.size, _p(out))
    return out


def wgrad_bf16(g, x, threads=0, absolute=False):
    """g [M,N] bf16 bits, x [M,K] bf16 bits -> dW [N,K] fp64."""
    g, x = _u16(g), _u16(x)
    M, N = g.shape
    K = x.shape[1]
    out = np.empty((N, K), np.float64)
    fn = _load().orc_wgrad_bf16_abs if absolute else _load().orc_wgrad_bf16
    fn(_p(g), _p(x), M, N, K, _p(out), int(threads))
    return out


def wgrad_bf16_sample(g, x, ns, ks, absolute=False):
    g, x = _u16(g), _u16(x)
    M, N = g.shape
    K = x.shape[1]
    ns = np.ascontiguousarray(ns, np.int64)
    ks = np.ascontiguousarray(ks, np.int64)
    out = np.empty(ns.shape, np.float64)
    fn = _load().orc_wgrad_bf16_abs_sample if absolute else _load().orc_wgrad_bf16_sample
    fn(_p(g), _p(x), M, N, K, _p(ns), _p(ks), ns.size, _p(out))
    return out


def grouped_wgrad_bf16(g, x, offsets, threads=0, absolute=False):
    """The MoE weight gradient over expert row ranges ("FP8 training on AMD
    GPUs with TorchTitan and TorchAO", section "Scaling FP8 to MoE
    Architectures": expert e owns rows [off[e], off[e+1]); Figure 1 caption:
    the weight-update GEMM stays in BF16): gw[e] = wgrad_bf16 of the expert's
    rows of g and x, zeros for an expert with no rows. Returns [E][N][K] in
    fp64, before the final bf16 rounding (absolute=True: sums of |products|)."""
    off = np.asarray(offsets, dtype=np.int64)
    E = off.size - 1
    N, K = g.shape[1], x.shape[1]
    out = np.zeros((E, N, K), dtype=np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            out[e] = wgrad_bf16(np.ascontiguousarray(g[a:b]), np.ascontiguousarray(x[a:b]), threads, absolute)
    return out


def threads_used(threads=0) -> int:
    return int(_load().orc_threads_used(int(threads)))
