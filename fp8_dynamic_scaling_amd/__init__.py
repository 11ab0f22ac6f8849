"""Python binding of libfp8dyn.so (include/fp8dyn.h) for MI355X (gfx950).

Argument marshalling only: every function has the C name, takes torch tensors
that already live on the GPU, passes their data pointers, sizes and the
current HIP stream to the C ABI, and raises Fp8Error on a non-OK status. All
work runs in the library's HIP kernels; there is no fallback. Loading fails
loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8dyn.so")

# enums (same values as include/fp8dyn.h)
E4M3FN, E4M3FNUZ, E5M2, E5M2FNUZ, E4M3_NATIVE, E5M2_NATIVE = range(6)
OK, ERR_INVALID_ARGUMENT, ERR_ALIGNMENT, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE = range(6)
SCALE_TENSOR, SCALE_ROW, SCALE_BLOCK128, SCALE_MX32 = range(4)
OUT_BF16, OUT_F32 = range(2)
MX_POW2_FLOOR, MX_OCP = range(2)
RECIPE_TENSORWISE, RECIPE_ROWWISE_BF16_WGRAD = range(2)

EXPORTS = [
    "fp8_probe", "fp8_status_string", "fp8_last_device_error", "fp8_format_max",
    "fp8_quant_tensor", "fp8_quant_tensor_ws_bytes", "fp8_quant_row", "fp8_quant_row_kpacked", "fp8_quant_row_kpaired", "fp8_quant_col",
    "fp8_quant_col_kpacked",
    "fp8_quant_col_ws_bytes", "fp8_quant_col_noalloc", "fp8_quant_dual", "fp8_quant_dual_ws_bytes", "fp8_norm_quant_row",
    "fp8_quant_block", "fp8_quant_mx", "fp8_quant_mx_kpacked", "fp8_quant_mx_kpaired",
    "fp8_scaled_mm", "fp8_scaled_mm_kpacked",
    "fp8_grouped_mm", "fp8_grouped_mm_kpacked", "fp8_wgrad_bf16", "fp8_grouped_wgrad_bf16", "fp8_linear_fwd", "fp8_linear_bwd",
    "fp8_linear_ws_bytes", "fp8_validate_offsets",
]


class Fp8Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.fp8_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn}: status {status} ({msg})")


_lib = None


def load(path: str = LIB_PATH):
    """Loads the library and declares the C signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with fp8_dynamic_scaling_amd/build.py "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I64, I32, I, D, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int,
                             ctypes.c_double, ctypes.c_size_t)
    sig = {
        "fp8_probe": (I, [I, P, P]),
        "fp8_status_string": (ctypes.c_char_p, [I]),
        "fp8_last_device_error": (I, []),
        "fp8_format_max": (D, [I]),
        "fp8_quant_tensor": (I, [P, I64, I, D, P, P, P, P, SZ, P]),
        "fp8_quant_tensor_ws_bytes": (SZ, []),
        "fp8_quant_row": (I, [P, I64, I64, I64, I, D, P, P, P, P]),
        "fp8_quant_row_kpacked": (I, [P, I64, I64, I64, I, D, P, P, P, P]),
        "fp8_quant_row_kpaired": (I, [P, I64, I64, I64, I, D, P, P, P, P]),
        "fp8_quant_col": (I, [P, I64, I64, I64, I, D, P, P, P, P, SZ, P]),
        "fp8_quant_col_kpacked": (I, [P, I64, I64, I64, I, D, P, P, P, P, SZ, P]),
        "fp8_quant_col_ws_bytes": (SZ, [I64, I64, I64]),
        "fp8_quant_col_noalloc": (I, [P, I64, I64, I64, I, D, P, P, P, P]),
        "fp8_quant_dual": (I, [P, P, I64, I64, I64, I, I, D, P, P, P, P, P, P, P, P, SZ, P]),
        "fp8_norm_quant_row": (I, [P, P, P, I64, I64, I, D, I, D, P, P, P, P, P]),
        "fp8_quant_dual_ws_bytes": (SZ, []),
        "fp8_quant_block": (I, [P, I64, I64, I64, I, I, I, D, P, P, P, P]),
        "fp8_quant_mx": (I, [P, I64, I64, I64, I, I, D, P, P, P]),
        "fp8_quant_mx_kpacked": (I, [P, I64, I64, I64, I, I, D, P, P, P]),
        "fp8_quant_mx_kpaired": (I, [P, I64, I64, I64, I, I, D, P, P, P]),
        "fp8_scaled_mm": (I, [P, I, P, I, I, P, P, I64, I64, I64, I, P, I, P]),
        "fp8_scaled_mm_kpacked": (I, [P, I, P, I, I, P, P, I64, I64, I64, I, P, I, P]),
        "fp8_grouped_mm": (I, [P, I, P, I, I, P, P, P, I32, I64, I64, I64, I, P, I, P]),
        "fp8_grouped_mm_kpacked": (I, [P, I, P, I, I, P, P, P, I32, I64, I64, I64, I, P, I, P]),
        "fp8_wgrad_bf16": (I, [P, P, I64, I64, I64, P, P]),
        "fp8_grouped_wgrad_bf16": (I, [P, P, P, I32, I64, I64, I64, P, P]),
        "fp8_linear_fwd": (I, [P, P, I64, I64, I64, I, D, I, I, P, P, SZ, P]),
        "fp8_linear_bwd": (I, [P, P, P, I64, I64, I64, I, D, P, P, P, SZ, P]),
        "fp8_linear_ws_bytes": (SZ, [I64, I64, I64, I]),
        "fp8_validate_offsets": (I, [P, I32, I64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != OK:
        raise Fp8Error(fn, status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _brc(x):
    if x.dim() == 2:
        return 1, x.shape[0], x.shape[1]
    if x.dim() == 3:
        return x.shape[0], x.shape[1], x.shape[2]
    if x.dim() == 1:
        return 1, 1, x.shape[0]
    raise ValueError("x must have 1 to 3 dimensions")


def _arg(fn, name, t, nbytes, esize=None):
    """Marshalling check of one operand: a contiguous GPU tensor of at least nbytes
    bytes (with elements of esize bytes when given). None passes when nbytes is 0."""
    if t is None:
        if nbytes > 0:
            raise ValueError(f"{fn}: {name} is required")
        return
    if not t.is_cuda:
        raise ValueError(f"{fn}: {name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be contiguous")
    if esize is not None and t.element_size() != esize:
        raise ValueError(f"{fn}: {name} must have {esize}-byte elements (got {t.dtype})")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{fn}: {name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")


def _offsets(fn, offsets, E):
    """Device int32 offsets of E + 1 entries (an int64 tensor, torch.cumsum's default,
    would be read as pairs of int32 words)."""
    import torch
    if offsets is None:
        raise ValueError(f"{fn}: offsets is required")
    if offsets.dtype != torch.int32:
        raise ValueError(f"{fn}: offsets must be int32 (got {offsets.dtype})")
    if offsets.numel() != E + 1:
        raise ValueError(f"{fn}: offsets must hold E + 1 = {E + 1} entries (got {offsets.numel()})")
    _arg(fn, "offsets", offsets, 4 * (E + 1))


def _gemm_scale_bytes(scaling, M, N, K, E=1):
    """Bytes of (a_scale, b_scale) for a GEMM's scaling."""
    if scaling == SCALE_TENSOR:
        return 4, 4
    if scaling == SCALE_ROW:
        return 4 * M, 4 * E * N
    if scaling == SCALE_BLOCK128:
        return 4 * M * (K // 128), 4 * E * (N // 128) * (K // 128)
    return M * (K // 32), E * N * (K // 32)


# ---- device facts -------------------------------------------------------------

def fp8_probe(device: int = 0):
    """Returns (e4m3_native, e5m2_native) format ids measured on the device."""
    lib = load()
    e4, e5 = ctypes.c_int(), ctypes.c_int()
    _check("fp8_probe", lib.fp8_probe(int(device), ctypes.byref(e4), ctypes.byref(e5)))
    return e4.value, e5.value


def fp8_status_string(status: int) -> str:
    return load().fp8_status_string(int(status)).decode()


def fp8_last_device_error() -> int:
    return load().fp8_last_device_error()


def fp8_format_max(fmt: int) -> float:
    return load().fp8_format_max(int(fmt))


# ---- quantization -------------------------------------------------------------

def fp8_quant_tensor_ws_bytes() -> int:
    return load().fp8_quant_tensor_ws_bytes()


def fp8_quant_tensor(x, fmt, eps, q, scale, inv_scale, ws, stream=None):
    fn, n = "fp8_quant_tensor", x.numel()
    _arg(fn, "x", x, 2 * n, 2)
    _arg(fn, "q", q, n, 1)
    _arg(fn, "scale", scale, 4, 4)
    _arg(fn, "inv_scale", inv_scale, 0, 4)
    _arg(fn, "ws", ws, 0)
    _check(fn, load().fp8_quant_tensor(
        _ptr(x), n, int(fmt), float(eps), _ptr(q), _ptr(scale), _ptr(inv_scale),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def _quant_rowlike(fn, x, q, scale, inv_scale, groups):
    b, r, c = _brc(x)
    _arg(fn, "x", x, 2 * b * r * c, 2)
    _arg(fn, "q", q, b * r * c, 1)
    _arg(fn, "scale", scale, 4 * groups(b, r, c), 4)
    if inv_scale is not None:
        _arg(fn, "inv_scale", inv_scale, 4 * groups(b, r, c), 4)
    return b, r, c


def fp8_quant_row(x, fmt, eps, q, scale, inv_scale=None, stream=None):
    b, r, c = _quant_rowlike("fp8_quant_row", x, q, scale, inv_scale, lambda b, r, c: b * r)
    _check("fp8_quant_row", load().fp8_quant_row(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(q), _ptr(scale), _ptr(inv_scale), _stream(stream)))


def fp8_quant_row_kpacked(x, fmt, eps, q, scale, inv_scale=None, stream=None):
    """fp8_quant_row with the codes in 1 KB chunks of 16 rows x 64 columns (q: any
    uint8 tensor of x.numel() bytes); the B layout of fp8_grouped_mm_kpacked."""
    b, r, c = _quant_rowlike("fp8_quant_row_kpacked", x, q, scale, inv_scale, lambda b, r, c: b * r)
    _check("fp8_quant_row_kpacked", load().fp8_quant_row_kpacked(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(q), _ptr(scale), _ptr(inv_scale), _stream(stream)))


def fp8_quant_row_kpaired(x, fmt, eps, q, scale, inv_scale=None, stream=None):
    """fp8_quant_row with the codes pair-interleaved (rows 2i and 2i + 1 share each
    128-byte line of a 64-column block); the A layout of fp8_grouped_mm_kpacked."""
    b, r, c = _quant_rowlike("fp8_quant_row_kpaired", x, q, scale, inv_scale, lambda b, r, c: b * r)
    _check("fp8_quant_row_kpaired", load().fp8_quant_row_kpaired(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(q), _ptr(scale), _ptr(inv_scale), _stream(stream)))


def fp8_quant_col_ws_bytes(batch: int, rows: int, cols: int) -> int:
    return load().fp8_quant_col_ws_bytes(int(batch), int(rows), int(cols))


def fp8_quant_col(x, fmt, eps, qT, scale, inv_scale=None, ws=None, stream=None):
    b, r, c = _quant_rowlike("fp8_quant_col", x, qT, scale, inv_scale, lambda b, r, c: b * c)
    _arg("fp8_quant_col", "ws", ws, 0)
    _check("fp8_quant_col", load().fp8_quant_col(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(qT), _ptr(scale), _ptr(inv_scale),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def fp8_quant_col_noalloc(x, fmt, eps, qT, scale, inv_scale=None, stream=None):
    """fp8_quant_col without a workspace argument: the library's own device buffer
    holds the column-amax words (for callers that cannot allocate)."""
    b, r, c = _quant_rowlike("fp8_quant_col_noalloc", x, qT, scale, inv_scale, lambda b, r, c: b * c)
    _check("fp8_quant_col_noalloc", load().fp8_quant_col_noalloc(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(qT), _ptr(scale), _ptr(inv_scale), _stream(stream)))


NORM_RMS, NORM_LAYER = 0, 1


def fp8_quant_col_kpacked(x, fmt, eps, qT, scale, inv_scale=None, ws=None, stream=None):
    """fp8_quant_col with qT k-packed as the [cols][rows] B operand (qT: any uint8
    tensor of x.numel() bytes)."""
    b, r, c = _quant_rowlike("fp8_quant_col_kpacked", x, qT, scale, inv_scale, lambda b, r, c: b * c)
    _arg("fp8_quant_col_kpacked", "ws", ws, 0)
    _check("fp8_quant_col_kpacked", load().fp8_quant_col_kpacked(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(qT), _ptr(scale), _ptr(inv_scale),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def fp8_norm_quant_row(x, gamma, beta, kind, norm_eps, fmt, eps, y, q, scale, inv_scale=None, stream=None):
    """x [rows][cols] bf16 -> y (bf16, or None), q/scale/inv (rowwise FP8 of y, or q None)."""
    fn = "fp8_norm_quant_row"
    rows, cols = x.shape
    _arg(fn, "x", x, 2 * rows * cols, 2)
    _arg(fn, "gamma", gamma, 2 * cols, 2)
    _arg(fn, "beta", beta, 0 if beta is None else 2 * cols, 2)
    _arg(fn, "y", y, 0 if y is None else 2 * rows * cols, 2)
    _arg(fn, "q", q, 0 if q is None else rows * cols, 1)
    _arg(fn, "scale", scale, 0 if scale is None else 4 * rows, 4)
    _arg(fn, "inv_scale", inv_scale, 0 if inv_scale is None else 4 * rows, 4)
    _check(fn, load().fp8_norm_quant_row(
        _ptr(x), _ptr(gamma), _ptr(beta), rows, cols, int(kind), float(norm_eps), int(fmt), float(eps),
        _ptr(y), _ptr(q), _ptr(scale), _ptr(inv_scale), _stream(stream)))


def fp8_quant_dual_ws_bytes() -> int:
    return load().fp8_quant_dual_ws_bytes()


def fp8_quant_dual(gy, x, g_fmt, x_fmt, eps, gq, gqT, g_scale, g_inv, xqT, x_scale, x_inv, ws, stream=None):
    """gy [M][N] and x [M][K] bf16 -> gq [M][N] (or None), gqT [N][M], xqT [K][M]."""
    fn = "fp8_quant_dual"
    M, N = gy.shape
    K = x.shape[1]
    if x.shape[0] != M:
        raise ValueError(f"{fn}: gy and x must have the same number of rows")
    _arg(fn, "gy", gy, 2 * M * N, 2)
    _arg(fn, "x", x, 2 * M * K, 2)
    _arg(fn, "gq", gq, 0 if gq is None else M * N, 1)
    _arg(fn, "gqT", gqT, M * N, 1)
    _arg(fn, "xqT", xqT, M * K, 1)
    for name, t in (("g_scale", g_scale), ("x_scale", x_scale)):
        _arg(fn, name, t, 4, 4)
    for name, t in (("g_inv", g_inv), ("x_inv", x_inv)):
        _arg(fn, name, t, 0, 4)
    _arg(fn, "ws", ws, 0)
    _check(fn, load().fp8_quant_dual(
        _ptr(gy), _ptr(x), M, N, K, int(g_fmt), int(x_fmt), float(eps), _ptr(gq), _ptr(gqT),
        _ptr(g_scale), _ptr(g_inv), _ptr(xqT), _ptr(x_scale), _ptr(x_inv),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def fp8_quant_block(x, block_rows, block_cols, fmt, eps, q, scale, inv_scale=None, stream=None):
    br, bc = int(block_rows), int(block_cols)
    groups = (lambda b, r, c: b * -(-r // br) * -(-c // bc)) if br > 0 and bc > 0 else (lambda b, r, c: 0)
    b, r, c = _quant_rowlike("fp8_quant_block", x, q, scale, inv_scale, groups)
    _check("fp8_quant_block", load().fp8_quant_block(
        _ptr(x), b, r, c, br, bc, int(fmt), float(eps), _ptr(q), _ptr(scale), _ptr(inv_scale), _stream(stream)))


def fp8_quant_mx(x, fmt, mode, eps, q, e8m0, stream=None):
    fn = "fp8_quant_mx"
    b, r, c = _brc(x)
    _arg(fn, "x", x, 2 * b * r * c, 2)
    _arg(fn, "q", q, b * r * c, 1)
    _arg(fn, "e8m0", e8m0, b * r * (c // 32), 1)
    _check(fn, load().fp8_quant_mx(
        _ptr(x), b, r, c, int(fmt), int(mode), float(eps), _ptr(q), _ptr(e8m0), _stream(stream)))


def _quant_mx_packed(fn, x, fmt, mode, eps, q, e8m0, stream):
    b, r, c = _brc(x)
    _arg(fn, "x", x, 2 * b * r * c, 2)
    _arg(fn, "q", q, b * r * c, 1)
    _arg(fn, "e8m0", e8m0, b * r * (c // 32), 1)
    _check(fn, getattr(load(), fn)(
        _ptr(x), b, r, c, int(fmt), int(mode), float(eps), _ptr(q), _ptr(e8m0), _stream(stream)))


def fp8_quant_mx_kpacked(x, fmt, mode, eps, q, e8m0, stream=None):
    """fp8_quant_mx with the codes k-packed (1 KB chunks of 16 rows x 64 columns per
    batch slice: fp8_grouped_mm_kpacked's B); q is any uint8 tensor of x.numel() bytes."""
    _quant_mx_packed("fp8_quant_mx_kpacked", x, fmt, mode, eps, q, e8m0, stream)


def fp8_quant_mx_kpaired(x, fmt, mode, eps, q, e8m0, stream=None):
    """fp8_quant_mx with the codes pair-interleaved (rows 2i, 2i + 1 sharing each
    128-byte line of a 64-column block: fp8_grouped_mm_kpacked's A)."""
    _quant_mx_packed("fp8_quant_mx_kpaired", x, fmt, mode, eps, q, e8m0, stream)


# ---- GEMMs ----------------------------------------------------------------------

def _gemm_args(fn, a, b, scaling, a_scale, b_scale, out, out_type, M, N, K, E=1):
    _arg(fn, "a", a, M * K, 1)
    _arg(fn, "b", b, E * N * K, 1)
    sa, sb = _gemm_scale_bytes(int(scaling), M, N, K, E)
    esz = 1 if int(scaling) == SCALE_MX32 else 4
    _arg(fn, "a_scale", a_scale, sa if K > 0 else 0, esz)
    _arg(fn, "b_scale", b_scale, sb if K > 0 else 0, esz)
    _arg(fn, "out", out, M * N * (4 if int(out_type) == OUT_F32 else 2), 4 if int(out_type) == OUT_F32 else 2)


def fp8_scaled_mm(a, fa, b, fb, scaling, a_inv, b_inv, out_type, out, use_fast_accum=True, stream=None):
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("fp8_scaled_mm: a and b must have the same K")
    _gemm_args("fp8_scaled_mm", a, b, scaling, a_inv, b_inv, out, out_type, M, N, K)
    _check("fp8_scaled_mm", load().fp8_scaled_mm(
        _ptr(a), int(fa), _ptr(b), int(fb), int(scaling), _ptr(a_inv), _ptr(b_inv), M, N, K,
        int(out_type), _ptr(out), int(bool(use_fast_accum)), _stream(stream)))


def fp8_grouped_mm(a, fa, b, fb, scaling, a_scale, b_scale, offsets, out_type, out, use_fast_accum=True,
                   stream=None):
    Mtot, K = a.shape
    E, N, Kb = b.shape
    if Kb != K:
        raise ValueError("fp8_grouped_mm: a and b must have the same K")
    _gemm_args("fp8_grouped_mm", a, b, scaling, a_scale, b_scale, out, out_type, Mtot, N, K, E)
    _offsets("fp8_grouped_mm", offsets, E)
    _check("fp8_grouped_mm", load().fp8_grouped_mm(
        _ptr(a), int(fa), _ptr(b), int(fb), int(scaling), _ptr(a_scale), _ptr(b_scale),
        _ptr(offsets), E, Mtot, N, K, int(out_type), _ptr(out), int(bool(use_fast_accum)), _stream(stream)))


def fp8_scaled_mm_kpacked(a, fa, b, fb, scaling, a_inv, b_inv, out_type, out, N, use_fast_accum=True, stream=None):
    """fp8_scaled_mm with b k-packed ([N][K] codes in 1 KB chunks of 16 rows x 64 K);
    b is any uint8 tensor of N * K bytes."""
    M, K = a.shape
    if b.numel() * b.element_size() != N * K:
        raise ValueError("fp8_scaled_mm_kpacked: b must hold N * K bytes")
    _gemm_args("fp8_scaled_mm_kpacked", a, b, scaling, a_inv, b_inv, out, out_type, M, N, K)
    _check("fp8_scaled_mm_kpacked", load().fp8_scaled_mm_kpacked(
        _ptr(a), int(fa), _ptr(b), int(fb), int(scaling), _ptr(a_inv), _ptr(b_inv), M, N, K,
        int(out_type), _ptr(out), int(bool(use_fast_accum)), _stream(stream)))


def fp8_grouped_mm_kpacked(a, fa, b, fb, scaling, a_scale, b_scale, offsets, out_type, out, N, use_fast_accum=True,
                           stream=None):
    """fp8_grouped_mm with a pair-interleaved (fp8_quant_row_kpaired's layout; a is
    [Mtot][K] shaped) and b k-packed (fp8_quant_row_kpacked's layout of the [E][N][K]
    codes); b is any uint8 tensor of E * N * K bytes with b.shape[0] == E."""
    Mtot, K = a.shape
    E = b.shape[0]
    if b.numel() * b.element_size() != E * N * K:
        raise ValueError("fp8_grouped_mm_kpacked: b must hold E * N * K bytes")
    _gemm_args("fp8_grouped_mm_kpacked", a, b, scaling, a_scale, b_scale, out, out_type, Mtot, N, K, E)
    _offsets("fp8_grouped_mm_kpacked", offsets, E)
    _check("fp8_grouped_mm_kpacked", load().fp8_grouped_mm_kpacked(
        _ptr(a), int(fa), _ptr(b), int(fb), int(scaling), _ptr(a_scale), _ptr(b_scale),
        _ptr(offsets), E, Mtot, N, K, int(out_type), _ptr(out), int(bool(use_fast_accum)), _stream(stream)))


def fp8_wgrad_bf16(gy, x, gw, stream=None):
    fn = "fp8_wgrad_bf16"
    M, N = gy.shape
    K = x.shape[1]
    if x.shape[0] != M:
        raise ValueError(f"{fn}: gy and x must have the same number of rows")
    _arg(fn, "gy", gy, 2 * M * N, 2)
    _arg(fn, "x", x, 2 * M * K, 2)
    _arg(fn, "gw", gw, 2 * N * K, 2)
    _check(fn, load().fp8_wgrad_bf16(_ptr(gy), _ptr(x), M, N, K, _ptr(gw), _stream(stream)))


def fp8_grouped_wgrad_bf16(gy, x, offsets, gw, stream=None):
    """gy [Mtot][N], x [Mtot][K] bf16, offsets device int32 [E+1] -> gw [E][N][K] bf16."""
    fn = "fp8_grouped_wgrad_bf16"
    Mtot, N = gy.shape
    K = x.shape[1]
    E = offsets.numel() - 1
    if x.shape[0] != Mtot:
        raise ValueError(f"{fn}: gy and x must have the same number of rows")
    _arg(fn, "gy", gy, 2 * Mtot * N, 2)
    _arg(fn, "x", x, 2 * Mtot * K, 2)
    _offsets(fn, offsets, E)
    _arg(fn, "gw", gw, 2 * E * N * K, 2)
    _check(fn, load().fp8_grouped_wgrad_bf16(
        _ptr(gy), _ptr(x), _ptr(offsets), E, Mtot, N, K, _ptr(gw), _stream(stream)))


# ---- Linear layer -----------------------------------------------------------------

def fp8_linear_ws_bytes(M, N, K, recipe) -> int:
    return load().fp8_linear_ws_bytes(int(M), int(N), int(K), int(recipe))


def fp8_linear_fwd(x, w, recipe, eps, out_type, y, ws, use_fast_accum=True, stream=None):
    fn = "fp8_linear_fwd"
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"{fn}: x and w must have the same K")
    _arg(fn, "x", x, 2 * M * K, 2)
    _arg(fn, "w", w, 2 * N * K, 2)
    osz = 4 if int(out_type) == OUT_F32 else 2
    _arg(fn, "y", y, osz * M * N, osz)
    _arg(fn, "ws", ws, 0)
    _check(fn, load().fp8_linear_fwd(
        _ptr(x), _ptr(w), M, N, K, int(recipe), float(eps), int(out_type), int(bool(use_fast_accum)), _ptr(y),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def fp8_linear_bwd(gy, x, w, recipe, eps, gx, gw, ws, stream=None):
    fn = "fp8_linear_bwd"
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or gy.shape[0] != M or gy.shape[1] != N:
        raise ValueError(f"{fn}: gy [M][N], x [M][K], w [N][K] shapes disagree")
    _arg(fn, "gy", gy, 2 * M * N, 2)
    _arg(fn, "x", x, 2 * M * K, 2)
    _arg(fn, "w", w, 2 * N * K, 2)
    _arg(fn, "gx", gx, 2 * M * K, 2)
    _arg(fn, "gw", gw, 2 * N * K, 2)
    _arg(fn, "ws", ws, 0)
    _check(fn, load().fp8_linear_bwd(
        _ptr(gy), _ptr(x), _ptr(w), M, N, K, int(recipe), float(eps), _ptr(gx), _ptr(gw), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def fp8_validate_offsets(host_offsets, Mtot: int) -> int:
    """host_offsets: a CPU int32 tensor or numpy array of E+1 entries. Returns the status."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(host_offsets, dtype=np.int32))
    return load().fp8_validate_offsets(arr.ctypes.data, len(arr) - 1, int(Mtot))
