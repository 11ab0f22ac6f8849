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
    "fp8_quant_block", "fp8_quant_mx",
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
        "fp8_scaled_mm": (I, [P, I, P, I, I, P, P, I64, I64, I64, I, P, I, P]),
        "fp8_scaled_mm_kpacked": (I, [P, I, P, I, I, P, P, I64, I64, I64, I, P, P]),
        "fp8_grouped_mm": (I, [P, I, P, I, I, P, P, P, I32, I64, I64, I64, I, P, P]),
        "fp8_grouped_mm_kpacked": (I, [P, I, P, I, I, P, P, P, I32, I64, I64, I64, I, P, P]),
        "fp8_wgrad_bf16": (I, [P, P, I64, I64, I64, P, P]),
        "fp8_grouped_wgrad_bf16": (I, [P, P, P, I32, I64, I64, I64, P, P]),
        "fp8_linear_fwd": (I, [P, P, I64, I64, I64, I, D, I, P, P, SZ, P]),
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
    _check("fp8_quant_tensor", load().fp8_quant_tensor(
        _ptr(x), x.numel(), int(fmt), float(eps), _ptr(q), _ptr(scale), _ptr(inv_scale),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def fp8_quant_row(x, fmt, eps, q, scale, inv_scale=None, stream=None):
    b, r, c = _brc(x)
    _check("fp8_quant_row", load().fp8_quant_row(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(q), _ptr(scale), _ptr(inv_scale), _stream(stream)))


def fp8_quant_row_kpacked(x, fmt, eps, q, scale, inv_scale=None, stream=None):
    """fp8_quant_row with the codes in 1 KB chunks of 16 rows x 64 columns (q: any
    uint8 tensor of x.numel() bytes); the B layout of fp8_grouped_mm_kpacked."""
    b, r, c = _brc(x)
    if q.numel() * q.element_size() != b * r * c:
        raise ValueError("fp8_quant_row_kpacked: q must hold one byte per element of x")
    _check("fp8_quant_row_kpacked", load().fp8_quant_row_kpacked(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(q), _ptr(scale), _ptr(inv_scale), _stream(stream)))


def fp8_quant_row_kpaired(x, fmt, eps, q, scale, inv_scale=None, stream=None):
    """fp8_quant_row with the codes pair-interleaved (rows 2i and 2i + 1 share each
    128-byte line of a 64-column block); the A layout of fp8_grouped_mm_kpacked."""
    b, r, c = _brc(x)
    if q.numel() * q.element_size() != b * r * c:
        raise ValueError("fp8_quant_row_kpaired: q must hold one byte per element of x")
    _check("fp8_quant_row_kpaired", load().fp8_quant_row_kpaired(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(q), _ptr(scale), _ptr(inv_scale), _stream(stream)))


def fp8_quant_col_ws_bytes(batch: int, rows: int, cols: int) -> int:
    return load().fp8_quant_col_ws_bytes(int(batch), int(rows), int(cols))


def fp8_quant_col(x, fmt, eps, qT, scale, inv_scale=None, ws=None, stream=None):
    b, r, c = _brc(x)
    _check("fp8_quant_col", load().fp8_quant_col(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(qT), _ptr(scale), _ptr(inv_scale),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def fp8_quant_col_noalloc(x, fmt, eps, qT, scale, inv_scale=None, stream=None):
    """fp8_quant_col without a workspace argument: the library's own device buffer
    holds the column-amax words (for callers that cannot allocate)."""
    b, r, c = _brc(x)
    _check("fp8_quant_col_noalloc", load().fp8_quant_col_noalloc(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(qT), _ptr(scale), _ptr(inv_scale), _stream(stream)))


NORM_RMS, NORM_LAYER = 0, 1


def fp8_quant_col_kpacked(x, fmt, eps, qT, scale, inv_scale=None, ws=None, stream=None):
    """fp8_quant_col with qT k-packed as the [cols][rows] B operand (qT: any uint8
    tensor of x.numel() bytes)."""
    b, r, c = _brc(x)
    if qT.numel() * qT.element_size() != b * r * c:
        raise ValueError("fp8_quant_col_kpacked: qT must hold one byte per element of x")
    _check("fp8_quant_col_kpacked", load().fp8_quant_col_kpacked(
        _ptr(x), b, r, c, int(fmt), float(eps), _ptr(qT), _ptr(scale), _ptr(inv_scale),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def fp8_norm_quant_row(x, gamma, beta, kind, norm_eps, fmt, eps, y, q, scale, inv_scale=None, stream=None):
    """x [rows][cols] bf16 -> y (bf16, or None), q/scale/inv (rowwise FP8 of y, or q None)."""
    rows, cols = x.shape
    _check("fp8_norm_quant_row", load().fp8_norm_quant_row(
        _ptr(x), _ptr(gamma), _ptr(beta), rows, cols, int(kind), float(norm_eps), int(fmt), float(eps),
        _ptr(y), _ptr(q), _ptr(scale), _ptr(inv_scale), _stream(stream)))


def fp8_quant_dual_ws_bytes() -> int:
    return load().fp8_quant_dual_ws_bytes()


def fp8_quant_dual(gy, x, g_fmt, x_fmt, eps, gq, gqT, g_scale, g_inv, xqT, x_scale, x_inv, ws, stream=None):
    """gy [M][N] and x [M][K] bf16 -> gq [M][N] (or None), gqT [N][M], xqT [K][M]."""
    M, N = gy.shape
    K = x.shape[1]
    _check("fp8_quant_dual", load().fp8_quant_dual(
        _ptr(gy), _ptr(x), M, N, K, int(g_fmt), int(x_fmt), float(eps), _ptr(gq), _ptr(gqT),
        _ptr(g_scale), _ptr(g_inv), _ptr(xqT), _ptr(x_scale), _ptr(x_inv),
        _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def fp8_quant_block(x, block_rows, block_cols, fmt, eps, q, scale, inv_scale=None, stream=None):
    b, r, c = _brc(x)
    _check("fp8_quant_block", load().fp8_quant_block(
        _ptr(x), b, r, c, int(block_rows), int(block_cols), int(fmt), float(eps), _ptr(q),
        _ptr(scale), _ptr(inv_scale), _stream(stream)))


def fp8_quant_mx(x, fmt, mode, eps, q, e8m0, stream=None):
    b, r, c = _brc(x)
    _check("fp8_quant_mx", load().fp8_quant_mx(
        _ptr(x), b, r, c, int(fmt), int(mode), float(eps), _ptr(q), _ptr(e8m0), _stream(stream)))


# ---- GEMMs ----------------------------------------------------------------------

def fp8_scaled_mm(a, fa, b, fb, scaling, a_inv, b_inv, out_type, out, use_fast_accum=True, stream=None):
    M, K = a.shape
    N = b.shape[0]
    _check("fp8_scaled_mm", load().fp8_scaled_mm(
        _ptr(a), int(fa), _ptr(b), int(fb), int(scaling), _ptr(a_inv), _ptr(b_inv), M, N, K,
        int(out_type), _ptr(out), int(bool(use_fast_accum)), _stream(stream)))


def fp8_grouped_mm(a, fa, b, fb, scaling, a_scale, b_scale, offsets, out_type, out, stream=None):
    Mtot, K = a.shape
    E, N, _ = b.shape
    _check("fp8_grouped_mm", load().fp8_grouped_mm(
        _ptr(a), int(fa), _ptr(b), int(fb), int(scaling), _ptr(a_scale), _ptr(b_scale),
        _ptr(offsets), E, Mtot, N, K, int(out_type), _ptr(out), _stream(stream)))


def fp8_scaled_mm_kpacked(a, fa, b, fb, scaling, a_inv, b_inv, out_type, out, N, stream=None):
    """fp8_scaled_mm with b k-packed ([N][K] codes in 1 KB chunks of 16 rows x 64 K);
    b is any uint8 tensor of N * K bytes."""
    M, K = a.shape
    if b.numel() * b.element_size() != N * K:
        raise ValueError("fp8_scaled_mm_kpacked: b must hold N * K bytes")
    _check("fp8_scaled_mm_kpacked", load().fp8_scaled_mm_kpacked(
        _ptr(a), int(fa), _ptr(b), int(fb), int(scaling), _ptr(a_inv), _ptr(b_inv), M, N, K,
        int(out_type), _ptr(out), _stream(stream)))


def fp8_grouped_mm_kpacked(a, fa, b, fb, scaling, a_scale, b_scale, offsets, out_type, out, N, stream=None):
    """fp8_grouped_mm with a pair-interleaved (fp8_quant_row_kpaired's layout; a is
    [Mtot][K] shaped) and b k-packed (fp8_quant_row_kpacked's layout of the [E][N][K]
    codes); b is any uint8 tensor of E * N * K bytes with b.shape[0] == E."""
    Mtot, K = a.shape
    E = b.shape[0]
    if b.numel() * b.element_size() != E * N * K:
        raise ValueError("fp8_grouped_mm_kpacked: b must hold E * N * K bytes")
    _check("fp8_grouped_mm_kpacked", load().fp8_grouped_mm_kpacked(
        _ptr(a), int(fa), _ptr(b), int(fb), int(scaling), _ptr(a_scale), _ptr(b_scale),
        _ptr(offsets), E, Mtot, N, K, int(out_type), _ptr(out), _stream(stream)))


def fp8_wgrad_bf16(gy, x, gw, stream=None):
    M, N = gy.shape
    K = x.shape[1]
    _check("fp8_wgrad_bf16", load().fp8_wgrad_bf16(_ptr(gy), _ptr(x), M, N, K, _ptr(gw), _stream(stream)))


# ---- Linear layer -----------------------------------------------------------------

def fp8_grouped_wgrad_bf16(gy, x, offsets, gw, stream=None):
    """gy [Mtot][N], x [Mtot][K] bf16, offsets device int32 [E+1] -> gw [E][N][K] bf16."""
    Mtot, N = gy.shape
    K = x.shape[1]
    E = offsets.numel() - 1
    _check("fp8_grouped_wgrad_bf16", load().fp8_grouped_wgrad_bf16(
        _ptr(gy), _ptr(x), _ptr(offsets), E, Mtot, N, K, _ptr(gw), _stream(stream)))


def fp8_linear_ws_bytes(M, N, K, recipe) -> int:
    return load().fp8_linear_ws_bytes(int(M), int(N), int(K), int(recipe))


def fp8_linear_fwd(x, w, recipe, eps, out_type, y, ws, stream=None):
    M, K = x.shape
    N = w.shape[0]
    _check("fp8_linear_fwd", load().fp8_linear_fwd(
        _ptr(x), _ptr(w), M, N, K, int(recipe), float(eps), int(out_type), _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def fp8_linear_bwd(gy, x, w, recipe, eps, gx, gw, ws, stream=None):
    M, K = x.shape
    N = w.shape[0]
    _check("fp8_linear_bwd", load().fp8_linear_bwd(
        _ptr(gy), _ptr(x), _ptr(w), M, N, K, int(recipe), float(eps), _ptr(gx), _ptr(gw), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def fp8_validate_offsets(host_offsets, Mtot: int) -> int:
    """host_offsets: a CPU int32 tensor or numpy array of E+1 entries. Returns the status."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(host_offsets, dtype=np.int32))
    return load().fp8_validate_offsets(arr.ctypes.data, len(arr) - 1, int(Mtot))
