"""The C-ABI library loads and exports every symbol include/fp8dyn.h declares;
host-side validation rejects bad arguments before any GPU work (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8dyn.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"FP8DYN_API\s+[\w\s\*]+?\b(fp8_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def f():
    import fp8_dynamic_scaling_amd as f
    if not os.path.exists(f.LIB_PATH):
        from fp8_dynamic_scaling_amd import build
        build.build()
    f.load()
    return f


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["fp8_quant_tensor", "fp8_quant_row", "fp8_quant_col", "fp8_quant_block", "fp8_quant_mx",
                 "fp8_scaled_mm", "fp8_grouped_mm", "fp8_linear_fwd", "fp8_linear_bwd", "fp8_probe"]:
        assert want in names


def test_exports_every_declared_symbol(f):
    lib = ctypes.CDLL(f.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(f.EXPORTS) == declared_functions()


def test_only_the_abi_is_exported(f):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", f.LIB_PATH], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    ours = {s for s in syms if s.startswith("fp8_")}
    assert ours == set(declared_functions())


def test_status_strings(f):
    for s in range(6):
        assert f.fp8_status_string(s)


def test_host_validation_without_gpu(f):
    lib = f.load()
    FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first
    # negative sizes
    assert lib.fp8_quant_row(FAKE, 1, -1, 8, f.E4M3_NATIVE, 1e-12, FAKE, FAKE, None, None) == f.ERR_INVALID_ARGUMENT
    # eps must be finite and positive
    for eps in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.fp8_quant_row(FAKE, 1, 4, 8, f.E4M3_NATIVE, eps, FAKE, FAKE, None, None) == f.ERR_INVALID_ARGUMENT
    # null pointers with non-zero sizes
    assert lib.fp8_quant_row(None, 1, 4, 8, f.E4M3_NATIVE, 1e-12, FAKE, FAKE, None, None) == f.ERR_INVALID_ARGUMENT
    # misaligned data pointer
    assert lib.fp8_quant_row(FAKE + 2, 1, 4, 8, f.E4M3_NATIVE, 1e-12, FAKE, FAKE, None, None) == f.ERR_ALIGNMENT
    # zero-size problems without groups are a no-op success
    assert lib.fp8_quant_row(None, 0, 4, 8, f.E4M3_NATIVE, 1e-12, None, None, None, None) == f.OK
    assert lib.fp8_quant_col(None, 0, 0, 8, f.E4M3_NATIVE, 1e-12, None, None, None, None, 0, None) == f.OK
    # ... but empty groups still get their (eps-clamped) scales, so those must be given
    assert lib.fp8_quant_col(None, 1, 0, 8, f.E4M3_NATIVE, 1e-12, None, None, None, None, 0, None) == f.ERR_INVALID_ARGUMENT
    assert lib.fp8_quant_row(None, 1, 4, 0, f.E4M3_NATIVE, 1e-12, None, None, None, None) == f.ERR_INVALID_ARGUMENT
    assert lib.fp8_quant_tensor(None, 0, f.E4M3_NATIVE, 1e-12, None, None, None, None, 0, None) == f.ERR_INVALID_ARGUMENT
    # MX needs cols % 32 == 0, and eps >= 2^-100 (the E8M0 range)
    assert lib.fp8_quant_mx(FAKE, 1, 4, 48, f.E4M3_NATIVE, f.MX_POW2_FLOOR, 1e-12, FAKE, FAKE, None) == f.ERR_ALIGNMENT
    for mode in (f.MX_POW2_FLOOR, f.MX_OCP):
        assert lib.fp8_quant_mx(FAKE, 1, 4, 64, f.E4M3_NATIVE, mode, 2.0 ** -101, FAKE, FAKE, None) == \
            f.ERR_INVALID_ARGUMENT
    # packed MX: cols % 64, rows % 16 (k-packed) or % 2 (pair-interleaved), 16-byte
    # aligned x and q, and the same eps bound
    kp, kq = lib.fp8_quant_mx_kpacked, lib.fp8_quant_mx_kpaired
    assert kp(FAKE, 1, 16, 96, f.E4M3_NATIVE, f.MX_POW2_FLOOR, 1e-12, FAKE, FAKE, None) == f.ERR_ALIGNMENT
    assert kp(FAKE, 1, 8, 64, f.E4M3_NATIVE, f.MX_POW2_FLOOR, 1e-12, FAKE, FAKE, None) == f.ERR_ALIGNMENT
    assert kq(FAKE, 1, 3, 64, f.E4M3_NATIVE, f.MX_POW2_FLOOR, 1e-12, FAKE, FAKE, None) == f.ERR_ALIGNMENT
    assert kq(FAKE + 8, 1, 2, 64, f.E4M3_NATIVE, f.MX_POW2_FLOOR, 1e-12, FAKE, FAKE, None) == f.ERR_ALIGNMENT
    assert kp(FAKE, 1, 16, 64, f.E4M3_NATIVE, f.MX_OCP, 2.0 ** -101, FAKE, FAKE, None) == f.ERR_INVALID_ARGUMENT
    assert kq(FAKE, 1, 2, 64, f.E4M3_NATIVE, 7, 1e-12, FAKE, FAKE, None) == f.ERR_INVALID_ARGUMENT
    assert kp(FAKE, 0, 16, 64, f.E4M3_NATIVE, f.MX_POW2_FLOOR, 1e-12, FAKE, FAKE, None) == f.OK
    # block geometry
    assert lib.fp8_quant_block(FAKE, 1, 4, 8, 2, 128, f.E4M3_NATIVE, 1e-12, FAKE, FAKE, None, None) == f.ERR_INVALID_ARGUMENT
    # tensorwise needs a workspace
    assert lib.fp8_quant_tensor(FAKE, 64, f.E4M3_NATIVE, 1e-12, FAKE, FAKE, None, None, 0, None) == f.ERR_WORKSPACE
    # GEMM: K % 16, block K % 128, MX K % 32, bad enum
    args = (FAKE, f.E4M3_NATIVE, FAKE, f.E4M3_NATIVE)
    assert lib.fp8_scaled_mm(*args, f.SCALE_ROW, FAKE, FAKE, 16, 16, 40, f.OUT_BF16, FAKE, 1, None) == f.ERR_ALIGNMENT
    assert lib.fp8_scaled_mm(*args, 7, FAKE, FAKE, 16, 16, 64, f.OUT_BF16, FAKE, 1, None) == f.ERR_UNSUPPORTED
    assert lib.fp8_scaled_mm(*args, f.SCALE_ROW, FAKE, FAKE, 16, 16, 64, 9, FAKE, 1, None) == f.ERR_INVALID_ARGUMENT
    assert lib.fp8_grouped_mm(*args, f.SCALE_BLOCK128, FAKE, FAKE, FAKE, 2, 16, 128, 64, f.OUT_BF16, FAKE, 1, None) == f.ERR_ALIGNMENT
    assert lib.fp8_grouped_mm(*args, f.SCALE_MX32, FAKE, FAKE, FAKE, 2, 16, 128, 48, f.OUT_BF16, FAKE, 1, None) == f.ERR_ALIGNMENT
    assert lib.fp8_grouped_mm(*args, f.SCALE_ROW, FAKE, FAKE, FAKE, 0, 16, 128, 64, f.OUT_BF16, FAKE, 1, None) == f.ERR_INVALID_ARGUMENT
    assert lib.fp8_grouped_mm(*args, f.SCALE_ROW, FAKE, FAKE, None, 2, 16, 128, 64, f.OUT_BF16, FAKE, 1, None) == f.ERR_INVALID_ARGUMENT
    # k-packed rowwise codes: rows % 16, cols % 64, at most 16384 columns
    kp = (f.E4M3_NATIVE, 1e-12, FAKE, FAKE, None, None)
    assert lib.fp8_quant_row_kpacked(FAKE, 1, 8, 64, *kp) == f.ERR_ALIGNMENT
    assert lib.fp8_quant_row_kpacked(FAKE, 1, 16, 32, *kp) == f.ERR_ALIGNMENT
    assert lib.fp8_quant_row_kpacked(FAKE, 1, 16, 16448, *kp) == f.ERR_UNSUPPORTED
    # k-packed grouped GEMM: ROW or MX32 only, N % 16, K % 128, N * K < 2^31
    assert lib.fp8_grouped_mm_kpacked(*args, f.SCALE_BLOCK128, FAKE, FAKE, FAKE, 2, 16, 128, 128, f.OUT_BF16, FAKE,
                                      1, None) == f.ERR_UNSUPPORTED
    assert lib.fp8_grouped_mm_kpacked(*args, f.SCALE_ROW, FAKE, FAKE, FAKE, 2, 16, 40, 128, f.OUT_BF16, FAKE,
                                      1, None) == f.ERR_ALIGNMENT
    assert lib.fp8_grouped_mm_kpacked(*args, f.SCALE_ROW, FAKE, FAKE, FAKE, 2, 16, 64, 64, f.OUT_BF16, FAKE,
                                      1, None) == f.ERR_ALIGNMENT
    assert lib.fp8_grouped_mm_kpacked(*args, f.SCALE_ROW, FAKE, FAKE, FAKE, 2, 16, 65536, 32768, f.OUT_BF16, FAKE,
                                      1, None) == f.ERR_UNSUPPORTED
    assert lib.fp8_grouped_mm_kpacked(*args, f.SCALE_ROW, FAKE, FAKE, FAKE, 2, 17, 64, 128, f.OUT_BF16, FAKE,
                                      1, None) == f.ERR_ALIGNMENT
    # pair-interleaved rowwise codes: rows % 2, cols % 64
    assert lib.fp8_quant_row_kpaired(FAKE, 1, 3, 64, *kp) == f.ERR_ALIGNMENT
    assert lib.fp8_quant_row_kpaired(FAKE, 1, 2, 96, *kp) == f.ERR_ALIGNMENT
    # k-packed transposed column codes: rows % 64, cols % 16, a workspace for the split form
    assert lib.fp8_quant_col_kpacked(FAKE, 1, 32, 16, f.E4M3_NATIVE, 1e-12, FAKE, FAKE, None, None, 0,
                                     None) == f.ERR_ALIGNMENT
    assert lib.fp8_quant_col_kpacked(FAKE, 1, 64, 8, f.E4M3_NATIVE, 1e-12, FAKE, FAKE, None, None, 0,
                                     None) == f.ERR_ALIGNMENT
    assert lib.fp8_quant_col_kpacked(FAKE, 1, 14336, 4096, f.E4M3_NATIVE, 1e-12, FAKE, FAKE, None, None, 0,
                                     None) == f.ERR_WORKSPACE
    # k-packed dense GEMM: TENSOR or ROW, N % 16, K % 128
    assert lib.fp8_scaled_mm_kpacked(*args, f.SCALE_BLOCK128, FAKE, FAKE, 16, 16, 128, f.OUT_BF16, FAKE,
                                     1, None) == f.ERR_UNSUPPORTED
    assert lib.fp8_scaled_mm_kpacked(*args, f.SCALE_ROW, FAKE, FAKE, 16, 24, 128, f.OUT_BF16, FAKE,
                                     1, None) == f.ERR_ALIGNMENT
    assert lib.fp8_scaled_mm_kpacked(*args, f.SCALE_ROW, FAKE, FAKE, 16, 16, 64, f.OUT_BF16, FAKE,
                                     1, None) == f.ERR_ALIGNMENT
    # linear: workspace too small
    need = lib.fp8_linear_ws_bytes(64, 64, 64, f.RECIPE_ROWWISE_BF16_WGRAD)
    assert need > 64 * 64 * 2
    assert lib.fp8_linear_fwd(FAKE, FAKE, 64, 64, 64, f.RECIPE_ROWWISE_BF16_WGRAD, 1e-12, f.OUT_BF16, 1, FAKE, FAKE,
                              need - 1, None) == f.ERR_WORKSPACE
    assert lib.fp8_wgrad_bf16(FAKE, FAKE, 16, 12, 16, FAKE, None) == f.ERR_ALIGNMENT
    assert lib.fp8_wgrad_bf16(FAKE, FAKE, 16, 16, 12, FAKE, None) == f.ERR_ALIGNMENT
    assert lib.fp8_wgrad_bf16(FAKE + 8, FAKE, 16, 16, 16, FAKE, None) == f.ERR_ALIGNMENT
    # B must be an e4m3 variant: every e5m2 request is refused before any device work
    for fb in (f.E5M2, f.E5M2FNUZ, f.E5M2_NATIVE):
        ab = (FAKE, f.E4M3_NATIVE, FAKE, fb)
        assert lib.fp8_scaled_mm(*ab, f.SCALE_ROW, FAKE, FAKE, 16, 16, 64, f.OUT_BF16, FAKE, 1, None) == \
            f.ERR_UNSUPPORTED
        assert lib.fp8_grouped_mm(*ab, f.SCALE_ROW, FAKE, FAKE, FAKE, 2, 16, 16, 128, f.OUT_BF16, FAKE, 0, None) == \
            f.ERR_UNSUPPORTED
        assert lib.fp8_scaled_mm_kpacked(*ab, f.SCALE_ROW, FAKE, FAKE, 16, 16, 128, f.OUT_BF16, FAKE, 1, None) == \
            f.ERR_UNSUPPORTED
        assert lib.fp8_grouped_mm_kpacked(*ab, f.SCALE_ROW, FAKE, FAKE, FAKE, 2, 16, 16, 128, f.OUT_BF16, FAKE, 1,
                                          None) == f.ERR_UNSUPPORTED
    # full-precision accumulation on the packed grouped GEMM: ROW scaling only
    assert lib.fp8_grouped_mm_kpacked(*args, f.SCALE_MX32, FAKE, FAKE, FAKE, 2, 16, 16, 128, f.OUT_BF16, FAKE, 0,
                                      None) == f.ERR_UNSUPPORTED


def test_workspace_sizes(f):
    assert f.fp8_quant_tensor_ws_bytes() >= 4
    assert f.fp8_quant_col_ws_bytes(32, 2048, 7168) == 0       # single pass
    assert f.fp8_quant_col_ws_bytes(1, 14336, 4096) == 4096 * 4  # split form: one word per column


def test_validate_offsets(f):
    assert f.fp8_validate_offsets(np.array([0, 3, 3, 10], np.int32), 10) == f.OK
    assert f.fp8_validate_offsets(np.array([0, 3, 2, 10], np.int32), 10) == f.ERR_INVALID_ARGUMENT
    assert f.fp8_validate_offsets(np.array([1, 3, 3, 10], np.int32), 10) == f.ERR_INVALID_ARGUMENT
    assert f.fp8_validate_offsets(np.array([0, 3, 3, 9], np.int32), 10) == f.ERR_INVALID_ARGUMENT


def test_product_path_does_not_touch_the_oracle():
    # the package and its C sources never reference the oracle
    pkg = os.path.join(ROOT, "fp8_dynamic_scaling_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower().replace("oracle_", ""), fn
