"""The Python binding's marshalling checks (no GPU): operands that the C ABI would read
or write out of bounds, or reinterpret, are refused before any call reaches the
library. The library takes raw pointers, so these checks are the only guard against
an int64 offsets tensor (torch.cumsum's default) read as pairs of int32 words, a
host tensor, a non-contiguous view or an undersized output."""
import pytest
import torch

import fp8_dynamic_scaling_amd as f


def test_offsets_must_be_int32_with_e_plus_one_entries():
    with pytest.raises(ValueError, match="int32"):
        f._offsets("fp8_grouped_mm", torch.zeros(5, dtype=torch.int64), 4)
    with pytest.raises(ValueError, match="E \\+ 1"):
        f._offsets("fp8_grouped_mm", torch.zeros(4, dtype=torch.int32), 4)
    with pytest.raises(ValueError, match="required"):
        f._offsets("fp8_grouped_mm", None, 4)


def test_host_tensors_are_refused():
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    q = torch.zeros(4, 64, dtype=torch.uint8)
    s = torch.zeros(4, dtype=torch.float32)
    with pytest.raises(ValueError, match="on the GPU"):
        f.fp8_quant_row(x, f.E4M3_NATIVE, 1e-12, q, s)
    a = torch.zeros(16, 128, dtype=torch.uint8)
    with pytest.raises(ValueError, match="on the GPU"):
        f.fp8_scaled_mm(a, f.E4M3_NATIVE, a, f.E4M3_NATIVE, f.SCALE_ROW, s, s, f.OUT_BF16,
                        torch.zeros(16, 16, dtype=torch.bfloat16))


def test_required_bytes_per_operand():
    # (scaling, M, N, K, E) -> bytes of the A and B scales
    assert f._gemm_scale_bytes(f.SCALE_TENSOR, 8, 16, 128) == (4, 4)
    assert f._gemm_scale_bytes(f.SCALE_ROW, 8, 16, 128, 3) == (32, 4 * 3 * 16)
    assert f._gemm_scale_bytes(f.SCALE_BLOCK128, 8, 256, 512, 2) == (4 * 8 * 4, 4 * 2 * 2 * 4)
    assert f._gemm_scale_bytes(f.SCALE_MX32, 8, 16, 128, 2) == (8 * 4, 2 * 16 * 4)


class _FakeCuda:
    """Stands in for a GPU tensor in the size checks (they read only these fields)."""

    def __init__(self, n, esize, contiguous=True):
        self.is_cuda = True
        self._n, self._e, self._c = n, esize, contiguous
        self.dtype = f"a {esize}-byte dtype"

    def is_contiguous(self):
        return self._c

    def element_size(self):
        return self._e

    def numel(self):
        return self._n


def test_undersized_and_strided_operands_are_refused():
    with pytest.raises(ValueError, match="needs 64"):
        f._arg("fp8_quant_row", "q", _FakeCuda(63, 1), 64, 1)
    with pytest.raises(ValueError, match="contiguous"):
        f._arg("fp8_quant_row", "q", _FakeCuda(64, 1, contiguous=False), 64, 1)
    with pytest.raises(ValueError, match="2-byte"):
        f._arg("fp8_quant_row", "x", _FakeCuda(64, 4), 128, 2)
    f._arg("fp8_quant_row", "q", _FakeCuda(64, 1), 64, 1)
    f._arg("fp8_quant_row", "inv_scale", None, 0, 4)
    with pytest.raises(ValueError, match="required"):
        f._arg("fp8_quant_row", "scale", None, 16, 4)
