"""Host-side behaviour of Float8Linear (no GPU): argument checks fail loudly; there is
no CPU fallback."""
import pytest
import torch

from fp8_dynamic_scaling_amd.nn import Float8Linear


def test_rejects_unknown_recipe():
    with pytest.raises(ValueError):
        Float8Linear(64, 64, recipe="blockwise")


def test_parameters_are_bf16_linear_shaped():
    m = Float8Linear(64, 32, bias=True)
    assert m.weight.shape == (32, 64) and m.weight.dtype == torch.bfloat16
    assert m.bias.shape == (32,)
    assert "recipe=rowwise" in repr(m)


def test_cpu_input_is_refused():
    m = Float8Linear(64, 32)
    with pytest.raises(RuntimeError, match="ROCm GPU"):
        m(torch.zeros(16, 64, dtype=torch.bfloat16))
