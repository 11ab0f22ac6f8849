"""fp8_quant_col_noalloc: the column quantization without a workspace argument, for
callers that cannot allocate. Called through the C ABI, it must give exactly the bytes
and scales of fp8_quant_col with a caller-allocated workspace, on two calls in a row
(the second smaller, so stale scratch contents from the first would show), and reject
problems whose column-amax words exceed its scratch before launching anything."""
import ctypes

import numpy as np
import pytest

import synth
from tests.gpu_util import gpu, have_gpu, lib

EPS = 1e-12


def test_noalloc_rejects_sizes_beyond_the_scratch_on_the_host():
    """16400 columns in the split form need 65600 bytes of amax words: more than the
    64 KiB scratch; the call returns FP8_ERR_UNSUPPORTED before any device work."""
    import fp8_dynamic_scaling_amd as f
    L = f.load()
    FAKE = 0x100000
    assert L.fp8_quant_col_ws_bytes(1, 2100, 16400) == 4 * 16400
    assert L.fp8_quant_col_noalloc(FAKE, 1, 2100, 16400, f.E4M3_NATIVE, EPS, FAKE, FAKE, None, None) == \
        f.ERR_UNSUPPORTED
    assert L.fp8_quant_col_noalloc(FAKE, 1, -1, 8, f.E4M3_NATIVE, EPS, FAKE, FAKE, None, None) == \
        f.ERR_INVALID_ARGUMENT


@gpu
@pytest.mark.skipif(not have_gpu(), reason="needs an MI355X")
def test_noalloc_matches_the_workspace_call_twice():
    import torch
    f = lib()
    L = f.load()
    stream = torch.cuda.current_stream().cuda_stream
    # both shapes take the split form (more than 2048 rows, fewer than 1024 strips)
    for i, (R, C) in enumerate([(4096, 1024), (3008, 520)]):
        assert f.fp8_quant_col_ws_bytes(1, R, C) > 0
        x = torch.from_numpy(synth.normal_bf16((R, C), 77000 + i, 1.0).view(np.int16)).to("cuda:0")
        outs = []
        for noalloc in (False, True):
            qT = torch.full((C, R), 0xA5, dtype=torch.uint8, device="cuda:0")
            sc = torch.full((C,), -1.0, dtype=torch.float32, device="cuda:0")
            iv = torch.full((C,), -1.0, dtype=torch.float32, device="cuda:0")
            if noalloc:
                st = L.fp8_quant_col_noalloc(x.data_ptr(), 1, R, C, f.E4M3_NATIVE, EPS, qT.data_ptr(),
                                             sc.data_ptr(), iv.data_ptr(), stream)
            else:
                ws = torch.empty(f.fp8_quant_col_ws_bytes(1, R, C), dtype=torch.uint8, device="cuda:0")
                st = L.fp8_quant_col(x.data_ptr(), 1, R, C, f.E4M3_NATIVE, EPS, qT.data_ptr(), sc.data_ptr(),
                                     iv.data_ptr(), ws.data_ptr(), ws.numel(), stream)
            assert st == f.OK
            torch.cuda.synchronize()
            outs.append((qT.cpu().numpy(), sc.cpu().numpy(), iv.cpu().numpy()))
        for a, b in zip(outs[0], outs[1]):
            assert np.array_equal(a, b), (R, C)
