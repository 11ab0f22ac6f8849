"""Host-side parts of bench.py (no GPU): the one-GPU guard, the input digests
and the gating of the stored HBM-traffic figure by the kernel sources."""
import hashlib
import os
import subprocess
import sys

import numpy as np

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _small():
    synth.build(force=False)
    return {"linear_tensorwise": synth.linear_tensorwise(M=32, K=64, N=48),
            "moe_grouped": synth.moe_grouped(tokens=64, topk=2, E=4, N=32, K=64, n_empty=1)}


def test_input_digests_cover_every_generated_input():
    bench.EXTRA_INPUT_SHA.clear()
    wls = _small()
    d = bench.input_digests(wls)
    assert set(d) == {"linear_tensorwise.x", "linear_tensorwise.w", "moe_grouped.a", "moe_grouped.w",
                      "moe_grouped.offsets"}
    # the first 16 hex digits of sha256 over the array's bytes
    a = wls["moe_grouped"].tensors["a"]
    assert d["moe_grouped.a"] == hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
    off = wls["moe_grouped"].meta["offsets"]
    assert d["moe_grouped.offsets"] == hashlib.sha256(np.asarray(off).tobytes()).hexdigest()[:16]
    # regenerating gives the same bytes; another seed does not
    assert bench.input_digests(_small()) == d
    other = synth.normal_bf16(a.shape, 999, 1.0)
    assert synth.sha256(other) != d["moe_grouped.a"]


def test_extra_inputs_join_the_digests():
    bench.EXTRA_INPUT_SHA.clear()
    bench.EXTRA_INPUT_SHA["moe_grouped.grad_out"] = "0123456789abcdef"
    try:
        d = bench.input_digests(_small())
        assert d["moe_grouped.grad_out"] == "0123456789abcdef"
    finally:
        bench.EXTRA_INPUT_SHA.clear()


def test_stored_traffic_needs_matching_sources(tmp_path, monkeypatch):
    table = tmp_path / "traffic.md"
    cur = bench.sources_digest("gemm8")
    table.write_text("| bench row | sources | a | b | bytes |\n|---|---|---|---|---|\n"
                     f"| moe_grouped.grouped_gemm | {cur} | 1 | 2 | 4416396415 |\n"
                     "| linear_rowwise.gemm_fwd | 0000000000000000 | 1 | 2 | 123 |\n")
    monkeypatch.setattr(bench, "TRAFFIC_TABLE", str(table))
    assert bench.stored_traffic("moe_grouped.grouped_gemm", "gemm8") == 4416396415
    # taken for other sources: not reported
    assert bench.stored_traffic("linear_rowwise.gemm_fwd", "gemm8") is None
    assert bench.stored_traffic("no.such_row", "gemm8") is None
    monkeypatch.setattr(bench, "TRAFFIC_TABLE", str(tmp_path / "missing.md"))
    assert bench.stored_traffic("moe_grouped.grouped_gemm", "gemm8") is None


def test_sources_digest_follows_the_kernel_files():
    # one digest per kernel kind, over the files that build its kernels
    assert bench.sources_digest("gemm8") != bench.sources_digest("quant")
    h = hashlib.sha256()
    for fn in bench.KERNEL_SOURCES["quant"]:
        with open(os.path.join(ROOT, "fp8_dynamic_scaling_amd", "csrc", fn), "rb") as fh:
            h.update(fh.read())
    assert bench.sources_digest("quant") == h.hexdigest()[:16]


def test_clock_sampler_parses_dpm_levels():
    """The current DPM level line ('*') of pp_dpm_sclk / pp_dpm_mclk, and rocm-smi's
    '(2100Mhz)' strings, give MHz; no samples give None."""
    assert bench.ClockSampler._mhz("2: 2400Mhz *") == 2400
    assert bench.ClockSampler._mhz("(1900Mhz)") == 1900
    assert bench.ClockSampler._mhz("level 3") is None
    c = bench.ClockSampler()
    c.samples = {"sclk": [2000, 2100, 2400], "mclk": []}
    s = c.summary()
    assert s["sclk_mhz"] == {"min": 2000, "median": 2100, "max": 2400, "samples": 3}
    assert s["mclk_mhz"] is None
