"""Regression checks on our own gfx950 builds (CPU only), from the device assembly
hipcc -S produces for the library's sources with the library's flags:
 1. no matrix-core instruction writes a destination that overlaps its A or B source
    registers (the multi-pass f8f6f4 MFMAs return wrong values when it does, and this
    compiler does not prevent it by itself; the kernels keep operands live past each
    MFMA);
 2. no VGPR an MFMA reads (A, B or scale) is written by a VALU instruction less than
    two VALU issue slots (VALU instructions or s_nop wait states) before it: measured
    on MI355X, an f8f6f4 MFMA issued right after the VALU write of its first source
    registers reads the old value, and scalar instructions in between do not help."""
import os
import re
import subprocess

import pytest

from fp8_dynamic_scaling_amd import build as hb

REG = re.compile(r"^([va])(?:\[(\d+):(\d+)\]|(\d+))$")


def _range(tok):
    m = REG.match(tok.strip())
    if not m:
        return None
    if m.group(4) is not None:
        i = int(m.group(4))
        return m.group(1), i, i
    return m.group(1), int(m.group(2)), int(m.group(3))


def mfma_overlaps(asm: str):
    bad = []
    for line in asm.splitlines():
        line = line.strip()
        if not line.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in line.split(None, 1)[1].split(",")]
        dst, a, b = (_range(o) for o in ops[:3])
        for src in (a, b):
            if dst and src and dst[0] == src[0] and not (dst[2] < src[1] or src[2] < dst[1]):
                bad.append(line)
    return bad


def _slots(line):
    """VALU issue slots an instruction provides between a write and a read."""
    if line.startswith("s_nop"):
        return int(line.split()[1]) + 1
    if line.startswith("v_"):
        return 1
    return 0


def mfma_raw_hazards(asm: str, need: int = 2):
    lines = [l.strip() for l in asm.splitlines()]
    lines = [l for l in lines if l and not l.startswith((";", ".")) and not l.endswith(":")]
    bad = []
    for i, line in enumerate(lines):
        if not line.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in line.split(None, 1)[1].split(",")]
        srcs = [_range(o.split()[0]) for o in ops[1:3] + ops[4:6]]
        srcs = [r for r in srcs if r and r[0] == "v"]
        slots = 0
        for j in range(i - 1, max(i - 40, -1), -1):
            prev = lines[j]
            if prev.startswith("v_") and not prev.startswith("v_mfma"):
                parts = prev.split(None, 1)
                dst = _range(parts[1].split(",")[0]) if len(parts) > 1 else None
                if dst and any(dst[0] == r[0] and not (dst[2] < r[1] or r[2] < dst[1]) for r in srcs):
                    if slots < need:
                        bad.append((prev, line, slots))
                    break
            slots += _slots(prev)
            if slots >= need + 8:
                break
    return bad


def test_raw_checker_flags_a_close_write():
    asm = "v_mov_b64_e32 v[100:101], v[2:3]\nv_mfma_scale_f32_16x16x128_f8f6f4 v[18:21], v[100:107], v[108:115], 0, v1, v1"
    assert mfma_raw_hazards(asm)
    asm = "v_mov_b32 v8, 0x7f\ns_getpc_b64 s[0:1]\nv_mfma_scale_f32_16x16x128_f8f6f4 a[0:3], v[0:7], v[0:7], 0, v8, v8"
    assert mfma_raw_hazards(asm)
    asm = "v_mov_b32 v8, 0x7f\ns_nop 7\nv_mfma_scale_f32_16x16x128_f8f6f4 a[0:3], v[0:7], v[0:7], 0, v8, v8"
    assert not mfma_raw_hazards(asm)


def test_checker_flags_an_overlap():
    assert mfma_overlaps("v_mfma_scale_f32_16x16x128_f8f6f4 v[6:9], v[6:13], v[6:13], 0, v1, v1")
    assert not mfma_overlaps("v_mfma_scale_f32_16x16x128_f8f6f4 v[18:21], v[2:9], v[10:17], 0, v1, v1")
    assert not mfma_overlaps("v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]")


@pytest.mark.parametrize("src", ["gemm_fp8.hip", "gemm_fp8_fast.hip", "gemm_bf16.hip", "probe.hip"])
def test_no_mfma_destination_overlaps_its_sources(src, tmp_path):
    path = os.path.join(hb.HERE, "csrc", src)
    out = tmp_path / (src + ".s")
    cmd = [hb.HIPCC] + hb.COMMON + ["--cuda-device-only", "-S", path, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert "v_mfma" in asm
    bad = mfma_overlaps(asm)
    assert not bad, bad[:5]
    raw = mfma_raw_hazards(asm)
    assert not raw, raw[:5]


def test_norm_kernels_fuse_no_fp32_multiply_add(tmp_path):
    """The fused normalization's fp32 steps round one by one, as the definition's
    (x - mean) * rstd * gamma + beta does: built with the library's flags for its file,
    no k_norm_quant_row instantiation may contain an fp32 fma (hip's __fmul_rn and
    __fadd_rn are plain operators that contraction would fuse)."""
    src = "quant.hip"
    path = os.path.join(hb.HERE, "csrc", src)
    out = tmp_path / (src + ".s")
    cmd = [hb.HIPCC] + hb.COMMON + hb.NO_CONTRACT.get(src, []) + ["--cuda-device-only", "-S", path, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    cur, seen, bad = None, 0, []
    for line in out.read_text().splitlines():
        m = re.match(r"^(_Z\S*k_norm_quant_row\S*):", line)
        if m:
            cur, seen = m.group(1), seen + 1
            continue
        if cur and line.strip().startswith(".Lfunc_end"):
            cur = None
        if cur and re.search(r"\bv_(pk_)?fmac?_f32\b", line):
            bad.append((cur, line.strip()))
    assert seen >= 4 and not bad, bad[:3]
