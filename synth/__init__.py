"""Seeded synthetic inputs, shared by the tests, the benchmark and the oracle checks.

This module holds no quantization or GEMM arithmetic. It produces bf16 bit
patterns (numpy uint16) from a counter-based SplitMix64 stream (synth.c), plus
the small host-side choices of the workloads (expert routing counts, zeroed
columns, per-row magnitude multipliers).

Workloads (the pages' model shapes; no dataset or trained weights exist here,
so seeded tensors with the stated distributions stand in for them):
  linear_tensorwise  X [256,512] ~N(0,1), W [512,512] ~N(0,0.02)
  linear_rowwise     Llama3-8B MLP: X [8192,4096] ~N(0,1) with 0.1% outliers x50,
                     W [14336,4096] ~N(0,0.02), grad_out [8192,14336] ~N(0,1e-3)
  expert_colwise     W [32][2048][7168] ~N(0,0.02), 2 zero columns per expert
  moe_grouped        16384 tokens x top-8 over 32 experts, Zipf(1.1) with 2 empty
                     experts; A [131072,7168] ~N(0,1), W [32][2048][7168] ~N(0,0.02)
  moe_block_mx       16 experts, K 5120, N 8192, 8192 rows split evenly;
                     N(0,1) * 2^u per row, u ~ U[-8, 8)
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", "-Wall", "-o", tmp, os.path.join(_HERE, "synth.c"), "-lm"],
                   check=True, cwd=_HERE)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, U64, D, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_float
        lib.synth_normal_bf16.restype = None
        lib.synth_normal_bf16.argtypes = [P, I64, I64, U64, D, P]
        lib.synth_outliers_bf16.restype = I64
        lib.synth_outliers_bf16.argtypes = [P, I64, U64, D, F]
        lib.synth_uniform.restype = None
        lib.synth_uniform.argtypes = [P, I64, U64]
        _lib = lib
    return _lib


def normal_bf16(shape, seed: int, sigma: float = 1.0, row_mult: np.ndarray | None = None) -> np.ndarray:
    """bf16 bits of fp32(sigma * N(0,1) * row_mult[row]); rows = prod(shape[:-1])."""
    shape = tuple(int(s) for s in shape)
    cols = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    out = np.empty(shape, np.uint16)
    rm = None
    if row_mult is not None:
        rm = np.ascontiguousarray(row_mult, np.float64)
        assert rm.size == rows
    _load().synth_normal_bf16(out.ctypes.data, rows, cols, int(seed), float(sigma),
                              None if rm is None else rm.ctypes.data)
    return out


def add_outliers(x: np.ndarray, seed: int, p: float = 0.001, mult: float = 50.0) -> int:
    assert x.dtype == np.uint16 and x.flags["C_CONTIGUOUS"]
    return int(_load().synth_outliers_bf16(x.ctypes.data, x.size, int(seed), float(p), float(mult)))


def uniform(n: int, seed: int) -> np.ndarray:
    out = np.empty(int(n), np.float64)
    _load().synth_uniform(out.ctypes.data, int(n), int(seed))
    return out


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()[:16]


def zero_columns(w: np.ndarray, per_expert: int, seed: int) -> np.ndarray:
    """Sets `per_expert` distinct seeded columns of each [R, C] matrix of w [E,R,C] to +0.0.
    Returns the chosen column indices [E, per_expert]."""
    E, _, C = w.shape
    u = uniform(E * C, seed).reshape(E, C)
    cols = np.argsort(u, axis=1, kind="stable")[:, :per_expert]
    for e in range(E):
        w[e][:, cols[e]] = 0
    return cols


def log_uniform_row_mult(rows: int, seed: int, lo: float = -8.0, hi: float = 8.0) -> np.ndarray:
    u = uniform(rows, seed)
    return np.exp2(lo + (hi - lo) * u)


def zipf_routing(tokens: int, topk: int, experts: int, s: float, n_empty: int, seed: int) -> np.ndarray:
    """Per-expert row counts for `tokens` tokens each routed to `topk` distinct experts.
    Expert weights follow rank^-s over a seeded permutation, `n_empty` seeded experts get
    weight 0, and each token picks its experts by Gumbel-top-k. Returns int64 counts [E]."""
    assert topk <= experts - n_empty
    perm = np.argsort(uniform(experts, seed), kind="stable")
    rank = np.empty(experts, np.int64)
    rank[perm] = np.arange(1, experts + 1)
    w = rank.astype(np.float64) ** (-s)
    empty = np.argsort(uniform(experts, seed + 1), kind="stable")[:n_empty]
    w[empty] = 0.0
    logw = np.full(experts, -np.inf)
    logw[w > 0] = np.log(w[w > 0])
    u = uniform(tokens * experts, seed + 2).reshape(tokens, experts)
    with np.errstate(divide="ignore"):
        g = -np.log(-np.log(u))
    keys = logw[None, :] + g
    top = np.argpartition(-keys, topk - 1, axis=1)[:, :topk]
    return np.bincount(top.ravel(), minlength=experts).astype(np.int64)


def offsets_from_counts(counts) -> np.ndarray:
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return off


# ---- workload recipes ----------------------------------------------------------
# Seeds are 1000 * workload_index + tensor_index.

@dataclass
class Workload:
    name: str
    tensors: dict = field(default_factory=dict)
    meta: dict = field(default_factory=dict)


def linear_tensorwise(M=256, K=512, N=512) -> Workload:
    return Workload("linear_tensorwise", {
        "x": normal_bf16((M, K), 1000, 1.0),
        "w": normal_bf16((N, K), 1001, 0.02),
    }, {"M": M, "N": N, "K": K})


def linear_rowwise(M=8192, K=4096, N=14336, with_grad=True) -> Workload:
    x = normal_bf16((M, K), 2000, 1.0)
    n_out = add_outliers(x, 2003, 0.001, 50.0)
    t = {"x": x, "w": normal_bf16((N, K), 2001, 0.02)}
    if with_grad:
        t["gy"] = normal_bf16((M, N), 2002, 1e-3)
    return Workload("linear_rowwise", t, {"M": M, "N": N, "K": K, "outliers": n_out})


def expert_colwise(E=32, R=2048, C=7168, zero_cols=2) -> Workload:
    w = normal_bf16((E, R, C), 3000, 0.02)
    cols = zero_columns(w, zero_cols, 3001) if zero_cols else None
    return Workload("expert_colwise", {"w": w}, {"E": E, "R": R, "C": C, "zero_cols": cols})


def moe_grouped(tokens=16384, topk=8, E=32, N=2048, K=7168, s=1.1, n_empty=2) -> Workload:
    counts = zipf_routing(tokens, topk, E, s, n_empty, 4000)
    off = offsets_from_counts(counts)
    Mtot = int(off[-1])
    return Workload("moe_grouped", {
        "a": normal_bf16((Mtot, K), 4001, 1.0),
        "w": normal_bf16((E, N, K), 4002, 0.02),
    }, {"E": E, "N": N, "K": K, "Mtot": Mtot, "offsets": off, "counts": counts})


def moe_block_mx(E=16, K=5120, N=8192, rows=8192) -> Workload:
    assert rows % E == 0
    off = offsets_from_counts([rows // E] * E)
    a = normal_bf16((rows, K), 5001, 1.0, row_mult=log_uniform_row_mult(rows, 5003))
    w = normal_bf16((E, N, K), 5002, 1.0, row_mult=log_uniform_row_mult(E * N, 5004))
    return Workload("moe_block_mx", {"a": a, "w": w},
                    {"E": E, "N": N, "K": K, "Mtot": rows, "offsets": off})
