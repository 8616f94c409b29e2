"""Seeded synthetic inputs for the O-projection front half.

This module only draws inputs.  It holds none of the method's arithmetic (no
RoPE, no quantisation, no contraction): both the oracle and the HIP library
read exactly the bytes produced here.

Generator (counter based, so any slice can be drawn independently):
  * SplitMix64 (Vigna): output i of stream ``seed`` is mix(seed + (i+1)*0x9E3779B97F4A7C15).
  * uniform u in (0, 1):   ((x >> 11) + 0.5) * 2**-53
  * standard normal:       Box-Muller cosine branch on the uniform pair (u[2i], u[2i+1])
  * bf16 values:           fp64 -> fp32 (nearest even) -> bf16 (nearest even)
  * seeds:                 (workload_id << 32) | tensor_id

The cos||sin table is an input of the method (the caller precomputes it): row p
holds cos(p * base**(-2i/rope_dim)) for i < rope_dim/2, then the matching sines,
evaluated in fp64 and rounded to fp32.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)

# tensor ids inside a workload's seed space
T_O, T_POS, T_WOA, T_WOB, T_OUTLIER, T_RAGGED, T_EXTRA = 1, 2, 3, 4, 5, 6, 7

_CHUNK = 1 << 22


def seed_of(workload_id: int, tensor_id: int) -> int:
    return ((int(workload_id) & 0xFFFFFFFF) << 32) | (int(tensor_id) & 0xFFFFFFFF)


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * M1
    z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, start: int, n: int) -> np.ndarray:
    """Outputs start .. start+n-1 of the SplitMix64 stream seeded with ``seed``."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        state = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * GOLDEN
        return _mix(state)


def uniform(seed: int, n: int, start: int = 0) -> np.ndarray:
    x = splitmix64(seed, start, n)
    return ((x >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def _normal_chunk(seed: int, start: int, n: int) -> np.ndarray:
    u = uniform(seed, 2 * n, 2 * start)
    u1, u2 = u[0::2], u[1::2]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def _chunked(n: int, fn, dtype) -> np.ndarray:
    out = np.empty(n, dtype=dtype)
    starts = list(range(0, n, _CHUNK))

    def work(s):
        e = min(n, s + _CHUNK)
        out[s:e] = fn(s, e - s)

    if len(starts) <= 1:
        for s in starts:
            work(s)
    else:
        with ThreadPoolExecutor(max_workers=8) as ex:
            list(ex.map(work, starts))
    return out


def normal(seed: int, n: int, std: float = 1.0) -> np.ndarray:
    """n standard normals times ``std``, fp64 (numpy; small draws)."""
    return _chunked(n, lambda s, m: _normal_chunk(seed, s, m) * std, np.float64)


# ---------------------------------------------------------------- bulk draws in C
_HERE = os.path.dirname(os.path.abspath(__file__))
_GEN_SRC = os.path.join(_HERE, "gen.c")
_GEN_LIB = os.path.join(_HERE, "libworkloads_gen.so")
_gen = None


def build(force: bool = False) -> str:
    """Compile the bulk generator (host only, gcc)."""
    if force or not os.path.exists(_GEN_LIB) or os.path.getmtime(_GEN_LIB) < os.path.getmtime(_GEN_SRC):
        tmp = _GEN_LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", tmp, _GEN_SRC, "-lm", "-lpthread"])
        os.replace(tmp, _GEN_LIB)
    return _GEN_LIB


def _genlib():
    global _gen
    if _gen is None:
        build()
        lib = ctypes.CDLL(_GEN_LIB)
        U64, P, D, I = ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
        lib.wl_normal_f32.argtypes = [U64, U64, D, P, I]
        lib.wl_normal_bf16.argtypes = [U64, U64, D, U64, D, D, P, I]
        lib.wl_normal_f32.restype = None
        lib.wl_normal_bf16.restype = None
        _gen = lib
    return _gen


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


def normal_f32_bulk(seed: int, n: int, std: float = 1.0) -> np.ndarray:
    """Same draws as ``normal(seed, n, std).astype(float32)`` (libm in C)."""
    out = np.empty(n, np.float32)
    _genlib().wl_normal_f32(seed & 0xFFFFFFFFFFFFFFFF, n, std, out.ctypes.data, _threads())
    return out


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, nearest even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, n: int, std: float = 1.0, outlier_seed: int | None = None,
                outlier_p: float = 0.0, outlier_mult: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of N(0, std^2) draws; optionally each element is
    multiplied by ``outlier_mult`` with probability ``outlier_p`` (drawn from
    ``outlier_seed``) before rounding.  Bulk path in C."""
    out = np.empty(n, np.uint16)
    op = outlier_p if outlier_seed is not None else 0.0
    _genlib().wl_normal_bf16(seed & 0xFFFFFFFFFFFFFFFF, n, std,
                             (outlier_seed or 0) & 0xFFFFFFFFFFFFFFFF, op, outlier_mult,
                             out.ctypes.data, _threads())
    return out


def normal_bf16_numpy(seed: int, n: int, std: float = 1.0, outlier_seed: int | None = None,
                      outlier_p: float = 0.0, outlier_mult: float = 1.0) -> np.ndarray:
    """numpy statement of ``normal_bf16`` (small n; checks the C path)."""

    def fn(s, m):
        v = _normal_chunk(seed, s, m) * std
        if outlier_seed is not None and outlier_p > 0.0:
            u = uniform(outlier_seed, m, s)
            v = np.where(u < outlier_p, v * outlier_mult, v)
        return f32_to_bf16_bits(v.astype(np.float32))

    return _chunked(n, fn, np.uint16)


def uniform_int(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi) (multiply-shift on the top 32 bits)."""
    x = splitmix64(seed, 0, n) >> np.uint64(32)
    span = np.uint64(hi - lo)
    return (lo + ((x * span) >> np.uint64(32))).astype(np.int64)


def fp8_codes(seed: int, n: int) -> np.ndarray:
    """n random e4m3fn codes (uint8): the bytes of the SplitMix64 stream, with
    the two NaN patterns (S.1111.111) turned into +-448 (S.1111.110)."""
    def chunk(s, m):  # chunk starts are multiples of 8 bytes
        w = (m + 7) // 8
        b = splitmix64(seed, s // 8, w).view(np.uint8)[:m]
        return np.where((b & 0x7F) == 0x7F, b ^ np.uint8(1), b)
    return _chunked(n, chunk, np.uint8)


def cos_sin_table(max_pos: int, rope_dim: int, base: float = 10000.0) -> np.ndarray:
    """fp32 [max_pos, rope_dim]: cos of each pair's angle, then the sines."""
    half = rope_dim // 2
    inv_freq = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / rope_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def ragged_positions(seed: int, T: int, n_seq: int, max_pos: int) -> np.ndarray:
    """T positions from n_seq sequences of random lengths (each >= 1, summing
    to T); sequence j occupies ctx_j + [0, L_j) with ctx_j uniform in
    [0, max_pos - L_j]."""
    u = uniform(seed, n_seq - 1 + n_seq)
    cuts = np.sort((u[: n_seq - 1] * (T - n_seq + 1)).astype(np.int64))
    extra = np.diff(np.concatenate([[0], cuts, [T - n_seq]]))
    lens = extra + 1
    pos = []
    for j, L in enumerate(lens):
        ctx = int(u[n_seq - 1 + j] * (max_pos - L + 1))
        pos.append(np.arange(ctx, ctx + L, dtype=np.int64))
    return np.concatenate(pos)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration of the path."""

    wid: int
    name: str
    T: int
    n_groups: int
    heads_per_group: int
    o_lora_rank: int
    max_pos: int
    positions: str  # "uniform" | "contiguous" | "ragged"
    pow2: bool = False
    w_block_rows: int = 128  # 128: 128x128 weight blocks; 1: 1x128 per-row blocks
    pad_groups: int = 0  # trailing padding groups of a pre-quantised input
    prequantised: bool = False
    outlier_p: float = 0.0
    outlier_mult: float = 1.0
    hidden: int = 0  # wo_b output width (0: no wo_b)
    n_seq: int = 1
    nope_dim: int = 448
    rope_dim: int = 64
    quant_block: int = 128
    rope_base: float = 10000.0

    @property
    def head_dim(self) -> int:
        return self.nope_dim + self.rope_dim

    @property
    def H(self) -> int:
        return self.n_groups * self.heads_per_group

    @property
    def D(self) -> int:
        return self.heads_per_group * self.head_dim

    @property
    def KB(self) -> int:
        return self.D // self.quant_block

    def scaled(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=T)


WORKLOADS = {
    "tiny": Workload(0, "tiny", T=4, n_groups=2, heads_per_group=2, o_lora_rank=64,
                     max_pos=4096, positions="uniform"),
    "decode": Workload(1, "decode", T=64, n_groups=16, heads_per_group=8, o_lora_rank=1024,
                       max_pos=32768, positions="uniform"),
    "prefill": Workload(2, "prefill", T=8192, n_groups=16, heads_per_group=8, o_lora_rank=1024,
                        max_pos=32768, positions="contiguous", n_seq=4, outlier_p=0.01,
                        outlier_mult=50.0),
    "pow2": Workload(3, "pow2", T=2048, n_groups=8, heads_per_group=8, o_lora_rank=1024,
                     max_pos=131072, positions="uniform", pow2=True, w_block_rows=1, pad_groups=2,
                     prequantised=True),
    "full": Workload(4, "full", T=4096, n_groups=16, heads_per_group=8, o_lora_rank=1024,
                     max_pos=131072, positions="ragged", n_seq=8, hidden=7168),
}


def positions(w: Workload) -> np.ndarray:
    s = seed_of(w.wid, T_POS)
    if w.positions == "uniform":
        return uniform_int(s, w.T, 0, w.max_pos)
    if w.positions == "contiguous":
        return np.arange(w.T, dtype=np.int64) % w.max_pos
    if w.positions == "ragged":
        return ragged_positions(seed_of(w.wid, T_RAGGED), w.T, w.n_seq, w.max_pos)
    raise ValueError(w.positions)


def attn_out(w: Workload) -> np.ndarray:
    """bf16 bit patterns [T, H, head_dim] of the attention output."""
    n = w.T * w.H * w.head_dim
    h = normal_bf16(seed_of(w.wid, T_O), n, 1.0,
                    outlier_seed=seed_of(w.wid, T_OUTLIER) if w.outlier_p > 0 else None,
                    outlier_p=w.outlier_p, outlier_mult=w.outlier_mult)
    return h.reshape(w.T, w.H, w.head_dim)


def table(w: Workload) -> np.ndarray:
    return cos_sin_table(w.max_pos, w.rope_dim, w.rope_base)


def wo_a_f32(w: Workload) -> np.ndarray:
    """fp32 [G*R, D] wo_a weight before quantisation, N(0, 0.02^2)."""
    n = w.n_groups * w.o_lora_rank * w.D
    return normal_f32_bulk(seed_of(w.wid, T_WOA), n, 0.02).reshape(
        w.n_groups * w.o_lora_rank, w.D)


def wo_a_bf16(w: Workload) -> np.ndarray:
    """bf16 bit patterns [G*R, D] of an unquantised wo_a: the fp32 weight of
    wo_a_f32 rounded to bf16 (nearest even)."""
    return f32_to_bf16_bits(wo_a_f32(w))


def wo_b_bf16(w: Workload) -> np.ndarray:
    """bf16 bit patterns [hidden, G*R] of wo_b, N(0, 0.02^2)."""
    n = w.hidden * w.n_groups * w.o_lora_rank
    return normal_bf16(seed_of(w.wid, T_WOB), n, 0.02).reshape(w.hidden, w.n_groups * w.o_lora_rank)


def bf16_matrix(seed: int, rows: int, cols: int, std: float) -> np.ndarray:
    return normal_bf16(seed, rows * cols, std).reshape(rows, cols)
