"""CPU oracle of the O-projection front half (TEST INFRASTRUCTURE ONLY).

Thin ctypes wrapper over ``oproj_oracle.c`` (plain C, fp64 accumulation).
Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the product library never does and
shares no code with it.

Every function here marshals numpy arrays and calls the C routine that does the
arithmetic; the readings R1..R8 and the page citations are in the C file's
header.  Layouts on this side are plain and token-major:
  codes  uint8  [T, G, D]        scales float32 [T, G, D/128]
  z      float64 [T, G, R]       y      float64 [T, hidden]
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oproj_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboproj_oracle.so")
_CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (host only)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        INT = ctypes.c_int
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_e4m3_decode.restype = ctypes.c_float
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.orc_pow2_ceil.restype = ctypes.c_float
        lib.orc_pow2_ceil.argtypes = [ctypes.c_float]
        for name in ("orc_e4m3_encode_array", "orc_e4m3_decode_array", "orc_f64_to_bf16_array",
                     "orc_pow2_ceil_array"):
            getattr(lib, name).argtypes = [I64, P, P]
            getattr(lib, name).restype = None
        lib.orc_rope_f32.argtypes = [I64, I64, I64, I64, P, P, P, INT]
        lib.orc_block_quant_rows.argtypes = [I64, I64, I64, INT, P, P, P]
        lib.orc_inv_rope_quant.argtypes = [I64, I64, I64, I64, I64, I64, INT, P, P, P, P, P, INT]
        lib.orc_inv_rope_quant_f32.argtypes = [I64, I64, I64, I64, I64, I64, INT, P, P, P, P, P, INT]
        lib.orc_quant_weight.argtypes = [I64, I64, I64, INT, P, P, P]
        lib.orc_grouped_gemm.argtypes = [I64, I64, I64, I64, P, P, I64, I64, I64, I64, I64, P, P,
                                         I64, P, I64, P, INT]
        lib.orc_dense_gemm_bf16.argtypes = [I64, I64, I64, P, P, P, I64, P, INT]
        lib.orc_inv_rope_bf16.argtypes = [I64, I64, I64, I64, P, P, P, P]
        lib.orc_e8m0_byte.argtypes = [ctypes.c_float]
        lib.orc_e8m0_byte.restype = INT
        lib.orc_e8m0_pack.argtypes = [I64, I64, P, P]
        lib.orc_e8m0_pack.restype = INT
        for f in (lib.orc_rope_f32, lib.orc_block_quant_rows, lib.orc_inv_rope_quant, lib.orc_inv_rope_quant_f32,
                  lib.orc_quant_weight, lib.orc_grouped_gemm, lib.orc_dense_gemm_bf16,
                  lib.orc_inv_rope_bf16):
            f.restype = None
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads the oracle uses: the affinity set, capped at 16 (the CPU
    share of one GPU on the measurement hosts)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- codecs
def e4m3_encode(x) -> np.ndarray:
    x = _c(x, np.float32)
    q = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_encode_array(x.size, _p(x), _p(q))
    return q


def e4m3_decode(q) -> np.ndarray:
    q = _c(q, np.uint8)
    x = np.empty(q.shape, np.float32)
    _load().orc_e4m3_decode_array(q.size, _p(q), _p(x))
    return x


def f64_to_bf16(x) -> np.ndarray:
    x = _c(x, np.float64)
    h = np.empty(x.shape, np.uint16)
    _load().orc_f64_to_bf16_array(x.size, _p(x), _p(h))
    return h


def pow2_ceil(x) -> np.ndarray:
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.float32)
    _load().orc_pow2_ceil_array(x.size, _p(x), _p(y))
    return y


# ---------------------------------------------------------------- a1: RoPE
def rope_f32(x, positions, table, nope_dim: int, rope_dim: int, inverse: bool = True) -> np.ndarray:
    """RoPE on fp32 rows x[T, H, nope+rope] (a copy is returned)."""
    x = np.array(x, dtype=np.float32, order="C", copy=True)
    pos = _c(positions, np.int64)
    tab = _c(table, np.float32)
    T, H, hd = x.shape
    assert hd == nope_dim + rope_dim and tab.shape[1] == rope_dim
    _load().orc_rope_f32(T, H, nope_dim, rope_dim, _p(x), _p(pos), _p(tab), -1 if inverse else 1)
    return x


def inv_rope_bf16(o_bf16, positions, table, nope_dim: int = 448, rope_dim: int = 64) -> np.ndarray:
    """Unquantised a1: bf16 bits o[T, H, head_dim] -> bf16 bits x[T, H, head_dim]
    (rotated dims rounded to bf16, the rest copied); view it as [T, G, D]."""
    o = _c(o_bf16, np.uint16)
    pos = _c(positions, np.int64)
    tab = _c(table, np.float32)
    T, H, hd = o.shape
    assert hd == nope_dim + rope_dim and tab.shape[1] == rope_dim
    assert np.all((pos >= 0) & (pos < tab.shape[0]))
    x = np.empty_like(o)
    _load().orc_inv_rope_bf16(T, H, nope_dim, rope_dim, _p(o), _p(pos), _p(tab), _p(x))
    return x


# ---------------------------------------------------------------- a2: quant
def block_quant_rows(v, block: int = 128, pow2: bool = False):
    """Quantise fp32 rows v[rows, D] in 1 x block blocks -> (codes, scales)."""
    v = _c(v, np.float32)
    rows, D = v.shape
    q = np.empty((rows, D), np.uint8)
    s = np.empty((rows, D // block), np.float32)
    _load().orc_block_quant_rows(rows, D, block, int(pow2), _p(v), _p(q), _p(s))
    return q, s


def inv_rope_quant(o_bf16, positions, table, n_groups: int, heads_per_group: int,
                   nope_dim: int = 448, rope_dim: int = 64, block: int = 128, pow2: bool = False,
                   nthreads: int | None = None):
    """a1 + a2: bf16 bits o[T, H, head_dim] -> codes [T, G, D], scales [T, G, D/block]."""
    o = _c(o_bf16, np.uint16)
    pos = _c(positions, np.int64)
    tab = _c(table, np.float32)
    T, H, hd = o.shape
    assert H == n_groups * heads_per_group and hd == nope_dim + rope_dim
    assert np.all((pos >= 0) & (pos < tab.shape[0]))
    D = heads_per_group * hd
    q = np.empty((T, n_groups, D), np.uint8)
    s = np.empty((T, n_groups, D // block), np.float32)
    _load().orc_inv_rope_quant(T, n_groups, heads_per_group, nope_dim, rope_dim, block, int(pow2),
                               _p(o), _p(pos), _p(tab), _p(q), _p(s),
                               nthreads or default_threads())
    return q, s


def inv_rope_quant_f32(o_f32, positions, table, n_groups: int, heads_per_group: int,
                       nope_dim: int = 448, rope_dim: int = 64, block: int = 128, pow2: bool = False,
                       nthreads: int | None = None):
    """The attention-epilogue producer (R11): fp32 o[T, H, head_dim] -> codes
    [T, G, D], scales [T, G, D/block], the same steps as inv_rope_quant."""
    o = np.ascontiguousarray(o_f32)
    assert o.dtype == np.float32
    pos = _c(positions, np.int64)
    tab = _c(table, np.float32)
    T, H, hd = o.shape
    assert H == n_groups * heads_per_group and hd == nope_dim + rope_dim
    assert np.all((pos >= 0) & (pos < tab.shape[0]))
    D = heads_per_group * hd
    q = np.empty((T, n_groups, D), np.uint8)
    s = np.empty((T, n_groups, D // block), np.float32)
    _load().orc_inv_rope_quant_f32(T, n_groups, heads_per_group, nope_dim, rope_dim, block, int(pow2),
                                   _p(o), _p(pos), _p(tab), _p(q), _p(s),
                                   nthreads or default_threads())
    return q, s


def e8m0_pack(scales) -> np.ndarray:
    """Power-of-two fp32 scales [..., n] (n % 4 == 0) -> packed UE8M0 words
    [..., n/4], uint32; block 4j+b in byte b of word j."""
    s = _c(scales, np.float32)
    n = s.shape[-1]
    assert n % 4 == 0
    rows = s.size // n
    w = np.empty(s.shape[:-1] + (n // 4,), np.uint32)
    if _load().orc_e8m0_pack(rows, n, _p(s), _p(w)) != 0:
        raise ValueError("a scale is not a power of two representable in UE8M0")
    return w


def quant_weight(w, block_rows: int = 128, pow2: bool = False):
    """fp32 w[rows, K] -> codes [rows, K], scales [ceil(rows/block_rows), K/128]."""
    w = _c(w, np.float32)
    rows, K = w.shape
    q = np.empty((rows, K), np.uint8)
    s = np.empty(((rows + block_rows - 1) // block_rows, K // 128), np.float32)
    _load().orc_quant_weight(rows, K, block_rows, int(pow2), _p(w), _p(q), _p(s))
    return q, s


def dequant_weight(q, s, block_rows: int = 128) -> np.ndarray:
    """decode(q) * scale per block, fp64 (the scale is a multiplier)."""
    q = _c(q, np.uint8)
    rows, K = q.shape
    lut = e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)  # every code, decoded once
    d = lut[q].reshape(rows, K // 128, 128)
    srow = np.repeat(np.asarray(s, np.float64), block_rows, axis=0)[:rows]
    d *= srow[:, :, None]
    return d.reshape(rows, K)


# ---------------------------------------------------------------- a3: grouped wo_a
def grouped_gemm(qa, sa, qw, sw, n_groups: int, o_lora_rank: int, w_block_rows: int = 128,
                 idx=None, nthreads: int | None = None) -> np.ndarray:
    """fp64 grouped contraction.

    ``qa``/``sa`` are token-major [T, Gp, D] / [T, Gp, D/128] with Gp >= n_groups
    (groups >= n_groups are never read).  Dense result [T, G, R], or, when
    ``idx`` is an int64 array of (t, g, n) triples, the sampled values."""
    qa = _c(qa, np.uint8)
    sa = _c(sa, np.float32)
    qw = _c(qw, np.uint8)
    sw = _c(sw, np.float32)
    T, Gp, D = qa.shape
    KB = D // 128
    assert sa.shape == (T, Gp, KB) and Gp >= n_groups
    assert qw.shape == (n_groups * o_lora_rank, D)
    lib = _load()
    nt = nthreads or default_threads()
    if idx is None:
        z = np.empty((T, n_groups, o_lora_rank), np.float64)
        lib.orc_grouped_gemm(T, n_groups, D, o_lora_rank, _p(qa), _p(sa), Gp * D, D, Gp * KB, KB, 1,
                             _p(qw), _p(sw), w_block_rows, None, 0, _p(z), nt)
        return z
    idx = _c(idx, np.int64).reshape(-1, 3)
    z = np.empty(idx.shape[0], np.float64)
    lib.orc_grouped_gemm(T, n_groups, D, o_lora_rank, _p(qa), _p(sa), Gp * D, D, Gp * KB, KB, 1,
                         _p(qw), _p(sw), w_block_rows, _p(idx), idx.shape[0], _p(z), nt)
    return z


# ---------------------------------------------------------------- a4: wo_b
def dense_gemm_bf16(x_bf16, w_bf16, idx=None, nthreads: int | None = None) -> np.ndarray:
    """fp64 y = x @ w.T for bf16 bits x[M, K], w[N, K]; dense or sampled at (m, j) pairs."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2
    lib = _load()
    nt = nthreads or default_threads()
    if idx is None:
        y = np.empty((M, N), np.float64)
        lib.orc_dense_gemm_bf16(M, N, K, _p(x), _p(w), None, 0, _p(y), nt)
        return y
    idx = _c(idx, np.int64).reshape(-1, 2)
    y = np.empty(idx.shape[0], np.float64)
    lib.orc_dense_gemm_bf16(M, N, K, _p(x), _p(w), _p(idx), idx.shape[0], _p(y), nt)
    return y


# ---------------------------------------------------------------- a3 unquantised
def grouped_gemm_bf16(x_bf16, w_bf16, n_groups: int, o_lora_rank: int, idx=None,
                      nthreads: int | None = None) -> np.ndarray:
    """fp64 grouped contraction of bf16 operands: one matmul per group,
    z[t, g, n] = sum_k x[t, g, k] * w[g*R + n, k].

    ``x_bf16`` is [T, G, D] (any strides numpy can view), ``w_bf16`` [G*R, D].
    Dense result [T, G, R], or the values at int64 (t, g, n) triples ``idx``."""
    x = np.asarray(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    T, G, D = x.shape
    R = o_lora_rank
    assert G == n_groups and w.shape == (G * R, D)
    if idx is None:
        z = np.empty((T, G, R), np.float64)
        for g in range(G):
            z[:, g, :] = dense_gemm_bf16(np.ascontiguousarray(x[:, g, :]), w[g * R:(g + 1) * R],
                                         nthreads=nthreads)
        return z
    idx = _c(idx, np.int64).reshape(-1, 3)
    z = np.empty(idx.shape[0], np.float64)
    for g in np.unique(idx[:, 1]):
        sel = np.nonzero(idx[:, 1] == g)[0]
        pairs = np.stack([idx[sel, 0], idx[sel, 2]], axis=1)
        z[sel] = dense_gemm_bf16(np.ascontiguousarray(x[:, g, :]), w[g * R:(g + 1) * R], idx=pairs,
                                 nthreads=nthreads)
    return z


# ---------------------------------------------------------------- whole-tensor forms (full-size parity)
def dequant_act(qa, sa, n_groups: int | None = None) -> np.ndarray:
    """decode(q) * scale for token-major activations [T, Gp, D] / [T, Gp, D/128]
    (the scale multiplies its 128-wide block), fp64 [T, G, D]; only groups <
    n_groups are decoded (a pre-quantised input's padding groups are dropped)."""
    qa = np.asarray(qa, np.uint8)
    sa = np.asarray(sa, np.float32)
    T, Gp, D = qa.shape
    G = Gp if n_groups is None else n_groups
    lut = e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)  # every code, decoded once
    d = lut[qa[:, :G]].reshape(T, G, D // 128, 128)
    d *= sa[:, :G, :, None].astype(np.float64)
    return d.reshape(T, G, D)


def grouped_gemm_full(qa, sa, qw, sw, n_groups: int, o_lora_rank: int,
                      w_block_rows: int = 128) -> np.ndarray:
    """The contraction of grouped_gemm over every output, for full-size
    operands: each operand is dequantised once (decode(q) * scale, fp64) and
    group g's output is one fp64 matrix product of its [T, D] activations with
    weight rows g*R .. g*R+R-1 (vLLM API page
    "vllm.models.deepseek_v4.nvidia.ops.o_proj", deep_gemm_fp8_o_proj: einsum
    "bhr,hdr->bhd" over wo_a viewed [G, R, D]; the matrix product is numpy's).
    Token-major [T, Gp, D] / [T, Gp, D/128] in (Gp >= n_groups), fp64 [T, G, R] out."""
    G, R = n_groups, o_lora_rank
    qw = np.asarray(qw, np.uint8)
    assert qw.shape[0] == G * R and qa.shape[1] >= G
    wd = dequant_weight(qw, sw, w_block_rows)
    T = qa.shape[0]
    z = np.empty((T, G, R), np.float64)
    for g in range(G):
        ad = dequant_act(qa[:, g:g + 1], sa[:, g:g + 1])[:, 0]
        z[:, g, :] = ad @ wd[g * R:(g + 1) * R].T
    return z


def bf16_to_f64(h) -> np.ndarray:
    """bf16 bit patterns -> fp64 values (exact: the bits are the top half of an fp32)."""
    return (np.asarray(h, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def dense_gemm_bf16_full(x_bf16, w_bf16) -> np.ndarray:
    """fp64 y = x @ w.T over every output for bf16 bits x[M, K], w[N, K] (the
    linear layer wo_b of the sglang source page "python/sglang/srt/models/deepseek_v4.py",
    MQALayer.forward, over the flattened z); the matrix product is numpy's."""
    x = bf16_to_f64(x_bf16)
    w = bf16_to_f64(w_bf16)
    assert x.shape[1] == w.shape[1]
    return x @ w.T
