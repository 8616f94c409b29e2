"""ctypes binding of liboproj.so: one Python function per C entry point, same
names, argument marshalling only (tensor -> device pointer, stream handle,
status -> exception)."""
from __future__ import annotations

import ctypes
import dataclasses
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboproj.so")

OPROJ_SCALE_FP32 = 0
OPROJ_SCALE_POW2 = 1
OPROJ_SCALE_E8M0 = 2
OPROJ_WBLOCK_128x128 = 0
OPROJ_WBLOCK_1x128 = 1
OPROJ_WBLOCK_1x128_UE8M0 = 2
OPROJ_NOALLOC_SCRATCH_BYTES = 32 << 20  # include/oproj.h: the no-allocation entry point's scratch array

_STATUS = {0: "OPROJ_OK", 1: "OPROJ_E_NULL", 2: "OPROJ_E_SHAPE", 3: "OPROJ_E_ALIGN",
           4: "OPROJ_E_MODE", 5: "OPROJ_E_HIP", 6: "OPROJ_E_SCRATCH"}


class OprojError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} ({oproj_status_string(status)})")


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("T", "n_groups", "heads_per_group", "nope_dim",
                                              "rope_dim", "quant_block", "o_lora_rank", "max_pos")]


class _Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("stride_t", "stride_g", "s_stride_t", "s_stride_g",
                                              "s_stride_kb")]


class _Bf16Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("stride_t", "stride_g")]


@dataclasses.dataclass
class Shape:
    T: int
    n_groups: int
    heads_per_group: int
    o_lora_rank: int = 0
    max_pos: int = 1
    nope_dim: int = 448
    rope_dim: int = 64
    quant_block: int = 128

    @property
    def D(self) -> int:
        return self.heads_per_group * (self.nope_dim + self.rope_dim)

    @property
    def KB(self) -> int:
        return self.D // self.quant_block

    def _c(self) -> _Shape:
        return _Shape(self.T, self.n_groups, self.heads_per_group, self.nope_dim, self.rope_dim,
                      self.quant_block, self.o_lora_rank, self.max_pos)


@dataclasses.dataclass
class ActLayout:
    """Element strides of an FP8 activation operand (codes, then scales)."""

    stride_t: int
    stride_g: int
    s_stride_t: int
    s_stride_g: int
    s_stride_kb: int

    def _c(self) -> _Layout:
        return _Layout(self.stride_t, self.stride_g, self.s_stride_t, self.s_stride_g, self.s_stride_kb)


@dataclasses.dataclass
class Bf16Layout:
    """Element strides of a bf16 activation operand x(t, g, k)."""

    stride_t: int
    stride_g: int

    def _c(self) -> _Bf16Layout:
        return _Bf16Layout(self.stride_t, self.stride_g)


def default_layout(shape: Shape, scale_mode: int = OPROJ_SCALE_FP32) -> ActLayout:
    """Group-major codes [G][T][D] and MN-major scales [G][KB][T] ([G][KB/4][T]
    packed UE8M0 words in OPROJ_SCALE_E8M0 mode)."""
    nw = shape.KB // 4 if scale_mode == OPROJ_SCALE_E8M0 else shape.KB
    return ActLayout(shape.D, shape.T * shape.D, 1, nw * shape.T, shape.T)


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load liboproj.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m attention_output_projection_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        SP, LP, BP = ctypes.POINTER(_Shape), ctypes.POINTER(_Layout), ctypes.POINTER(_Bf16Layout)
        sig = {
            "oproj_inv_rope_quant": (I32, [SP, I32, P, P, P, P, P, LP, P]),
            "oproj_grouped_wo_a": (I32, [SP, I32, P, P, LP, P, P, I32, P, P]),
            "oproj_inv_rope_bf16": (I32, [SP, P, P, P, P, BP, P]),
            "oproj_grouped_wo_a_bf16": (I32, [SP, P, BP, P, P, P]),
            "oproj_dense_bf16_gemm": (I32, [I64, I64, I64, P, P, P, P]),
            "oproj_fused_workspace_bytes": (SZ, [SP, I64]),
            "oproj_fused_decode_workspace_bytes": (SZ, [SP]),
            "oproj_fused_bf16_workspace_bytes": (SZ, [SP, I64]),
            "oproj_fused_bf16": (I32, [SP, P, P, P, P, P, I64, P, SZ, P, P]),
            "oproj_fused": (I32, [SP, I32, P, P, P, P, P, I32, P, I64, P, SZ, P, P]),
            "oproj_inv_rope_quant_f32": (I32, [SP, I32, P, P, P, P, P, LP, P]),
            "oproj_fused_decode": (I32, [SP, I32, P, P, P, P, P, I32, P, SZ, P, P]),
            "oproj_fused_noalloc": (I32, [SP, I32, P, P, P, P, P, I32, P, I64, P, P]),
            "oproj_fused_decode_unsupported": (ctypes.c_char_p, [SP, I32, I32]),
            "oproj_quantize_weight": (I32, [I64, I64, I32, I32, P, P, P, P]),
            "oproj_status_string": (ctypes.c_char_p, [I32]),
            "oproj_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _ptr(x) -> int | None:
    """Device pointer of a tensor (or a raw int / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise OprojError(fn, status)


def _lay(layout):
    return ctypes.byref(layout._c()) if layout is not None else None


def oproj_status_string(status: int) -> str:
    return load_library().oproj_status_string(status).decode()


def oproj_version() -> str:
    return load_library().oproj_version().decode()


def oproj_inv_rope_quant(shape: Shape, scale_mode: int, o, positions, cos_sin, a_codes, a_scales,
                         out_layout: ActLayout | None = None, stream=None) -> None:
    st = load_library().oproj_inv_rope_quant(
        ctypes.byref(shape._c()), scale_mode, _ptr(o), _ptr(positions), _ptr(cos_sin),
        _ptr(a_codes), _ptr(a_scales), _lay(out_layout), _stream(stream))
    _check("oproj_inv_rope_quant", st)


def oproj_inv_rope_quant_f32(shape: Shape, scale_mode: int, o, positions, cos_sin, a_codes, a_scales,
                             out_layout: ActLayout | None = None, stream=None) -> None:
    st = load_library().oproj_inv_rope_quant_f32(
        ctypes.byref(shape._c()), scale_mode, _ptr(o), _ptr(positions), _ptr(cos_sin),
        _ptr(a_codes), _ptr(a_scales), _lay(out_layout), _stream(stream))
    _check("oproj_inv_rope_quant_f32", st)


def oproj_grouped_wo_a(shape: Shape, scale_mode: int, a_codes, a_scales, a_layout, w_codes, w_scales,
                       w_block: int, z, stream=None) -> None:
    st = load_library().oproj_grouped_wo_a(
        ctypes.byref(shape._c()), scale_mode, _ptr(a_codes), _ptr(a_scales), _lay(a_layout),
        _ptr(w_codes), _ptr(w_scales), w_block, _ptr(z), _stream(stream))
    _check("oproj_grouped_wo_a", st)


def oproj_inv_rope_bf16(shape: Shape, o, positions, cos_sin, x, x_layout: Bf16Layout | None = None,
                        stream=None) -> None:
    st = load_library().oproj_inv_rope_bf16(
        ctypes.byref(shape._c()), _ptr(o), _ptr(positions), _ptr(cos_sin), _ptr(x), _lay(x_layout),
        _stream(stream))
    _check("oproj_inv_rope_bf16", st)


def oproj_grouped_wo_a_bf16(shape: Shape, x, x_layout: Bf16Layout | None, w, z, stream=None) -> None:
    st = load_library().oproj_grouped_wo_a_bf16(
        ctypes.byref(shape._c()), _ptr(x), _lay(x_layout), _ptr(w), _ptr(z), _stream(stream))
    _check("oproj_grouped_wo_a_bf16", st)


def oproj_dense_bf16_gemm(M: int, N: int, K: int, x, w, y, stream=None) -> None:
    st = load_library().oproj_dense_bf16_gemm(M, N, K, _ptr(x), _ptr(w), _ptr(y), _stream(stream))
    _check("oproj_dense_bf16_gemm", st)


def oproj_fused_workspace_bytes(shape: Shape, hidden: int = 0) -> int:
    return int(load_library().oproj_fused_workspace_bytes(ctypes.byref(shape._c()), hidden))


def oproj_fused(shape: Shape, scale_mode: int, o, positions, cos_sin, w_codes, w_scales, w_block: int,
                wo_b, hidden: int, workspace, workspace_bytes: int, out, stream=None) -> None:
    st = load_library().oproj_fused(
        ctypes.byref(shape._c()), scale_mode, _ptr(o), _ptr(positions), _ptr(cos_sin), _ptr(w_codes),
        _ptr(w_scales), w_block, _ptr(wo_b), hidden, _ptr(workspace), workspace_bytes, _ptr(out),
        _stream(stream))
    _check("oproj_fused", st)


def oproj_fused_noalloc(shape: Shape, scale_mode: int, o, positions, cos_sin, w_codes, w_scales, w_block: int,
                        wo_b, hidden: int, out, stream=None) -> None:
    st = load_library().oproj_fused_noalloc(
        ctypes.byref(shape._c()), scale_mode, _ptr(o), _ptr(positions), _ptr(cos_sin), _ptr(w_codes),
        _ptr(w_scales), w_block, _ptr(wo_b), hidden, _ptr(out), _stream(stream))
    _check("oproj_fused_noalloc", st)


def oproj_fused_decode(shape: Shape, scale_mode: int, o, positions, cos_sin, w_codes, w_scales, w_block: int,
                       workspace, workspace_bytes: int, z, stream=None) -> None:
    st = load_library().oproj_fused_decode(
        ctypes.byref(shape._c()), scale_mode, _ptr(o), _ptr(positions), _ptr(cos_sin), _ptr(w_codes),
        _ptr(w_scales), w_block, _ptr(workspace), workspace_bytes, _ptr(z), _stream(stream))
    _check("oproj_fused_decode", st)


def oproj_fused_decode_unsupported(shape: Shape, scale_mode: int = 0, w_block: int = 0):
    """None when oproj_fused_decode can take this shape on the current device, else the reason."""
    r = load_library().oproj_fused_decode_unsupported(ctypes.byref(shape._c()), scale_mode, w_block)
    return None if r is None else r.decode()


def oproj_fused_decode_workspace_bytes(shape: Shape) -> int:
    return load_library().oproj_fused_decode_workspace_bytes(ctypes.byref(shape._c()))


def oproj_fused_bf16_workspace_bytes(shape: Shape, hidden: int = 0) -> int:
    return int(load_library().oproj_fused_bf16_workspace_bytes(ctypes.byref(shape._c()), hidden))


def oproj_fused_bf16(shape: Shape, o, positions, cos_sin, w, wo_b, hidden: int, workspace,
                     workspace_bytes: int, out, stream=None) -> None:
    st = load_library().oproj_fused_bf16(
        ctypes.byref(shape._c()), _ptr(o), _ptr(positions), _ptr(cos_sin), _ptr(w), _ptr(wo_b), hidden,
        _ptr(workspace), workspace_bytes, _ptr(out), _stream(stream))
    _check("oproj_fused_bf16", st)


def oproj_quantize_weight(rows: int, K: int, w_block: int, scale_mode: int, w, codes, scales,
                          stream=None) -> None:
    st = load_library().oproj_quantize_weight(rows, K, w_block, scale_mode, _ptr(w), _ptr(codes),
                                              _ptr(scales), _stream(stream))
    _check("oproj_quantize_weight", st)
