"""The C-ABI library on the host: it loads, exports every symbol include/oproj.h
declares, and its argument validation returns the documented status codes
before anything touches a GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import attention_output_projection_amd as ap
from attention_output_projection_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oproj.h")

E_OK, E_NULL, E_SHAPE, E_ALIGN, E_MODE = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ap.library_path()):
        pytest.fail("liboproj.so is not built (run __graft_entry__.build())")
    return ap.load_library()


def _declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(oproj_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = _declared_symbols()
    for s in ("oproj_inv_rope_quant", "oproj_grouped_wo_a", "oproj_fused", "oproj_inv_rope_bf16",
              "oproj_grouped_wo_a_bf16",
              "oproj_fused_workspace_bytes", "oproj_dense_bf16_gemm", "oproj_quantize_weight",
              "oproj_status_string", "oproj_version"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    for s in _declared_symbols():
        assert hasattr(lib, s), s


def test_status_strings_and_version(lib):
    assert ap.oproj_status_string(0) == "ok"
    assert "shape" in ap.oproj_status_string(2)
    assert re.fullmatch(r"\d+\.\d+\.\d+", ap.oproj_version())


def _shape(**kw):
    base = dict(T=4, n_groups=2, heads_per_group=2, o_lora_rank=64, max_pos=4096)
    base.update(kw)
    return _native.Shape(**base)


def _raw(fn, *args):
    return getattr(ap.load_library(), fn)(*args)


def _irq(shape, mode=0, ptrs=(0x1000,) * 5, layout=None):
    return _raw("oproj_inv_rope_quant", ctypes.byref(shape._c()), mode, *ptrs,
                ctypes.byref(layout._c()) if layout else None, None)


def _gemm(shape, mode=0, wblock=0, ptrs=(0x1000,) * 5, layout=None):
    a, sa, w, sw, z = ptrs
    return _raw("oproj_grouped_wo_a", ctypes.byref(shape._c()), mode, a, sa,
                ctypes.byref(layout._c()) if layout else None, w, sw, wblock, z, None)


BAD = 0x1001  # misaligned fake address: validation rejects it before any use


def test_inv_rope_quant_validation(lib):
    assert _irq(_shape(T=0), ptrs=(None,) * 5) == E_OK
    assert _irq(_shape(T=-1)) == E_SHAPE
    assert _irq(_shape(n_groups=0)) == E_SHAPE
    assert _irq(_shape(nope_dim=447)) == E_SHAPE  # head_dim % block != 0
    assert _irq(_shape(nope_dim=320, rope_dim=192)) == E_SHAPE  # nope % blk != blk - rope
    assert _irq(_shape(nope_dim=449, rope_dim=63)) == E_SHAPE  # odd rope_dim
    assert _irq(_shape(nope_dim=960, rope_dim=64)) == E_MODE  # consistent but not 448+64
    assert _irq(_shape(quant_block=64, nope_dim=448, rope_dim=64)) in (E_SHAPE, E_MODE)
    assert _irq(_shape(heads_per_group=3)) == E_MODE
    assert _irq(_shape(), mode=7) == E_MODE
    assert _irq(_shape(), ptrs=(None, 0x1000, 0x1000, 0x1000, 0x1000)) == E_NULL
    assert _irq(_shape(), ptrs=(BAD, 0x1000, 0x1000, 0x1000, 0x1000)) == E_ALIGN
    assert _irq(_shape(), ptrs=(0x1000, 0x1004, 0x1000, 0x1000, 0x1000)) == E_ALIGN  # int64 positions
    lay = _native.ActLayout(1000, 16, 1, 1, 1)  # stride_t not a multiple of 16
    assert _irq(_shape(), layout=lay) == E_ALIGN
    assert _irq(_shape(), layout=_native.ActLayout(-16, 16, 1, 1, 1)) == E_SHAPE


def test_grouped_gemm_validation(lib):
    assert _gemm(_shape(T=0), ptrs=(None,) * 5) == E_OK
    assert _gemm(_shape(o_lora_rank=0)) == E_SHAPE
    assert _gemm(_shape(o_lora_rank=96)) == E_SHAPE  # not a multiple of 64
    assert _gemm(_shape(), wblock=5) == E_MODE
    assert _gemm(_shape(), mode=3) == E_MODE
    assert _gemm(_shape(), ptrs=(0x1000, 0x1000, None, 0x1000, 0x1000)) == E_NULL
    assert _gemm(_shape(), ptrs=(0x1000, 0x1000, 0x1000, 0x1000, BAD)) == E_ALIGN
    assert _gemm(_shape(), ptrs=(0x1000, 0x1002, 0x1000, 0x1000, 0x1000)) == E_ALIGN
    # 32-bit lane offsets: one group of D = 4096 holds at most 2^20 - 1 tokens,
    # half as many with a token stride of two rows
    big = dict(n_groups=1, heads_per_group=8, o_lora_rank=64)
    assert _gemm(_shape(T=1 << 20, **big)) == E_SHAPE
    assert _gemm(_shape(T=(1 << 19) + 1, **big), layout=_native.ActLayout(8192, 4096, 1, 1, 1 << 20)) == E_SHAPE


def test_dense_gemm_validation(lib):
    f = lambda M, N, K, x=0x1000, w=0x1000, y=0x1000: _raw("oproj_dense_bf16_gemm", M, N, K, x, w, y, None)
    assert f(0, 7168, 16384) == E_OK
    assert f(-1, 7168, 16384) == E_SHAPE
    assert f(4, 7168, 100) == E_SHAPE
    assert f(4, 7000, 128) == E_SHAPE  # N % 16 != 0
    assert f(1 << 17, 16, 1 << 15) == E_SHAPE  # activation operand beyond 4 GiB
    assert f(4, 1 << 17, 1 << 15) == E_SHAPE  # weight operand beyond 4 GiB
    assert f(4, 16, 64, x=None) == E_NULL
    assert f(4, 16, 64, y=BAD) == E_ALIGN


def _rb(shape, ptrs=(0x1000,) * 4, layout=None):
    o, pos, tab, x = ptrs
    return _raw("oproj_inv_rope_bf16", ctypes.byref(shape._c()), o, pos, tab, x,
                ctypes.byref(layout._c()) if layout else None, None)


def _gb(shape, ptrs=(0x1000,) * 3, layout=None):
    x, w, z = ptrs
    return _raw("oproj_grouped_wo_a_bf16", ctypes.byref(shape._c()), x,
                ctypes.byref(layout._c()) if layout else None, w, z, None)


def test_inv_rope_bf16_validation(lib):
    assert _rb(_shape(T=0), ptrs=(None,) * 4) == E_OK
    assert _rb(_shape(T=-2)) == E_SHAPE
    assert _rb(_shape(nope_dim=960, rope_dim=64)) == E_MODE
    assert _rb(_shape(heads_per_group=3)) == E_MODE
    assert _rb(_shape(), ptrs=(0x1000, None, 0x1000, 0x1000)) == E_NULL
    assert _rb(_shape(), ptrs=(0x1000, 0x1000, 0x1000, BAD)) == E_ALIGN
    assert _rb(_shape(), ptrs=(0x1000, 0x1004, 0x1000, 0x1000)) == E_ALIGN  # int64 positions
    assert _rb(_shape(), layout=_native.Bf16Layout(1020, 8)) == E_ALIGN
    assert _rb(_shape(), layout=_native.Bf16Layout(1024, -8)) == E_SHAPE


def test_grouped_wo_a_bf16_validation(lib):
    assert _gb(_shape(T=0), ptrs=(None,) * 3) == E_OK
    assert _gb(_shape(o_lora_rank=96)) == E_SHAPE
    assert _gb(_shape(heads_per_group=3)) == E_MODE
    assert _gb(_shape(), ptrs=(0x1000, None, 0x1000)) == E_NULL
    assert _gb(_shape(), ptrs=(0x1000, 0x1000, BAD)) == E_ALIGN
    assert _gb(_shape(), layout=_native.Bf16Layout(4, 8)) == E_ALIGN
    # a group's activation rows beyond 4 GiB
    assert _gb(_shape(T=1 << 20), layout=_native.Bf16Layout(4096, 1024)) == E_SHAPE


def test_fused_bf16_workspace_and_validation(lib):
    shp = _shape(T=4, n_groups=2, heads_per_group=2, o_lora_rank=64)
    D = 2 * 512
    want = (4 * 2 * D * 2 + 255) // 256 * 256
    assert ap.oproj_fused_bf16_workspace_bytes(shp, 0) == want
    assert ap.oproj_fused_bf16_workspace_bytes(shp, 32) == want + (4 * 2 * 64 * 2 + 255) // 256 * 256
    f = lambda shape, ws_bytes=1 << 20, wo_b=None, hidden=0, o=0x1000, out=0x1000, ws=0x1000: _raw(
        "oproj_fused_bf16", ctypes.byref(shape._c()), o, 0x1000, 0x1000, 0x1000, wo_b, hidden, ws, ws_bytes,
        out, None)
    assert f(_shape(T=0), o=None, out=None, ws=None) == E_OK
    assert f(shp, o=None) == E_NULL
    assert f(shp, ws_bytes=16) == E_SHAPE
    assert f(shp, ws=BAD) == E_ALIGN
    assert f(shp, wo_b=0x1000, hidden=10) == E_SHAPE
    assert f(shp, wo_b=BAD, hidden=32) == E_ALIGN


def test_fused_workspace_and_validation(lib):
    shp = _shape(T=64, n_groups=16, heads_per_group=8, o_lora_rank=1024, max_pos=32768)
    n0 = ap.oproj_fused_workspace_bytes(shp, 0)
    D, KB = 4096, 32
    assert n0 == 64 * 16 * D + 64 * 16 * KB * 4
    n1 = ap.oproj_fused_workspace_bytes(shp, 7168)
    assert n1 == n0 + 64 * 16 * 1024 * 2
    assert ap.oproj_fused_workspace_bytes(_shape(o_lora_rank=10), 0) == 0
    P = 0x1000

    def fused(shape, ws_bytes, wo_b=None, hidden=0, mode=0, wblock=0, ws=P):
        return _raw("oproj_fused", ctypes.byref(shape._c()), mode, P, P, P, P, P, wblock, wo_b, hidden,
                    ws, ws_bytes, P, None)

    assert fused(shp, n0 - 1) == E_SHAPE
    assert fused(shp, n0, wo_b=P, hidden=7168) == E_SHAPE  # workspace lacks z
    assert fused(shp, n1, wo_b=P, hidden=7000) == E_SHAPE
    assert fused(shp, n0, ws=BAD) == E_ALIGN
    assert fused(shp, n0, mode=9) == E_MODE
    assert fused(_shape(T=0), 0) == E_OK


def test_fused_noalloc_validation(lib):
    """The no-allocation entry point refuses a call larger than its scratch
    array, and T == 0 / invalid shapes as oproj_fused does, all before any
    device work (so on a host without a GPU)."""
    P = 0x1000

    def noalloc(shape, wo_b=None, hidden=0, mode=0):
        return _raw("oproj_fused_noalloc", ctypes.byref(shape._c()), mode, P, P, P, P, P, 0, wo_b, hidden, P,
                    None)

    big = _shape(T=1024, n_groups=16, heads_per_group=8, o_lora_rank=1024, max_pos=32768)
    assert ap.oproj_fused_workspace_bytes(big, 0) > ap.OPROJ_NOALLOC_SCRATCH_BYTES
    assert noalloc(big) == 6
    assert "scratch" in ap.oproj_status_string(6)
    assert noalloc(_shape(o_lora_rank=10)) == E_SHAPE
    assert noalloc(_shape(T=0)) == E_OK
    assert noalloc(_shape(), mode=9) == E_MODE


def test_fused_decode_validation(lib):
    """The one-launch entry point's checks, all made before anything touches
    the device: shape limits, head geometry, pointers, workspace size."""
    shp = _shape(T=64, n_groups=16, heads_per_group=8, o_lora_rank=1024, max_pos=32768)
    n0 = ap.oproj_fused_workspace_bytes(shp, 0)
    P = 0x1000

    def dec(shape, ws_bytes=None, mode=0, wblock=0, ws=P, o=P, z=P):
        if ws_bytes is None:
            ws_bytes = ap.oproj_fused_decode_workspace_bytes(shape)
        return _raw("oproj_fused_decode", ctypes.byref(shape._c()), mode, o, P, P, P, P, wblock, ws, ws_bytes,
                    z, None)

    nd = ap.oproj_fused_decode_workspace_bytes(shp)
    assert nd == n0 + 16 * 128  # the groups' barrier words after the codes and scales
    assert dec(shp, ws_bytes=nd - 1) == E_SHAPE
    assert dec(_shape(T=0), 0, o=None, z=None, ws=None) == E_OK
    assert dec(_shape(T=65, n_groups=1, heads_per_group=8, o_lora_rank=64)) == E_SHAPE
    assert dec(_shape(T=8, n_groups=257, heads_per_group=8, o_lora_rank=64)) == E_SHAPE
    assert dec(_shape(T=8, n_groups=2, heads_per_group=1, o_lora_rank=64)) == E_MODE
    assert dec(shp, o=None) == E_NULL
    assert dec(shp, z=None) == E_NULL
    assert dec(shp, n0 - 1) == E_SHAPE
    assert dec(shp, ws=BAD) == E_ALIGN
    assert dec(shp, mode=3) == E_MODE
    assert dec(shp, mode=0, wblock=2) == E_MODE


def test_inv_rope_quant_f32_validation(lib):
    shp = _shape(T=4, n_groups=2, heads_per_group=2)
    P = 0x1000
    f = lambda shape, mode=0, o=P, c=P, s=P: _raw("oproj_inv_rope_quant_f32", ctypes.byref(shape._c()), mode,
                                                   o, P, P, c, s, None, None)
    assert f(_shape(T=0), o=None, c=None, s=None) == E_OK
    assert f(shp, o=None) == E_NULL
    assert f(shp, o=BAD) == E_ALIGN
    assert f(shp, mode=3) == E_MODE
    assert f(_shape(T=4, n_groups=2, heads_per_group=3)) == E_MODE


def test_fused_decode_unsupported_reasons(lib):
    """The eligibility query's static reasons (no device needed for these)."""
    q = ap.oproj_fused_decode_unsupported
    assert q(_shape(T=65, n_groups=2, heads_per_group=8, o_lora_rank=64)) == "more than 64 tokens"
    assert q(_shape(T=8, n_groups=257, heads_per_group=8, o_lora_rank=64)) == "more than 256 groups"
    assert "heads_per_group" in q(_shape(T=8, n_groups=2, heads_per_group=1, o_lora_rank=64))
    assert q(_shape(T=8, n_groups=2, heads_per_group=8, o_lora_rank=64), 3) == \
        "unsupported scale mode or weight block mode"
    assert q(_shape(T=8, n_groups=2, heads_per_group=8, o_lora_rank=64), 0, 2) == \
        "unsupported scale mode or weight block mode"
    assert q(_shape(T=8, n_groups=2, heads_per_group=8, o_lora_rank=10)) == "invalid shape"
    # a shape that passes the static checks reaches the device query (a string
    # either way: "no device to query" here, None or the CU limit on a GPU)
    r = q(_shape(T=8, n_groups=2, heads_per_group=8, o_lora_rank=64))
    assert r is None or isinstance(r, str)


def test_quantize_weight_validation(lib):
    f = lambda rows, K, blk=0, mode=0, w=0x1000, c=0x1000, s=0x1000: _raw(
        "oproj_quantize_weight", rows, K, blk, mode, w, c, s, None)
    assert f(0, 128) == E_OK
    assert f(4, 100) == E_SHAPE
    assert f(4, 128, blk=2) == E_MODE
    assert f(4, 128, mode=3) == E_MODE
    assert f(4, 512, blk=2, mode=0) == E_MODE  # UE8M0 weight scales need power-of-two scales
    assert f(4, 384, blk=2, mode=1) == E_SHAPE  # four blocks per word: K % 512
    assert f(4, 128, w=None) == E_NULL
    assert f(4, 128, s=0x1002) == E_ALIGN


def test_binding_raises_on_error_status(lib):
    with pytest.raises(ap.OprojError) as ei:
        ap.oproj_inv_rope_quant(_shape(heads_per_group=3), 0, 1, 1, 1, 1, 1, stream=0)
    assert ei.value.status == E_MODE


def test_torch_ops_checks_shapes_before_touching_a_device():
    import torch
    from attention_output_projection_amd import torch_ops as to
    o = torch.zeros((4, 6, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        to.fused_inv_rope_fp8_quant(o, torch.zeros(4, dtype=torch.int64), torch.zeros((16, 64)), 2, 2)


def test_product_and_oracle_share_no_code(lib):
    """The HIP path never routes through the oracle and the two share no code:
    no module of the package imports the oracle, no source of either side
    includes a file of the other, and the built library neither exports nor
    links any oracle symbol."""
    import ast
    import subprocess
    pkg = os.path.join(ROOT, "attention_output_projection_amd")
    orc = os.path.join(ROOT, "oracle")

    def sources(d, exts):
        for base, dirs, files in os.walk(d):
            dirs[:] = [x for x in dirs if not x.startswith(("_build", "__pycache__"))]
            for f in files:
                if f.endswith(exts):
                    yield os.path.join(base, f)

    for path in sources(pkg, (".py",)):
        for node in ast.walk(ast.parse(open(path).read())):
            names = [a.name for a in node.names] if isinstance(node, ast.Import) else (
                [node.module or ""] if isinstance(node, ast.ImportFrom) else [])
            assert not any(n.split(".")[0] == "oracle" for n in names), path
    for path in sources(pkg, (".hip", ".hpp", ".cpp", ".h")):
        for inc in re.findall(r'#include\s+"([^"]+)"', open(path).read()):
            assert "oracle" not in inc and "oproj_oracle" not in inc, (path, inc)
    for path in sources(orc, (".py", ".c", ".h")):
        text = open(path).read()
        assert "attention_output_projection_amd" not in text and "csrc" not in text, path
    assert not any(hasattr(lib, s) for s in ("orc_grouped_gemm", "orc_inv_rope_quant", "orc_irq_run"))
    dyn = subprocess.run(["readelf", "-d", ap.library_path()], capture_output=True, text=True).stdout
    assert "oracle" not in dyn


def test_missing_library_fails_loudly():
    """Without the built HIP library every call raises: there is no fallback."""
    import subprocess
    import sys
    code = ("import attention_output_projection_amd as ap, attention_output_projection_amd._native as n\n"
            "n._LIB_PATH = '/nonexistent/liboproj.so'\n"
            "ap.oproj_version()\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "RuntimeError" in r.stderr and "missing" in r.stderr
