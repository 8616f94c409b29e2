"""The one-launch decode kernel's publication order, checked in the gfx950
assembly built here (no GPU needed).

A workgroup of fused_decode_kernel quantises its share of the group into the
workspace and then announces it with one atomic add on the group's barrier
word; a reader on another XCD may take the codes straight from memory once
the barrier opens.  That is sound only if, in the generated code:
- every workspace store before the arrival is system-scope (sc0 sc1: written
  through to memory, not held in this XCD's L2),
- an `s_waitcnt vmcnt(0)` (the stores have completed) and an `s_barrier` (every
  wave's stores have) stand between the last such store and the arrival.
The test compiles gemm_fp8.hip with the library's own flags and checks this
in all eight instantiations of the kernel.

The same listings (and gemm_bf16.hip's) also show that no GEMM kernel spills
registers to scratch memory.
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    from attention_output_projection_amd import build as b

    if not os.path.exists(b.HIPCC):
        pytest.skip(f"{b.HIPCC} not available")
    out = tmp_path_factory.mktemp("asm") / "gemm_fp8.s"
    cmd = [b.HIPCC, *b.FLAGS, "--cuda-device-only", "-S", os.path.join(b.CSRC, "gemm_fp8.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=900)
    return out.read_text()


def _functions(text: str, pattern: str):
    for m in re.finditer(r"^(_Z\S*" + pattern + r"\S*):", text, re.M):
        end = text.index(".Lfunc_end", m.start())
        lines = [ln.strip() for ln in text[m.start():end].split("\n")
                 if ln.startswith("\t") and not ln.strip().startswith((".", ";"))]
        yield m.group(1), lines


def test_one_launch_stores_are_complete_and_system_scope_before_the_arrival(asm):
    fns = list(_functions(asm, "fused_decode_kernel"))
    assert len(fns) == 8, [n for n, _ in fns]  # MX x W1 x head chunk
    for name, lines in fns:
        arrive = next(i for i, ln in enumerate(lines) if ln.startswith("global_atomic_add_x2"))
        stores = [i for i in range(arrive) if lines[i].startswith("global_store")]
        assert stores, name
        for i in stores:
            assert "sc0 sc1" in lines[i], (name, lines[i])
        between = lines[stores[-1] + 1:arrive]
        assert "s_waitcnt vmcnt(0)" in between, name
        assert "s_barrier" in between, name
        # nothing else reaches memory between the last store and the arrival
        assert not any(ln.startswith(("global_store", "global_atomic", "buffer_store")) for ln in between), name


def test_plain_gemm_kernels_have_no_atomics(asm):
    # the plain decode and tile kernels synchronise through LDS only (both in
    # their four instantiations, MX x per-row weight scales, for each of
    # their two tile heights)
    for pattern, count in (("gemm_fp8_decode_kernel", 8), ("gemm_fp8_ptile_kernel", 8)):
        fns = list(_functions(asm, pattern))
        assert len(fns) == count, pattern
        for name, lines in fns:
            assert not any("atomic" in ln for ln in lines), name


def _resources(text: str):
    """(kernel symbol, VGPRs, private segment bytes) for every kernel in an
    assembly listing."""
    for m in re.finditer(r"^\s*\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.M | re.S):
        body = m.group(2)
        vgpr = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", body).group(1))
        scratch = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body).group(1))
        yield m.group(1), vgpr, scratch


def test_gemm_kernels_do_not_spill(asm):
    # every GEMM kernel keeps its accumulators, fragments and copy offsets in
    # registers: a spill to scratch memory inside the K loop costs more than
    # any schedule change gains (two waves per SIMD leave 256 VGPRs each)
    found = list(_resources(asm))
    assert len(found) >= 16, [k for k, _, _ in found]
    for name, vgpr, scratch in found:
        assert scratch == 0, (name, scratch)
        assert vgpr <= 256, (name, vgpr)


def test_bf16_gemm_kernels_do_not_spill(tmp_path):
    from attention_output_projection_amd import build as b

    if not os.path.exists(b.HIPCC):
        pytest.skip(f"{b.HIPCC} not available")
    out = tmp_path / "gemm_bf16.s"
    cmd = [b.HIPCC, *b.FLAGS, "--cuda-device-only", "-S", os.path.join(b.CSRC, "gemm_bf16.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=900)
    found = list(_resources(out.read_text()))
    assert len(found) >= 4, [k for k, _, _ in found]
    for name, vgpr, scratch in found:
        assert scratch == 0, (name, scratch)
