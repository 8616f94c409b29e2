"""The tensor-level calls (torch_ops) against the raw entry points: the same
bytes, the page-described output views (o_fp8 [T, G, D] with strides
(D, T*D, 1)), the padded pre-quantised input through strided views, and the
whole path with and without wo_b and in one launch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_output_projection_amd as ap
import workloads as wl
from attention_output_projection_amd import torch_ops as to

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ap.load_library()
    yield
    torch.cuda.synchronize()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _inputs(name="decode"):
    w = wl.WORKLOADS[name]
    o = _dev(wl.attn_out(w).view(np.int16)).view(torch.bfloat16)
    return w, o, _dev(wl.positions(w)), _dev(wl.table(w))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_fused_inv_rope_fp8_quant_views_and_bytes(mode):
    w, o, pos, tab = _inputs()
    q, s = to.fused_inv_rope_fp8_quant(o, pos, tab, w.n_groups, w.heads_per_group, scale_mode=mode)
    assert q.dtype == torch.float8_e4m3fn and q.shape == (w.T, w.n_groups, w.D)
    assert q.stride() == (w.D, w.T * w.D, 1)
    nw = w.KB // 4 if mode == 2 else w.KB
    assert s.shape == (w.T, w.n_groups, nw) and s.stride() == (1, nw * w.T, w.T)
    shp = ap.Shape(T=w.T, n_groups=w.n_groups, heads_per_group=w.heads_per_group, max_pos=w.max_pos)
    codes = torch.empty((w.n_groups, w.T, w.D), dtype=torch.uint8, device=DEV)
    scales = torch.empty((w.n_groups, nw, w.T), dtype=torch.int32, device=DEV)
    ap.oproj_inv_rope_quant(shp, mode, o, pos, tab, codes, scales)
    torch.cuda.synchronize()
    assert torch.equal(q.transpose(0, 1).view(torch.uint8), codes)
    assert torch.equal(s.permute(1, 2, 0).contiguous().view(torch.int32), scales)


def test_fp32_input_takes_the_epilogue_producer():
    w, o, pos, tab = _inputs()
    q1, s1 = to.fused_inv_rope_fp8_quant(o.float(), pos, tab, w.n_groups, w.heads_per_group)
    q2, s2 = to.fused_inv_rope_fp8_quant(o, pos, tab, w.n_groups, w.heads_per_group)
    torch.cuda.synchronize()
    # bf16 values in fp32: bit-identical to the bf16 path
    assert torch.equal(q1.view(torch.uint8), q2.view(torch.uint8))
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))


@pytest.mark.parametrize("w_block,mode", [(0, 0), (1, 1), (2, 2)])
def test_quantize_and_whole_path_match_the_raw_calls(w_block, mode):
    w, o, pos, tab = _inputs()
    wq, wsc = to.quantize_wo_a(_dev(wl.wo_a_f32(w)), w_block, mode)
    shp = ap.Shape(T=w.T, n_groups=w.n_groups, heads_per_group=w.heads_per_group, o_lora_rank=w.o_lora_rank,
                   max_pos=w.max_pos)
    z = to.deep_gemm_fp8_o_proj(o, pos, tab, wq, wsc, n_groups=w.n_groups, heads_per_group=w.heads_per_group,
                                o_lora_rank=w.o_lora_rank, scale_mode=mode, w_block=w_block)
    z1 = to.deep_gemm_fp8_o_proj(o, pos, tab, wq, wsc, n_groups=w.n_groups, heads_per_group=w.heads_per_group,
                                 o_lora_rank=w.o_lora_rank, scale_mode=mode, w_block=w_block, one_launch=True)
    nb = ap.oproj_fused_workspace_bytes(shp, 0)
    zr = torch.empty_like(z)
    ap.oproj_fused(shp, mode, o, pos, tab, wq, wsc, w_block, None, 0,
                   torch.empty(nb, dtype=torch.uint8, device=DEV), nb, zr)
    torch.cuda.synchronize()
    assert z.dtype == torch.bfloat16 and z.shape == (w.T, w.n_groups, w.o_lora_rank)
    assert torch.equal(z.view(torch.int16), zr.view(torch.int16))
    assert torch.equal(z1.view(torch.int16), zr.view(torch.int16))


def test_whole_path_with_wo_b():
    w, o, pos, tab = _inputs()
    wq, wsc = to.quantize_wo_a(_dev(wl.wo_a_f32(w)))
    hidden = 256
    wob = _dev(wl.bf16_matrix(wl.seed_of(95, 1), hidden, w.n_groups * w.o_lora_rank, 0.02).view(np.int16))
    y = to.deep_gemm_fp8_o_proj(o, pos, tab, wq, wsc, wob.view(torch.bfloat16), n_groups=w.n_groups,
                                heads_per_group=w.heads_per_group, o_lora_rank=w.o_lora_rank)
    z = to.deep_gemm_fp8_o_proj(o, pos, tab, wq, wsc, n_groups=w.n_groups, heads_per_group=w.heads_per_group,
                                o_lora_rank=w.o_lora_rank)
    yr = torch.empty((w.T, hidden), dtype=torch.bfloat16, device=DEV)
    ap.oproj_dense_bf16_gemm(w.T, hidden, w.n_groups * w.o_lora_rank, z, wob, yr)
    torch.cuda.synchronize()
    assert y.shape == (w.T, hidden) and torch.equal(y.view(torch.int16), yr.view(torch.int16))


def test_grouped_wo_a_reads_only_the_live_groups_of_a_padded_view():
    """A pre-quantised [T, 10, D] input with NaN-coded padding groups: the
    padding never reaches z."""
    w, o, pos, tab = _inputs()
    G = 8
    Gp = 10
    q, s = to.fused_inv_rope_fp8_quant(o[:, : G * w.heads_per_group], pos, tab, G, w.heads_per_group)
    qp = torch.full((w.T, Gp, w.D), 0x7F, dtype=torch.uint8, device=DEV)
    sp = torch.full((w.T, Gp, w.KB), float("nan"), dtype=torch.float32, device=DEV)
    qp[:, :G] = q.view(torch.uint8)
    sp[:, :G] = s
    wq, wsc = to.quantize_wo_a(_dev(wl.wo_a_f32(w)[: G * w.o_lora_rank]))
    zp = to.grouped_wo_a(qp.view(torch.float8_e4m3fn), sp, wq, wsc, n_groups=G, heads_per_group=w.heads_per_group,
                         o_lora_rank=w.o_lora_rank)
    z = to.grouped_wo_a(q, s, wq, wsc, n_groups=G, heads_per_group=w.heads_per_group, o_lora_rank=w.o_lora_rank)
    torch.cuda.synchronize()
    assert not torch.isnan(zp.float()).any()
    assert torch.equal(zp.view(torch.int16), z.view(torch.int16))
