"""Argument checks of the tensor-level calls, on the CPU: every bad argument
raises ValueError before anything is allocated or launched (dtypes, shapes,
contiguity, then the device: a host tensor is refused, since its pointer
would be dereferenced by a kernel)."""
from __future__ import annotations

import pytest
import torch

from attention_output_projection_amd import torch_ops as ops
from attention_output_projection_amd import _native as n

T, G, HPG, R = 4, 2, 2, 64
D, KB, H = HPG * 512, HPG * 4, G * HPG


def good():
    return dict(o=torch.zeros((T, H, 512), dtype=torch.bfloat16),
                positions=torch.zeros(T, dtype=torch.int64),
                cos_sin_cache=torch.zeros((16, 64), dtype=torch.float32),
                w_codes=torch.zeros((G * R, D), dtype=torch.uint8),
                w_scales=torch.zeros(((G * R + 127) // 128, KB), dtype=torch.float32))


def call_quant(a):
    return ops.fused_inv_rope_fp8_quant(a["o"], a["positions"], a["cos_sin_cache"], G, HPG)


def call_path(a, **kw):
    return ops.deep_gemm_fp8_o_proj(a["o"], a["positions"], a["cos_sin_cache"], a["w_codes"], a["w_scales"],
                                    a.get("wo_b"), n_groups=G, heads_per_group=HPG, o_lora_rank=R, **kw)


@pytest.mark.parametrize("field,value,match", [
    ("o", torch.zeros((T, H, 512), dtype=torch.float16), "o has dtype"),
    ("o", torch.zeros((T, H + 1, 512), dtype=torch.bfloat16), "o is"),
    ("positions", torch.zeros(T, dtype=torch.int32), "positions has dtype"),
    ("positions", torch.zeros(T + 1, dtype=torch.int64), "positions has shape"),
    ("positions", torch.zeros(2 * T, dtype=torch.int64)[::2], "positions must be contiguous"),
    ("cos_sin_cache", torch.zeros((16, 32), dtype=torch.float32), "cos_sin_cache has shape"),
    ("cos_sin_cache", torch.zeros((16, 64), dtype=torch.float64), "cos_sin_cache has dtype"),
])
def test_quant_bad_arguments(field, value, match):
    a = good()
    a[field] = value
    with pytest.raises(ValueError, match=match):
        call_quant(a)


def test_quant_host_tensors_refused():
    with pytest.raises(ValueError, match="must be on the GPU"):
        call_quant(good())


@pytest.mark.parametrize("field,value,match", [
    ("o", torch.zeros((T, H, 512), dtype=torch.float32), "bf16"),
    ("w_codes", torch.zeros((G * R, D), dtype=torch.int8), "w_codes has dtype"),
    ("w_codes", torch.zeros((G * R + 1, D), dtype=torch.uint8), "w_codes has shape"),
    ("w_codes", torch.zeros((D, G * R), dtype=torch.uint8).t(), "w_codes must be contiguous"),
    ("w_scales", torch.zeros((G * R, KB), dtype=torch.float32), "w_scales has shape"),
    ("w_scales", torch.zeros((1, KB), dtype=torch.float16), "w_scales has dtype"),
    ("wo_b", torch.zeros((256, G * R + 1), dtype=torch.bfloat16), "wo_b has shape"),
    ("wo_b", torch.zeros((256, G * R), dtype=torch.float32), "wo_b has dtype"),
])
def test_path_bad_arguments(field, value, match):
    a = good()
    a[field] = value
    with pytest.raises(ValueError, match=match):
        call_path(a)


def test_path_weight_block_modes():
    a = good()
    a["w_scales"] = torch.zeros((G * R, KB), dtype=torch.float32)  # 1x128 fp32 scales
    with pytest.raises(ValueError, match="must be on the GPU"):
        call_path(a, w_block=n.OPROJ_WBLOCK_1x128)
    a["w_scales"] = torch.zeros((G * R, KB // 4), dtype=torch.int32)  # packed UE8M0 words
    with pytest.raises(ValueError, match="power-of-two"):
        call_path(a, w_block=n.OPROJ_WBLOCK_1x128_UE8M0)
    with pytest.raises(ValueError, match="must be on the GPU"):
        call_path(a, w_block=n.OPROJ_WBLOCK_1x128_UE8M0, scale_mode=n.OPROJ_SCALE_POW2)
    with pytest.raises(ValueError, match="unknown w_block"):
        call_path(good(), w_block=7)


def test_grouped_wo_a_bad_arguments():
    codes = torch.zeros((T, G + 2, D), dtype=torch.uint8)
    scales = torch.zeros((T, G + 2, KB), dtype=torch.float32)
    a = good()
    kw = dict(n_groups=G, heads_per_group=HPG, o_lora_rank=R)
    with pytest.raises(ValueError, match="o_scale has dtype"):
        ops.grouped_wo_a(codes, scales.to(torch.int32), a["w_codes"], a["w_scales"], **kw)
    with pytest.raises(ValueError, match="o_fp8 has dtype"):
        ops.grouped_wo_a(codes.to(torch.int16), scales, a["w_codes"], a["w_scales"], **kw)
    with pytest.raises(ValueError, match=r"\[T, >=G, D\]"):
        ops.grouped_wo_a(codes[:, :1], scales, a["w_codes"], a["w_scales"], **kw)
    with pytest.raises(ValueError, match="must be on the GPU"):
        ops.grouped_wo_a(codes, scales, a["w_codes"], a["w_scales"], **kw)


def test_quantize_wo_a_bad_arguments():
    with pytest.raises(ValueError, match="w has dtype"):
        ops.quantize_wo_a(torch.zeros((128, 256), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must be on the GPU"):
        ops.quantize_wo_a(torch.zeros((128, 256), dtype=torch.float32))
