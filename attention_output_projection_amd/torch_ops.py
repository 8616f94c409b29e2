"""Tensor-level calls in the shape of the pages' functions, over the C ABI.

vLLM API page "vllm.models.deepseek_v4.common.ops.fused_inv_rope_fp8_quant"
(fused_inv_rope_fp8_quant: returns o_fp8 [T, G, D] with strides (D, T*D, 1)
and the MN-major scales) and vLLM API page
"vllm.models.deepseek_v4.nvidia.ops.o_proj" (deep_gemm_fp8_o_proj: inverse
RoPE + grouped wo_a + wo_b over the flattened z; a pre-quantised input is
sliced to its live groups).

Argument marshalling only: these functions allocate the outputs (and the
workspace) with torch.empty on the input's device, read strides off the
tensors, and call one entry point of liboproj.so; every arithmetic step runs
in the HIP kernels.  Differences from the pages: wo_a is passed as its FP8
codes and scales (as oproj_quantize_weight writes them), wo_b as a bf16
[hidden, G*R] tensor rather than a module, and the scale recipe as a scale
mode (OPROJ_SCALE_FP32, OPROJ_SCALE_POW2 or OPROJ_SCALE_E8M0, the last being
the packed UE8M0 words) instead of (einsum_recipe, tma_aligned_scales); scales
are not padded to a TMA-aligned token count.
"""
from __future__ import annotations

import torch

from . import _native as n


def _scale_dtype(scale_mode: int):
    return torch.int32 if scale_mode == n.OPROJ_SCALE_E8M0 else torch.float32


_FP8 = (torch.uint8, torch.float8_e4m3fn)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _tensor(name: str, t, dtypes, shape=None, contiguous: bool = True):
    """dtype, shape and contiguity of one argument (None entries of `shape`
    match any size); raises ValueError naming the argument."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.dtype in dtypes, f"{name} has dtype {t.dtype}; expected one of {list(dtypes)}")
    if shape is not None:
        ok = t.dim() == len(shape) and all(s is None or t.shape[i] == s for i, s in enumerate(shape))
        _need(ok, f"{name} has shape {list(t.shape)}; expected {['*' if s is None else s for s in shape]}")
    if contiguous:
        _need(t.is_contiguous(), f"{name} must be contiguous")


def _same_gpu(**tensors):
    """Every tensor on one GPU: the kernels receive raw device pointers, and a
    host pointer or another device's memory would be dereferenced on the GPU."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        _need(t.is_cuda, f"{name} is on {t.device}; every tensor must be on the GPU")
        dev = t.device if dev is None else dev
        _need(t.device == dev, f"{name} is on {t.device}, other arguments on {dev}")


def _weights(w_codes, w_scales, rows: int, D: int, w_block: int, scale_mode: int):
    KB = D // 128
    _tensor("w_codes", w_codes, _FP8, (rows, D))
    if w_block == n.OPROJ_WBLOCK_1x128_UE8M0:
        _need(scale_mode != n.OPROJ_SCALE_FP32, "packed UE8M0 weight scales need a power-of-two scale mode")
        _tensor("w_scales", w_scales, (torch.int32, torch.uint32), (rows, KB // 4))
    elif w_block == n.OPROJ_WBLOCK_1x128:
        _tensor("w_scales", w_scales, (torch.float32,), (rows, KB))
    elif w_block == n.OPROJ_WBLOCK_128x128:
        _tensor("w_scales", w_scales, (torch.float32,), ((rows + 127) // 128, KB))
    else:
        raise ValueError(f"unknown w_block {w_block}")


def _attn_inputs(o, positions, cos_sin_cache, T: int, H: int, hd: int, rope_dim: int):
    _tensor("o", o, (torch.bfloat16, torch.float32), (T, H, hd), contiguous=False)
    _tensor("positions", positions, (torch.int64,), (T,))
    _tensor("cos_sin_cache", cos_sin_cache, (torch.float32,), (None, rope_dim))


def fused_inv_rope_fp8_quant(o: torch.Tensor, positions: torch.Tensor, cos_sin_cache: torch.Tensor,
                             n_groups: int, heads_per_group: int, nope_dim: int = 448, rope_dim: int = 64,
                             quant_group_size: int = 128, scale_mode: int = n.OPROJ_SCALE_FP32):
    """a1 + a2 on bf16 o [T, H, 512] (fp32 o: the attention-epilogue producer).

    Returns (o_fp8, o_scale): o_fp8 is [T, G, D] float8_e4m3fn with strides
    (D, T*D, 1) over group-major storage; o_scale is [T, G, KB] float32 with
    strides (1, KB*T, T) over [G, KB, T] storage, or [T, G, KB/4] int32 packed
    UE8M0 words in OPROJ_SCALE_E8M0 mode."""
    _need(isinstance(o, torch.Tensor) and o.dim() == 3, "o must be a [T, H, head_dim] tensor")
    T, H, hd = o.shape
    if H != n_groups * heads_per_group or hd != nope_dim + rope_dim:
        raise ValueError(f"o is [{T}, {H}, {hd}]: expected [T, {n_groups * heads_per_group}, {nope_dim + rope_dim}]")
    _attn_inputs(o, positions, cos_sin_cache, T, H, hd, rope_dim)
    _need(scale_mode in (n.OPROJ_SCALE_FP32, n.OPROJ_SCALE_POW2, n.OPROJ_SCALE_E8M0),
          f"unknown scale_mode {scale_mode}")
    _same_gpu(o=o, positions=positions, cos_sin_cache=cos_sin_cache)
    shape = n.Shape(T=T, n_groups=n_groups, heads_per_group=heads_per_group, max_pos=cos_sin_cache.shape[0],
                    nope_dim=nope_dim, rope_dim=rope_dim, quant_block=quant_group_size)
    nw = shape.KB // 4 if scale_mode == n.OPROJ_SCALE_E8M0 else shape.KB
    codes = torch.empty((n_groups, T, shape.D), dtype=torch.float8_e4m3fn, device=o.device)
    scales = torch.empty((n_groups, nw, T), dtype=_scale_dtype(scale_mode), device=o.device)
    call = n.oproj_inv_rope_quant_f32 if o.dtype == torch.float32 else n.oproj_inv_rope_quant
    call(shape, scale_mode, o.contiguous(), positions, cos_sin_cache, codes, scales)
    return codes.transpose(0, 1), scales.permute(2, 0, 1)


def quantize_wo_a(w: torch.Tensor, w_block: int = n.OPROJ_WBLOCK_128x128,
                  scale_mode: int = n.OPROJ_SCALE_FP32):
    """Offline: fp32 wo_a [G*R, D] -> (FP8 codes [G*R, D], scales).  Scales are
    float32 [ceil(rows/128), D/128] (128x128 blocks) or [rows, D/128] (1x128),
    or int32 [rows, D/512] packed UE8M0 words (OPROJ_WBLOCK_1x128_UE8M0)."""
    _need(isinstance(w, torch.Tensor) and w.dim() == 2, "w must be a [rows, K] tensor")
    rows, K = w.shape
    _tensor("w", w, (torch.float32,), (rows, K), contiguous=False)
    _same_gpu(w=w)
    codes = torch.empty((rows, K), dtype=torch.float8_e4m3fn, device=w.device)
    if w_block == n.OPROJ_WBLOCK_1x128_UE8M0:
        scales = torch.empty((rows, K // 512), dtype=torch.int32, device=w.device)
    elif w_block == n.OPROJ_WBLOCK_1x128:
        scales = torch.empty((rows, K // 128), dtype=torch.float32, device=w.device)
    else:
        scales = torch.empty(((rows + 127) // 128, K // 128), dtype=torch.float32, device=w.device)
    n.oproj_quantize_weight(rows, K, w_block, scale_mode, w.contiguous(), codes, scales)
    return codes, scales


def grouped_wo_a(o_fp8: torch.Tensor, o_scale: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, *,
                 n_groups: int, heads_per_group: int, o_lora_rank: int, scale_mode: int = n.OPROJ_SCALE_FP32,
                 w_block: int = n.OPROJ_WBLOCK_128x128) -> torch.Tensor:
    """a3 on FP8 activations given as [T, >=G, D] codes and [T, >=G, KB] scales
    views of any strides (only groups < n_groups are read: a padded
    pre-quantised input is passed as it is).  Returns z bf16 [T, G, R]."""
    _need(isinstance(o_fp8, torch.Tensor) and o_fp8.dim() == 3, "o_fp8 must be a [T, >=G, D] tensor")
    T = o_fp8.shape[0]
    shape = n.Shape(T=T, n_groups=n_groups, heads_per_group=heads_per_group, o_lora_rank=o_lora_rank)
    _tensor("o_fp8", o_fp8, _FP8, (T, None, shape.D), contiguous=False)
    if o_fp8.shape[1] < n_groups or o_fp8.stride(2) != 1:
        raise ValueError("o_fp8 must be [T, >=G, D] with unit stride along D")
    nw = shape.KB // 4 if scale_mode == n.OPROJ_SCALE_E8M0 else shape.KB
    sdt = (torch.int32, torch.uint32) if scale_mode == n.OPROJ_SCALE_E8M0 else (torch.float32,)
    _tensor("o_scale", o_scale, sdt, (T, None, nw), contiguous=False)
    _need(o_scale.shape[1] >= n_groups, "o_scale must be [T, >=G, KB]")
    _weights(w_codes, w_scales, n_groups * o_lora_rank, shape.D, w_block, scale_mode)
    _same_gpu(o_fp8=o_fp8, o_scale=o_scale, w_codes=w_codes, w_scales=w_scales)
    lay = n.ActLayout(o_fp8.stride(0), o_fp8.stride(1), o_scale.stride(0), o_scale.stride(1), o_scale.stride(2))
    z = torch.empty((T, n_groups, o_lora_rank), dtype=torch.bfloat16, device=o_fp8.device)
    n.oproj_grouped_wo_a(shape, scale_mode, o_fp8, o_scale, lay, w_codes, w_scales, w_block, z)
    return z


def deep_gemm_fp8_o_proj(o: torch.Tensor, positions: torch.Tensor, cos_sin_cache: torch.Tensor,
                         w_codes: torch.Tensor, w_scales: torch.Tensor, wo_b: torch.Tensor | None = None, *,
                         n_groups: int, heads_per_group: int, o_lora_rank: int,
                         scale_mode: int = n.OPROJ_SCALE_FP32, w_block: int = n.OPROJ_WBLOCK_128x128,
                         one_launch: bool = False) -> torch.Tensor:
    """The whole path on bf16 o [T, H, 512]: y = wo_b(z.flatten(1)) bf16
    [T, hidden] when wo_b ([hidden, G*R] bf16) is given, else z bf16 [T, G, R].
    one_launch (experimental, off by default: slower than the two launches on
    MI355X) takes oproj_fused_decode (steps a1-a3 in one kernel) when it
    supports the shape and wo_b is None, and oproj_fused otherwise."""
    _need(isinstance(o, torch.Tensor) and o.dim() == 3, "o must be a [T, H, 512] tensor")
    T = o.shape[0]
    _attn_inputs(o, positions, cos_sin_cache, T, n_groups * heads_per_group, 512, 64)
    _need(o.dtype == torch.bfloat16, f"o has dtype {o.dtype}; the whole path takes bf16 attention output")
    shape = n.Shape(T=T, n_groups=n_groups, heads_per_group=heads_per_group, o_lora_rank=o_lora_rank,
                    max_pos=cos_sin_cache.shape[0])
    _weights(w_codes, w_scales, n_groups * o_lora_rank, shape.D, w_block, scale_mode)
    if wo_b is not None:
        _tensor("wo_b", wo_b, (torch.bfloat16,), (None, n_groups * o_lora_rank), contiguous=False)
    _same_gpu(o=o, positions=positions, cos_sin_cache=cos_sin_cache, w_codes=w_codes, w_scales=w_scales,
              wo_b=wo_b)
    hidden = 0 if wo_b is None else wo_b.shape[0]
    ws_bytes = n.oproj_fused_workspace_bytes(shape, hidden)
    o = o.contiguous()
    if wo_b is None:
        z = torch.empty((T, n_groups, o_lora_rank), dtype=torch.bfloat16, device=o.device)
        if one_launch and n.oproj_fused_decode_unsupported(shape, scale_mode, w_block) is None:
            # a fresh workspace: its barrier words start at zero
            dbytes = n.oproj_fused_decode_workspace_bytes(shape)
            ws = torch.zeros(dbytes, dtype=torch.uint8, device=o.device)
            n.oproj_fused_decode(shape, scale_mode, o, positions, cos_sin_cache, w_codes, w_scales, w_block,
                                 ws, dbytes, z)
        else:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=o.device)
            n.oproj_fused(shape, scale_mode, o, positions, cos_sin_cache, w_codes, w_scales, w_block, None, 0,
                          ws, ws_bytes, z)
        return z
    y = torch.empty((T, hidden), dtype=torch.bfloat16, device=o.device)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=o.device)
    n.oproj_fused(shape, scale_mode, o, positions, cos_sin_cache, w_codes, w_scales, w_block, wo_b.contiguous(),
                  hidden, ws, ws_bytes, y)
    return y
