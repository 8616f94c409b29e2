"""MI355X (gfx950) O-projection front half: inverse RoPE -> 1x128 FP8 e4m3fn
quantisation -> grouped wo_a GEMM [-> dense wo_b GEMM], plus the unquantised
variant (bf16 inverse RoPE -> grouped bf16 wo_a GEMM).

The compute runs in the HIP library ``liboproj.so`` (C ABI in
``include/oproj.h``).  This package is the thin Python binding over it:
argument marshalling only, with PyTorch supplying device memory and streams.
Importing works without a GPU; calling an entry point needs the built
library (``python -m attention_output_projection_amd.build``) and raises if it
is missing.  There is no CPU fallback.
"""
from ._native import (  # noqa: F401
    OPROJ_NOALLOC_SCRATCH_BYTES,
    OPROJ_SCALE_E8M0,
    OPROJ_SCALE_FP32,
    OPROJ_SCALE_POW2,
    OPROJ_WBLOCK_1x128,
    OPROJ_WBLOCK_1x128_UE8M0,
    OPROJ_WBLOCK_128x128,
    ActLayout,
    Bf16Layout,
    OprojError,
    Shape,
    default_layout,
    library_path,
    load_library,
    oproj_dense_bf16_gemm,
    oproj_fused,
    oproj_fused_bf16,
    oproj_fused_decode,
    oproj_fused_decode_workspace_bytes,
    oproj_fused_decode_unsupported,
    oproj_fused_noalloc,
    oproj_fused_bf16_workspace_bytes,
    oproj_fused_workspace_bytes,
    oproj_grouped_wo_a,
    oproj_grouped_wo_a_bf16,
    oproj_inv_rope_bf16,
    oproj_inv_rope_quant,
    oproj_inv_rope_quant_f32,
    oproj_quantize_weight,
    oproj_status_string,
    oproj_version,
)
