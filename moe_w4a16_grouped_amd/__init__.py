"""MI355X-native MoE W4A16 layer: Python binding of libmoe_w4a16 (HIP, gfx950).

The package holds the HIP sources (``csrc/``), their build script (``build.py``) and a ctypes binding
(``_lib.py``) whose functions carry the names of the C entry points declared in
``include/moe_w4a16.h``.
"""
from ._lib import (MOE_ACT_ROWS, MOE_ACT_TILED, MOE_EPI_NONE, MOE_EPI_SILU_MUL, MOE_LAYOUT_CANONICAL, MOE_LAYOUT_PACKED, MOE_OUT_BF16,
                   MOE_OUT_F32, MOE_OUT_F16E, MOE_OUT_H16, EXPORTED, LIB_PATH, MoEError,
                   load, moe_align, moe_align_workspace_bytes, moe_combine, moe_dense_ffn_w4a16,
                   moe_dense_ffn_workspace_bytes, moe_ffn_block_forward, moe_ffn_block_m,
                   moe_ffn_block_workspace_bytes, moe_ffn_forward, moe_ffn_workspace_bytes, moe_grouped_gemm_w4a16,
                   moe_max_tiles, moe_route_topk, moe_router_logits, moe_w4_prepack, moe_mx_quantize, moe_mx_quantize_tiles, moe_mx_prepack,
                   moe_grouped_gemm_mxfp4, moe_ffn_mxfp4_block_m, moe_ffn_mxfp4_workspace_bytes,
                   moe_ffn_forward_mxfp4, MOE_IN_BF16, MOE_IN_F32, MOE_OUT_F8, moe_f8_quantize, moe_grouped_gemm_f8,
                   moe_ffn_f8_block_m, moe_ffn_f8_workspace_bytes, moe_ffn_forward_f8, moe_mx8_quantize, moe_mx8_quantize_tiles,
                   moe_grouped_gemm_w4a8, moe_ffn_w4a8_block_m, moe_ffn_w4a8_workspace_bytes, moe_ffn_forward_w4a8,
                   moe_ffn_noalloc_scratch_bytes, moe_ffn_forward_noalloc,
                   moe_x_to_f16, moe_grouped_gemm_w4f16)

__all__ = ["MOE_ACT_ROWS", "MOE_ACT_TILED", "MOE_EPI_NONE", "MOE_EPI_SILU_MUL", "MOE_LAYOUT_CANONICAL", "MOE_LAYOUT_PACKED", "MOE_OUT_BF16",
           "MOE_OUT_F32", "MOE_OUT_F16E", "MOE_OUT_H16", "EXPORTED", "LIB_PATH", "MoEError", "load", "moe_align", "moe_align_workspace_bytes",
           "moe_combine", "moe_dense_ffn_w4a16", "moe_dense_ffn_workspace_bytes", "moe_ffn_block_forward",
           "moe_ffn_block_m", "moe_ffn_block_workspace_bytes", "moe_ffn_forward", "moe_ffn_workspace_bytes",
           "moe_grouped_gemm_w4a16", "moe_max_tiles", "moe_route_topk", "moe_router_logits", "moe_w4_prepack",
           "moe_mx_quantize", "moe_mx_quantize_tiles", "moe_mx_prepack", "moe_grouped_gemm_mxfp4", "moe_ffn_mxfp4_block_m", "moe_ffn_mxfp4_workspace_bytes",
           "moe_ffn_forward_mxfp4", "MOE_IN_BF16", "MOE_IN_F32", "MOE_OUT_F8", "moe_f8_quantize", "moe_grouped_gemm_f8",
           "moe_ffn_f8_block_m", "moe_ffn_f8_workspace_bytes", "moe_ffn_forward_f8", "moe_mx8_quantize", "moe_mx8_quantize_tiles",
           "moe_grouped_gemm_w4a8", "moe_ffn_w4a8_block_m", "moe_ffn_w4a8_workspace_bytes", "moe_ffn_forward_w4a8",
           "moe_ffn_noalloc_scratch_bytes", "moe_ffn_forward_noalloc", "moe_x_to_f16",
           "moe_grouped_gemm_w4f16"]
