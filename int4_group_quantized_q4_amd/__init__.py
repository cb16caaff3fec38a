"""W4A16 matmuls over Q4_0 group-32 weights for AMD Instinct MI355X (gfx950).

The compute lives in libw4a16.so (HIP kernels behind the C ABI declared in
include/w4a16.h); this package is a thin ctypes binding with the same entry
points (see ``ops``).  Build the library with
``python -m int4_group_quantized_q4_amd.build``.
"""

from ._lib import (LIB_PATH, LibraryNotBuilt, W4Error, W4_OK, W4_ERR_ARG, W4_ERR_SHAPE, W4_ERR_WORKSPACE,
                   W4_ERR_HIP, W4_EPI_NONE, W4_EPI_GEGLU_TANH, W4_EPI_SWIGLU, W4_OUT_BF16, W4_OUT_F32,
                   W4_KERNEL_AUTO, W4_KERNEL_STREAM, W4_KERNEL_TILED, W4_TILED_MIN_ROWS, W4_GROUP_OFF_GRID, W4_GROUP_NONFINITE, W4_NOALLOC_SCRATCH_BYTES, SIGNATURES, lib, status_string)
from .ops import (q4_group_repack, q4_group_dequant_f32, q4_pack_codes, q4_pack_scales, w4a16_set_gemm_kernel, gemm_kernel, w4a16_linear_workspace, w4a16_linear, w4a16_moe_route_workspace,
                  w4a16_moe_route, w4a16_moe_topk, w4a16_moe_gmm_ids, w4a16_moe_gmm_logits, w4a16_moe_gmm_workspace, w4a16_moe_gmm, moe_gmm, w4a16_moe_combine, w4a16_moe_layer_workspace,
                  w4a16_moe_layer_plan, w4a16_moe_layer_sorted, w4a16_moe_layer, w4a16_moe_layer_noalloc, repack, dequant, pack_codes, pack_scales, linear, moe_route,
                  moe_layer, w8a8_quantize_rows, w8a8_moe_gmm, w8a8_moe_layer_plan, w8a8_moe_layer_workspace,
                  w8a8_moe_layer, fp8_moe_layer)
