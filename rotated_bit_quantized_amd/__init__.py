"""Rotated low-bit linear layer for AMD MI355X (gfx950).

The compute path is the HIP library ``liboq.so`` built from ``csrc/``; this
package only exposes its C entry points (``include/oq.h``) to Python.
Importing fails loudly when the library has not been built.
"""
from ._binding import (  # noqa: F401
    EXPORTED, LIB_PATH, OQError, Rotation,
    OQ_A4, OQ_A6, OQ_A8, OQ_MXFP4, OQ_W4, OQ_W_MXFP4,
    OQ_OP_GEMM_LM, OQ_OP_GEMM_W4A4, OQ_OP_GEMM_W4A8, OQ_OP_LINEAR,
    OQ_ROT_DENSE32, OQ_ROT_KRON, OQ_ROT_RPBH, OQ_SCALE_PCTL, OQ_TILED,
    OQ_ERR_ALIGNMENT, OQ_ERR_HIP, OQ_ERR_INVALID_ARG, OQ_ERR_UNSUPPORTED, OQ_ERR_WORKSPACE,
    lib, oq_center, oq_gemm_w4a4, oq_gemm_w4a8, oq_linear_fused, oq_quant_act, oq_quant_weight,
    oq_rotate, oq_workspace_bytes, oq_tiled_bytes, oq_prepack_w4, oq_tiled_mx_bytes, oq_prepack_mx,
    oq_lloyd_max_levels, oq_lloyd_max_tables, oq_tiled_f16_bytes, oq_quant_act_lm, oq_prepack_w16, oq_gemm_lm,
    oq_quant_weight_asym, oq_prepack_w4_asym, oq_quant_act_gsum, oq_gemm_w4a4_asym, oq_kron_plan,
    oq_linear_fused_noalloc, OQ_NOALLOC_SCRATCH_BYTES,
    oq_probe_mfma, OQ_PROBE_FP6, OQ_PROBE_FP4, OQ_PROBE_FP8, OQ_PROBE_I8, OQ_PROBE_BF16, OQ_PROBE_F16,
    OQ_PROBE_FP6_UPDATE,
)
