"""K-grouped weight-gradient GEMM for MoE training on AMD MI355X (gfx950).

The computation lives in libkgwgrad.so (HIP kernels behind the C ABI declared in
include/kgwgrad.h); `_binding` marshals torch device tensors into it, and
`inputs` makes seeded synthetic inputs.
"""
from ._binding import (KG_BF16, KG_E4M3_F32SCALE, KG_E4M3_UE8M0, KG_ERR_ALIAS,  # noqa: F401
                       KG_ERR_ALIGN, KG_ERR_DTYPE, KG_ERR_GRAN, KG_ERR_HIP, KG_ERR_KSUM,
                       KG_ERR_NULL, KG_ERR_SCALE_RANGE, KG_ERR_SCALE_ROWS, KG_ERR_SHAPE, KG_ERR_SPLIT, KG_ERR_UNSUPPORTED,
                       KG_FLAG_D_BF16, KG_FLAG_FP8_MFMA, KG_OK, KgError, kg_debug_offsets, kg_max_groups,
                       kg_status, kg_wgrad, kg_wgrad_raw, kg_wgrad_workspace_bytes,
                       kg_wgrad_workspace_flag_bytes,
                       kg_wgrad_ws_raw, kg_wgrad_noalloc_raw, new_workspace, scale_rows_of, KG_SRC_BF16, KG_SRC_E4M3_1X128,
                       kg_requant, kg_requant_raw, kg_dgrad, kg_dgrad_raw,
                       kg_wgrad_nt, kg_wgrad_nt_raw)
