"""Weight-quantized decode GEMV / skinny GEMM for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libqgemv.so`` (C ABI: include/qgemv.h);
this package is its thin binding plus seeded synthetic inputs (``synth``) and
host-side byte/roofline accounting (``roofline``).
"""
from ._lib import (  # noqa: F401
    EXPORTS, FMT_MXFP4_G32, FMT_Q4_ASYM_G64, FMT_Q8_SYM_G32, FMT_Q8_ROW, OUT_BF16, OUT_F32, OUT_I32_GROUPS,
    KERNEL_AUTO, KERNEL_VALU, KERNEL_MFMA,
    QGError, affine_format, hadamard32_quant_run, moe_expert_gemv_run, moe_workspace_bytes, packed_bytes,
    moe_expert_skinny_run, moe_skinny_workspace_bytes, moe_expert_gemv_run_noalloc,
    MOE_NOALLOC_SCRATCH_BYTES, QG_ESIZE,
    qgemm_skinny_run, qgemv_pack, qgemv_run, raw, status_string, qg_batch_plan_build,
    qg_batch_run, qg_batch_worklist_bytes, qg_plain_read, GemvDesc, BatchPlan, Plan,
)

__version__ = "0.1.0"
