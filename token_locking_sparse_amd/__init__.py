"""SureLock decoding step for masked diffusion LMs, native on AMD MI355X (gfx950).

The computation lives in libsurelock.so (hand-written HIP kernels behind the C
ABI of include/surelock.h); this package only loads it and marshals arguments.
"""
from .surelock import (SL_BF16, SL_F32, SureLockError, PinnedInt, lib, sl_attn_active,  # noqa: F401
                       sl_attn_workspace_size, sl_cache_scatter, sl_compact, sl_kl_lock, sl_kl_lock_noalloc,
                       sl_kl_lock_workspace_size, sl_rope_table, sl_step, sl_step_workspace_size,
                       sl_step_workspace_min, sl_gemm, sl_gemm_plan, sl_gemm_clocked, sl_peak_mfma,
                       sl_peak_mfma_operands, sl_peak_stream, sl_peak_gemm_loop, SL_EPI_QKV_ROPE, SL_EPI_RESIDUAL,
                       SL_EPI_SWIGLU, SL_EPI_LOGITS)
from .runtime import CapturedLoop, DeviceModel, DeviceState  # noqa: F401
