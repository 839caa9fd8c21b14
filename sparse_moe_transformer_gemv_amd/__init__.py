"""Flint routed-expert MoE layer for AMD Instinct MI355X (gfx950).

The compute is the HIP library libflint_moe.so (C ABI in include/flint_moe.h);
this package holds its kernels (csrc/), the build step and the ctypes binding.
"""
from .flint_moe import (  # noqa: F401
    EXPORTED, FLINT_BF16, FLINT_DEBUG_POISON_WORKSPACE, FLINT_F32, FLINT_FORCE_DECODE_PATH,
    FLINT_FORCE_PREFILL_PATH, FLINT_UNFUSED_DECODE, KERNEL_FORWARD, KERNEL_FUSED,
    check_forward_args,
    FLINT_NVFP4, KERNEL_COMBINE, KERNEL_EXPERT_DOWN, KERNEL_EXPERT_UP, KERNEL_ROUTE, KERNEL_SORT,
    DenseFFN, ExpertWeights, FlintError, MoELayer, flint_expert_weights, flint_moe_config,
    flint_moe_create, flint_moe_destroy, flint_moe_forward_noalloc, flint_rmsnorm_forward, load_library,
)
