"""Group-scaled INT8 linear layers (W8A8 G128, W4A16 g128) for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI in
``include/i8gs.h`` (``libi8gs.so``, built in-tree by ``_build.py``); this package
is the thin Python binding over it.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    I8GSError,
    I8GSValueError,
    KERNEL_AUTO,
    KERNEL_DECODE,
    KERNEL_TILED,
    OP_W4A16,
    OP_W8A8,
    OP_WEIGHT_ONLY,
    abi_version,
    attn_pv_int8,
    attn_qk_int8,
    gemm_w4a16_g128,
    gemm_w8a8_g128,
    gemm_w8a8_g128_ex,
    gemm_w8a8_g128_group_partials,
    gemm_w8a8_g128_noalloc,
    gemm_weight_only,
    gptq_quantize_rtn,
    gptq_quantize_rtn_group,
    gptq_unpack,
    kv_quant_int8_block128,
    last_error,
    load_library,
    noalloc_scratch_bytes,
    quant_act_per_token,
    rmsnorm_quant_per_token,
    workspace_bytes,
)
