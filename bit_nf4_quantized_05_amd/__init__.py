"""QLoRA NF4 linear layer for MI355X (gfx950): NF4 + double quantisation,
double dequantisation, fused forward, input gradient and adapter gradients, as
hand-written HIP kernels behind the C ABI in include/qlora_nf4.h."""
from ._lib import (  # noqa: F401
    DQ_CODES,
    NF4Weight,
    QLoRAError,
    alloc_weight,
    codebook,
    double_dequant,
    linear_bwd_x,
    linear_fwd,
    linear_workspace_bytes,
    lora_grads,
    lora_grads_workspace_bytes,
    nf4_sizes,
    profile_enable,
    profile_read,
    quantize,
    quantize_workspace_bytes,
    version,
)
