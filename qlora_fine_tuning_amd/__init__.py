"""MI355X (gfx950) QLoRA linear layer and gated MLP, forward and backward.

The computation lives in the HIP library libqlora_mi355x.so (C ABI in
include/qlora.h); this package is its thin Python binding plus the seeded
synthetic-input generator (``inputs``). Importing the package does not load
the library; the first call does, and fails loudly if it was not built.
"""

__all__ = [
    "NF4Weight", "AbsmaxDQ", "absmax_dq_quantize", "absmax_dq_dequant", "nf4_double_quantize",
    "MlpWeights", "version", "nf4_levels", "gemm_split_count", "nf4_dequant", "nf4_quantize",
    "linear_workspace_bytes", "linear_fwd", "linear_bwd", "linear_fwd_noalloc",
    "linear_fwd_noalloc_max_bytes",
    "mlp_workspace_bytes", "mlp_fwd", "mlp_bwd", "trace_enable", "trace_read", "probe_mfma_peak",
    "linear16_workspace_bytes", "linear16_fwd", "linear16_bwd",
    "Mlp16Weights", "mlp16_workspace_bytes", "mlp16_fwd", "mlp16_bwd",
    "QkvWeights", "Qkv16Weights", "qkv_workspace_bytes", "qkv_fwd", "qkv_bwd", "qkv16_fwd",
    "qkv16_bwd", "rmsnorm_fwd", "rmsnorm_bwd", "rope_fwd", "rope_bwd", "cross_entropy_fwd",
    "cross_entropy_bwd", "cross_entropy_fused",
]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
