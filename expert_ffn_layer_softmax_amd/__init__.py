"""MI355X (gfx950) Mixture-of-Experts layer library: Python binding.

Thin ctypes marshalling over the C ABI in ``include/moe.h``; every step of
the layer runs in the HIP kernels of ``libmoe_mi355x.so``.  PyTorch supplies
device memory and the current HIP stream only.  The library is opened on
first use; that first call raises ImportError if it has not been built
(``python -m expert_ffn_layer_softmax_amd.build``).  There is no CPU fallback.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    MOE_DTYPE_BF16,
    MOE_DTYPE_F32,
    MOE_DTYPE_MXFP4,
    MOE_DTYPE_NVFP4,
    MOE_FLAG_EXPERT_NORM,
    MOE_FLAG_FP8_ACTIVATIONS,
    MoeError,
    lib,
    load,
    moe_combine,
    moe_debug_check,
    moe_expert_ffn,
    moe_layer_forward,
    moe_layer_forward_noalloc,
    moe_permute,
    moe_quantize_mxfp8,
    moe_route,
    moe_status_string,
    moe_timing_names,
    moe_timing_query,
    moe_timing_start,
    moe_timing_stop,
    moe_workspace_size,
)
