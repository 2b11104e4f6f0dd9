"""CPU oracle for the forward pass of one Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code with the HIP library.
"""

from .moe_oracle import (  # noqa: F401
    E2M1_VALUES,
    EXPERT_NORM_EPS,
    combine,
    decode_bf16,
    decode_e4m3,
    decode_e8m0,
    decode_mxfp4,
    decode_nvfp4,
    dense_layer,
    expert_ffn,
    layer,
    permute,
    route,
    quantize_mxfp8,
    round_e4m3,
    router_logits,
    swiglu_expert,
)
