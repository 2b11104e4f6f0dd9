"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the layer itself: it only draws random
activations, weights and router logits, and encodes weights into the storage
formats the layer reads (bf16 by torch's round-to-nearest-even cast, MX-FP4 by
the OCP MX quantisation rule, NVFP4 by its two-level scale recipe).  The
oracle decodes those bytes with its own code; the HIP library decodes them with
its own code.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    gen_expert_weights,
    gen_logits,
    gen_router,
    gen_x,
    quantize_mxfp4,
    quantize_nvfp4,
)
