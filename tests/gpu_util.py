"""Helpers for the GPU parity tests: device inputs from the seeded generators,
host copies for the oracle, and error metrics.  The expected values always come
from ``oracle/`` applied to the exact bytes the device consumed."""

from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
from synth import Workload, gen_expert_weights, gen_logits, gen_router, gen_x

ACT_TOL = {"f32": 1e-5, "bf16": 5e-3}
MXFP4_TOL = 2e-2


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    import expert_ffn_layer_softmax_amd  # noqa: F401  (raises if the library is missing)


def to_host_act(t: torch.Tensor) -> np.ndarray:
    """Device activations/weights (fp32 or bf16) -> fp64 numpy, exactly."""
    if t.dtype == torch.bfloat16:
        return oracle.decode_bf16(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def expert_getter(w: dict, wfmt: str):
    """Oracle-side expert decoder over device weights (one D2H copy per call)."""
    def get(e):
        if wfmt == "nvfp4":
            return tuple(oracle.decode_nvfp4(w["w_" + n][e].cpu().numpy(),
                                             w["s_" + n][e].view(torch.uint8).cpu().numpy(),
                                             float(w["t_" + n][e]))
                         for n in ("gate", "up", "down"))
        if wfmt == "mxfp4":
            return tuple(oracle.decode_mxfp4(w["w_" + n][e].cpu().numpy(), w["s_" + n][e].cpu().numpy())
                         for n in ("gate", "up", "down"))
        return tuple(to_host_act(w["w_" + n][e]) for n in ("gate", "up", "down"))
    return get


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm((got - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    return float(num / den) if den > 0 else float(num)


def make_inputs(wl: Workload, device="cuda", weights=None, logit_set=0):
    x = gen_x(wl.T, wl.d, wl.act, wl.seed, device, std=wl.x_std)
    w = weights if weights is not None else gen_expert_weights(wl, device)
    w_r = gen_router(wl.E, wl.d, wl.act, wl.seed, device) if wl.router else None
    logits = None
    if not wl.router:
        logits = gen_logits(wl.T, wl.E, wl.seed, device, sets=max(wl.logit_sets, logit_set + 1),
                            bias_std=wl.bias_std)[logit_set].contiguous()
    return x, w, w_r, logits


def check_routing(res, logits_host, k, E):
    """Bit-exact routing given the device's own logits."""
    idx, w = oracle.route(logits_host, k)
    got_idx = res["topk_idx"].cpu().numpy()
    assert np.array_equal(got_idx, idx), "top-k indices differ from the oracle"
    got_w = res["topk_w"].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got_w, w, rtol=1e-5, atol=1e-7)
    return idx, w


def run_layer_and_oracle(wl: Workload, x, w, w_r, logits, k=None, sample=None, fp8=False):
    """Run moe_layer_forward on the device and the oracle on the same bytes.
    ``sample``: token indices to check (the layer is per-token independent).
    ``fp8``: FP8-activation mode on both sides (the oracle quantises x and h
    to MXFP8 with its own code)."""
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    k = wl.k if k is None else k
    res = moe_layer_forward(x, w, k, logits=logits, w_router=w_r, fp8=fp8)
    torch.cuda.synchronize()
    lg = res["logits"].cpu().numpy()
    xh = to_host_act(x)
    if w_r is not None:
        ref_logits = oracle.router_logits(xh, to_host_act(w_r))
        assert rel_l2(lg.astype(np.float64), ref_logits) <= 1e-5
    check_routing(res, lg, k, wl.E)
    S = np.arange(wl.T) if sample is None else np.asarray(sample)
    ref = oracle.layer(xh[S], lg[S], k, expert_getter(w, wl.wfmt), E=wl.E,
                       act_quant=oracle.quantize_mxfp8 if fp8 else None)
    got = to_host_act(res["out"])[S]
    return got, ref, res
