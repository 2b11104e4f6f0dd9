"""Helpers for the GPU parity tests: device inputs from the seeded generators,
host copies for the oracle, and error metrics.  The expected values always come
from ``oracle/`` applied to the exact bytes the device consumed."""

from __future__ import annotations

import concurrent.futures as cf
import json
import os
import sys

import numpy as np
import torch

import oracle
from synth import Workload, gen_expert_weights, gen_logits, gen_router, gen_x

ACT_TOL = {"f32": 1e-5, "bf16": 5e-3}
# 4-bit weights: the oracle decodes exactly the bytes the kernels read, and a
# decoded weight is exact in bf16 (MX-FP4: E2M1 x 2^s; NVFP4: E2M1 x E4M3,
# the fp32 matrix scale applied to fp32 sums), so these paths carry the bf16
# path's roundings (h and out to bf16, fp32 sums) and are held to its bound,
# tighter than the 2e-2 allowed for 4-bit layers.  Measured: 2.0-2.9e-3 over
# a whole output, at most 3.3e-3 for a single token.
MXFP4_TOL = 5e-3
# FP8 activations, per token: h's MX block scale and E4M3 codes are decided
# on fp32 sums on the device and on fp64 sums in the oracle.  When a block's
# largest |h| lies within that accumulation error of a power of two, the two
# sides choose scales a factor 2 apart and the element at amax moves by up to
# 1/8 (it saturates at 448 on the finer scale); a code at an E4M3 rounding
# tie flips by one step (1/16 to 1/8 of the element).  Both are outcomes of
# the same rule on values equal within rounding.  One such block among a
# token's 8 x f/32 blocks moves that token's output by up to ~3e-3 (measured:
# 5.0e-3 worst token of 562 at T=4096, 1.8e-3 over the whole output), so a
# single token is held to 1e-2 and the whole output to 5e-3.
FP8_TOKEN_TOL = 1e-2


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    import expert_ffn_layer_softmax_amd
    expert_ffn_layer_softmax_amd.load()  # raises if the library is missing


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


def token_rel_l2(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative L2 error of each token's output row ([T, d] -> [T])."""
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def record(case: str, **fields):
    """Append one parity measurement to $MOE_PARITY_LOG (JSON lines), if set."""
    path = os.environ.get("MOE_PARITY_LOG")
    if not path:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as fh:
        fh.write(json.dumps(dict(case=case, **fields)) + "\n")


def check_out(case: str, got: np.ndarray, ref: np.ndarray, tol: float, tokens=None,
              token_tol: float = None) -> float:
    """Layer output parity: the relative L2 error over the whole [T, d] output
    must be within `tol`, and that of every single token's row within
    `token_tol` (default `tol`).  Logs and records both; returns the global
    error."""
    token_tol = tol if token_tol is None else token_tol
    err = rel_l2(got, ref)
    per = token_rel_l2(got, ref)
    worst = float(per.max()) if per.size else 0.0
    wt = int(np.argmax(per)) if per.size else -1
    if tokens is not None and wt >= 0:
        wt = int(np.asarray(tokens)[wt])
    log(f"  {case}: rel_l2={err:.3e} worst token={worst:.3e} (token {wt}, {per.size} tokens) "
        f"tol={tol:.0e}/{token_tol:.0e}")
    record(case, rel_l2=err, worst_token=worst, worst_token_index=wt, tokens=int(per.size), tol=tol,
           token_tol=token_tol)
    assert err <= tol, f"{case}: relative L2 {err:.3e} > {tol:.0e}"
    assert worst <= token_tol, f"{case}: token {wt} relative L2 {worst:.3e} > {token_tol:.0e}"
    return err


class PrefetchGetter:
    """The oracle's expert getter with decoding done ahead, on host threads.

    ``oracle.layer`` asks for experts in ascending order (only those with
    routed rows); this decodes up to `window` of the next ones in parallel
    with what the oracle is computing.  The decode itself is the oracle's."""

    def __init__(self, get, experts, workers: int = 8, window: int = 12):
        self._get = get
        self._order = list(experts)
        self._pool = cf.ThreadPoolExecutor(workers)
        self._fut = {}
        self._next = 0
        self._window = window
        self._fill()

    def _fill(self):
        while self._next < len(self._order) and len(self._fut) < self._window:
            e = self._order[self._next]
            self._fut[e] = self._pool.submit(self._get, e)
            self._next += 1

    def __call__(self, e):
        fut = self._fut.pop(e, None)
        val = fut.result() if fut is not None else self._get(e)
        self._fill()
        return val

    def close(self):
        self._pool.shutdown(wait=True, cancel_futures=True)


def stratified_tokens(topk_idx: np.ndarray, E: int, bm: int = 128, extra: int = 8, seed: int = 7):
    """Tokens that own the rows at every edge of the grouped GEMM's row
    tiling: the first and last row of every expert's segment (so every
    expert's last, ragged m-tile) and the rows either side of each m-tile
    boundary inside a segment, plus `extra` random tokens.  Each sampled
    token's whole output row (all d columns, so every column-tile edge of the
    down projection) is compared."""
    T, k = topk_idx.shape
    _, offsets, sorted_src, _ = oracle.permute(topk_idx, E)
    rows = []
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        rows += [r0, r1 - 1]
        for b in range(r0 + bm, r1, bm):
            rows += [b - 1, b]
    toks = set((sorted_src[np.asarray(rows)] // k).tolist())
    rng = np.random.default_rng(seed)
    toks |= set(rng.choice(T, min(extra, T), replace=False).tolist())
    return np.array(sorted(toks))


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
