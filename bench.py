"""Throughput of the MI355X Mixture-of-Experts layer (one GPU).

A step is one ``moe_layer_forward`` call (route -> permute -> expert FFN ->
combine) over one synthetic batch whose inputs are already resident in HBM.
Each step routes by the next of 64 pre-drawn logit sets, so consecutive steps
touch different experts and the 256 MB Infinity Cache cannot serve the weights.

Prints one JSON line: tokens/s, the dominant kernel's roofline fraction
(its algorithmic bytes over its HIP-event duration, measured on the launch
stream inside this run), and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA TFLOP/s as % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="decode_bf16")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU oracle sample budget (seconds of oracle work)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    return p.parse_args()


def _expert_bytes(wl) -> dict:
    d, f = wl.d, wl.f
    if wl.wfmt == "mxfp4":
        gu = 2 * (f * d // 2 + f * d // 32)
        dn = d * f // 2 + d * f // 32
    else:
        b = 4 if wl.wfmt == "f32" else 2
        gu = 2 * f * d * b
        dn = d * f * b
    return dict(gate_up=gu, down=dn, total=gu + dn)


def _source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# Dominant kernel per path and the sources that define it (for the traffic
# counters recorded under profiles/).
DOMINANT = {
    "decode": ("gemv_gate_up", ["expert_ffn_layer_softmax_amd/csrc/gemv.hip",
                                "expert_ffn_layer_softmax_amd/csrc/device.h"]),
    "prefill": ("gg_gate_up", ["expert_ffn_layer_softmax_amd/csrc/grouped_gemm.hip",
                               "expert_ffn_layer_softmax_amd/csrc/device.h"]),
}
RIDGE_FLOP_PER_BYTE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)


def _traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, x, w, logit_sets, budget_s: float):
    """The oracle, as it stands, on the host: one token per logit set until the
    budget is spent.  Expert weights are copied to host memory untimed; decoding
    them to fp64 is part of the oracle's timed work."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1

    def raw(t):
        if wl.wfmt == "mxfp4":
            return t.cpu().numpy()
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    xh_raw = raw(x)
    T = wl.T
    done_tokens, spent, sets_used = 0, 0.0, 0
    for s in range(logit_sets.shape[0]):
        lg = logit_sets[s].cpu().numpy()
        idx, _ = oracle.route(lg, wl.k)
        experts = sorted(set(idx.ravel().tolist()))
        host = {}
        for e in experts:      # untimed staging to host memory
            host[e] = {n: raw(w[n][e]) for n in w}

        def get(e):
            h = host[e]
            if wl.wfmt == "mxfp4":
                return tuple(oracle.decode_mxfp4(h["w_" + n], h["s_" + n]) for n in ("gate", "up", "down"))
            return tuple(oracle.decode_bf16(h["w_" + n]) for n in ("gate", "up", "down"))

        t0 = time.perf_counter()
        xh = oracle.decode_bf16(xh_raw) if wl.act == "bf16" else xh_raw.astype(np.float64)
        oracle.layer(xh, lg, wl.k, get, E=wl.E)
        spent += time.perf_counter() - t0
        done_tokens += T
        sets_used += 1
        del host
        if spent >= budget_s:
            break
    return {"value": done_tokens / spent, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{sets_used} layer call(s) of the {wl.name} workload ({done_tokens} tokens, "
                      f"each with its own routing), numpy fp64, {spent:.1f} s; host affinity "
                      f"{len(os.sched_getaffinity(0))} cores"}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    from expert_ffn_layer_softmax_amd import (moe_layer_forward, moe_timing_names, moe_timing_query,
                                              moe_timing_start, moe_timing_stop)
    from synth import WORKLOADS, gen_expert_weights, gen_logits, gen_x

    wl = WORKLOADS[args.workload]
    assert not wl.router, "bench workloads route by pre-drawn logits"
    dev = torch.device("cuda:0")
    print(f"[bench] generating {wl.name} inputs", file=sys.stderr, flush=True)
    x = gen_x(wl.T, wl.d, wl.act, wl.seed, dev, std=wl.x_std)
    w = gen_expert_weights(wl, dev)
    sets = gen_logits(wl.T, wl.E, wl.seed, dev, sets=wl.logit_sets, bias_std=wl.bias_std)
    nsets = sets.shape[0]
    k = wl.k
    out = torch.empty(wl.T, wl.d, dtype=x.dtype, device=dev)
    topk_idx = torch.empty(wl.T, k, dtype=torch.int32, device=dev)
    topk_w = torch.empty(wl.T, k, dtype=torch.float32, device=dev)
    res = moe_layer_forward(x, w, k, logits=sets[0], topk_idx=topk_idx, topk_w=topk_w, out=out)
    ws = res["workspace"]

    # Steps call the C entry point directly with pre-marshalled arguments, so
    # host-side Python work does not pace the GPU.
    import ctypes

    from expert_ffn_layer_softmax_amd import _lib as L
    wfmt = L._wfmt(w)
    dims = L._dims(wl.T, wl.d, wl.E, k, wl.f, L._ACT[x.dtype], wfmt)
    wts = L._weights(w, wl.E, wl.d, wl.f, wfmt, dev)
    stream = L._stream(x)
    lptr = [ctypes.c_void_p(sets[i].data_ptr()) for i in range(nsets)]
    fixed = [ctypes.c_void_p(t.data_ptr()) for t in (x, topk_idx, topk_w, out, ws)]
    fwd = L.lib.moe_layer_forward
    dref, wref = ctypes.byref(dims), ctypes.byref(wts)
    wsn = ws.numel()

    def step(i):
        st = fwd(dref, fixed[0], None, lptr[i % nsets], wref, fixed[1], fixed[2], fixed[3], fixed[4],
                 wsn, stream)
        if st != 0:
            raise L.MoeError(st, "moe_layer_forward")

    # unique experts per step (for algorithmic bytes), from the device's routing
    uniq = []
    for i in range(nsets):
        step(i)
        uniq.append(int(torch.unique(topk_idx).numel()))
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms = el * 1e3 / args.steps
    tokens_per_s = wl.T * args.steps / el

    # per-kernel HIP-event durations on the launch stream (separate pass)
    moe_timing_start()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    moe_timing_stop()
    path = "decode" if wl.T <= 16 else "prefill"
    kname, srcs = DOMINANT[path]
    n_launch, tot_ms = moe_timing_query(kname)
    if n_launch == 0:
        raise RuntimeError(f"no timed launches of {kname}")
    kernel_us = tot_ms * 1e3 / n_launch
    eb = _expert_bytes(wl)
    act_b = 4 if wl.act == "f32" else 2
    mean_uniq = sum(uniq[i % nsets] for i in range(args.steps)) / args.steps
    # the gate/up kernel's algorithmic work: the active experts' gate and up
    # weights read once, x read, h written; 2 FLOPs per MAC over T*k rows
    k_bytes = mean_uniq * eb["gate_up"] + wl.T * wl.d * act_b + wl.T * k * wl.f * act_b
    k_flops = 4.0 * wl.T * k * wl.d * wl.f
    if k_flops / k_bytes > RIDGE_FLOP_PER_BYTE:
        bound, unit, peak = "mfma", "TFLOP/s", BF16_PEAK_TFLOPS
        achieved = k_flops / (kernel_us * 1e-6) / 1e12
    else:
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBS
        achieved = k_bytes / (kernel_us * 1e-6) / 1e9
    step_bytes = (mean_uniq * eb["total"] + 2 * wl.T * wl.d * act_b + wl.T * wl.E * 4 + wl.T * k * 8)
    step_flops = 6.0 * wl.T * k * wl.d * wl.f
    t_floor = max(step_bytes / (HBM_PEAK_GBS * 1e9), step_flops / (BF16_PEAK_TFLOPS * 1e12))
    digest = _source_digest(srcs)
    traffic = _traffic(kname, wl.name, digest)
    breakdown = {}
    for kn in moe_timing_names():
        n, t = moe_timing_query(kn)
        if n:
            breakdown[kn] = round(t * 1e3 / n, 2)

    rec = {
        "metric": METRIC, "value": round(tokens_per_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.act == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E, "k": k, "f": wl.f,
                   "weights": wl.wfmt, "logit_sets": nsets, "mean_unique_experts": round(mean_uniq, 2)},
        "roofline": {"bound": bound, "kernel": kname, "achieved": round(achieved, 1),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic, "kernel_us": round(kernel_us, 2),
                     "algorithmic_bytes_per_launch": int(k_bytes),
                     "algorithmic_flops_per_launch": k_flops},
        "step": {"algorithmic_bytes": int(step_bytes), "algorithmic_flops": step_flops,
                 "hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(step_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "attainable_frac": round(t_floor / (ms * 1e-3), 4),
                 "kernel_us": breakdown},
    }
    if not args.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, x, w, sets, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
