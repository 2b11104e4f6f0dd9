"""Throughput of the MI355X Mixture-of-Experts layer (one GPU).

A step is one ``moe_layer_forward`` call (route -> permute -> expert FFN ->
combine) over one synthetic batch whose inputs are already resident in HBM.
Decode steps route by the next of 64 pre-drawn logit sets, so consecutive
steps touch different experts and the 256 MB Infinity Cache cannot serve the
weights.

Prints one JSON line per workload: tokens/s (median of three timed loops),
the dominant kernel's roofline fraction (its algorithmic bytes or FLOPs over
its HIP-event duration, measured on the launch stream inside this run), and
the CPU oracle timed on a bounded sample.  Without --workload it runs
single-token bf16 decode, then MX-FP4 prefill, then bf16 prefill (T=4096).

``--calibrate-counters`` instead runs three plain 1 GiB device-to-device
copies: the reference that scales the FETCH_SIZE / WRITE_SIZE hardware
counters into bytes.
"""

from __future__ import annotations

import argparse
import dataclasses
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
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the FP8 x FP4 scaled MFMA runs at this rate)

# Default workloads, in print order: the single-token decode the headline is
# quoted on, then 4K-token prefill with MX-FP4 and with bf16 weights.
DEFAULT_WORKLOADS = ("decode_bf16", "prefill_mxfp4", "prefill_bf16")


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=None,
                   help="one workload (default: " + ", ".join(DEFAULT_WORKLOADS) + ", in that order)")
    p.add_argument("--repeats", type=int, default=3,
                   help="timed loops of --steps steps each; value is their median")
    p.add_argument("--cpu-tokens", type=int, default=16,
                   help="tokens per CPU oracle call on workloads with more tokens than that")
    p.add_argument("--calibrate-counters", action="store_true",
                   help="run three 1 GiB device copies (counter calibration) and exit")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU oracle sample budget (seconds of oracle work)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--T", type=int, default=None,
                   help="override the workload's token count; the name gets a _T<n> suffix")
    p.add_argument("--sweep", default=None,
                   help="comma-separated token counts: one JSON line per T (weights generated once)")
    p.add_argument("--layers", type=int, default=1,
                   help="chain this many layers per step, each with its own weights (out of one "
                        "layer is x of the next); tokens/s counts each token once per step")
    p.add_argument("--fp8", action="store_true",
                   help="FP8 activations (MXFP8); MX-FP4 (scaled FP8 MFMA) and NVFP4 (bf16 MFMA) workloads")
    p.add_argument("--expert-norm", action="store_true",
                   help="RMS-normalise each expert's output row before the combine "
                        "(MOE_FLAG_EXPERT_NORM)")
    p.add_argument("--share", choices=["ep8", "tp8"], default=None,
                   help="time one GPU's share of the layer split over 8 GPUs: ep8 = 1/8 of the "
                        "experts with the T*k/8 rows dispatched to them (k=1 locally), tp8 = every "
                        "expert with f/8; tokens/s counts the whole layer's tokens")
    p.add_argument("--streams", type=int, default=1,
                   help="independent requests per step: each a layer call (its own logit set, "
                        "workspace and outputs) on its own HIP stream at the default priority, "
                        "so their kernels may overlap; tokens/s counts every request's tokens")
    p.add_argument("--graph", action="store_true",
                   help="replay each step from a captured HIP graph (one graph per logit-set "
                        "offset, rotated) instead of launching it")
    return p.parse_args()


def _expert_bytes(wl) -> dict:
    d, f = wl.d, wl.f
    if wl.wfmt in ("mxfp4", "nvfp4"):
        sd = 32 if wl.wfmt == "mxfp4" else 16   # elements per scale byte
        gu = 2 * (f * d // 2 + f * d // sd)
        dn = d * f // 2 + d * f // sd
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
                                "expert_ffn_layer_softmax_amd/csrc/device.h",
                                "expert_ffn_layer_softmax_amd/csrc/route_dev.h"]),
    "prefill": ("gg_gate_up", ["expert_ffn_layer_softmax_amd/csrc/grouped_gemm.hip",
                               "expert_ffn_layer_softmax_amd/csrc/device.h"]),
}


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


def cpu_baseline(wl, x, w, logit_sets, budget_s: float, fp8: bool = False,
                 expert_norm: bool = False, chunk: int = 16):
    """The oracle, as it stands, on the host, until the budget is spent.
    Workloads of up to `chunk` tokens run whole, one call per logit set; larger
    ones run `chunk` consecutive tokens of the batch per call (the layer is
    per-token independent), from the first token on.  Expert weights are
    copied to host memory untimed; decoding them to fp64 is part of the
    oracle's timed work."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1

    def raw(t):
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.contiguous().view(torch.uint8).cpu().numpy()
        return t.cpu().numpy()

    xh_all = raw(x)
    T = wl.T
    calls = []  # (logit set, first token, tokens)
    if T <= chunk:
        calls = [(s, 0, T) for s in range(logit_sets.shape[0])]
    else:
        calls = [(0, t0, min(chunk, T - t0)) for t0 in range(0, T, chunk)]
    done_tokens, spent, ncalls = 0, 0.0, 0
    for s, t0, n in calls:
        lg = logit_sets[s][t0:t0 + n].cpu().numpy()
        xh_raw = xh_all[t0:t0 + n]
        idx, _ = oracle.route(lg, wl.k)
        experts = sorted(set(idx.ravel().tolist()))
        host = {}
        for e in experts:      # untimed staging to host memory
            host[e] = {nm: raw(w[nm][e]) for nm in w}

        def get(e):
            h = host[e]
            if wl.wfmt == "mxfp4":
                return tuple(oracle.decode_mxfp4(h["w_" + n], h["s_" + n]) for n in ("gate", "up", "down"))
            if wl.wfmt == "nvfp4":
                return tuple(oracle.decode_nvfp4(h["w_" + n], h["s_" + n], h["t_" + n])
                             for n in ("gate", "up", "down"))
            if wl.wfmt == "f32":
                return tuple(h["w_" + n].astype(np.float64) for n in ("gate", "up", "down"))
            return tuple(oracle.decode_bf16(h["w_" + n]) for n in ("gate", "up", "down"))

        t_start = time.perf_counter()
        xh = oracle.decode_bf16(xh_raw) if wl.act == "bf16" else xh_raw.astype(np.float64)
        oracle.layer(xh, lg, wl.k, get, E=wl.E, act_quant=oracle.quantize_mxfp8 if fp8 else None,
                     expert_norm=expert_norm)
        spent += time.perf_counter() - t_start
        done_tokens += n
        ncalls += 1
        del host
        if spent >= budget_s:
            break
    if T <= chunk:
        what = (f"{ncalls} layer call(s) of the {wl.name} workload ({done_tokens} tokens, each call "
                f"with its own routing)")
    else:
        what = (f"the first {done_tokens} of the {T} tokens of the {wl.name} workload, {chunk} tokens "
                f"per oracle call ({ncalls} calls), with the batch's own routing")
    return {"value": done_tokens / spent, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what}; numpy fp64, {spent:.1f} s; host affinity "
                      f"{len(os.sched_getaffinity(0))} cores"}


def measure(wl, ws_list, args, with_cpu: bool):
    """Time `args.steps` steps of `args.layers` chained layers of workload `wl`
    (weights `ws_list[i]` for layer i) and return the JSON record."""
    import ctypes

    import torch

    from expert_ffn_layer_softmax_amd import (moe_layer_forward, moe_timing_names, moe_timing_query,
                                              moe_timing_start, moe_timing_stop)
    from expert_ffn_layer_softmax_amd import _lib as L
    from synth import gen_logits, gen_x

    dev = torch.device("cuda:0")
    nl = len(ws_list)
    x = gen_x(wl.T, wl.d, wl.act, wl.seed, dev, std=wl.x_std)
    sets = gen_logits(wl.T, wl.E, wl.seed, dev, sets=wl.logit_sets, bias_std=wl.bias_std)
    nsets = sets.shape[0]
    k = wl.k
    # layer i reads acts[i] and writes acts[i + 1]; acts[0] is x
    acts = [x] + [torch.empty(wl.T, wl.d, dtype=x.dtype, device=dev) for _ in range(nl)]
    topk_idx = torch.empty(wl.T, k, dtype=torch.int32, device=dev)
    topk_w = torch.empty(wl.T, k, dtype=torch.float32, device=dev)
    res = moe_layer_forward(x, ws_list[0], k, logits=sets[0], topk_idx=topk_idx, topk_w=topk_w,
                            out=acts[1], fp8=args.fp8, expert_norm=args.expert_norm)
    ws = res["workspace"]

    # Steps call the C entry point directly with pre-marshalled arguments, so
    # host-side Python work does not pace the GPU.
    wfmt = L._wfmt(ws_list[0])
    dims = L._dims(wl.T, wl.d, wl.E, k, wl.f, L._ACT[x.dtype], wfmt,
                   L._flags(args.fp8, args.expert_norm))
    wts = [L._weights(w, wl.E, wl.d, wl.f, wfmt, dev) for w in ws_list]
    lptr = [ctypes.c_void_p(sets[i].data_ptr()) for i in range(nsets)]
    aptr = [ctypes.c_void_p(t.data_ptr()) for t in acts]
    fixed = [ctypes.c_void_p(t.data_ptr()) for t in (topk_idx, topk_w, ws)]
    fwd = L.lib.moe_layer_forward
    dref, wref = ctypes.byref(dims), [ctypes.byref(t) for t in wts]
    wsn = ws.numel()

    def launch(i, stream, bufs=None):
        ap, fx = (aptr, fixed) if bufs is None else bufs
        for layer in range(nl):
            st = fwd(dref, ap[layer], None, lptr[(i + layer) % nsets], wref[layer], fx[0],
                     fx[1], ap[layer + 1], fx[2], wsn, stream)
            if st != 0:
                raise L.MoeError(st, "moe_layer_forward")

    stream0 = L._stream(x)

    def step(i):
        launch(i, stream0)

    # --streams S: requests 1..S-1 get their own outputs, workspace and stream
    # (request 0 is the one above, on the current stream)
    S = max(1, args.streams)
    others = []
    for _ in range(S - 1):
        a_s = [x] + [torch.empty_like(t) for t in acts[1:]]
        f_s = [torch.empty_like(topk_idx), torch.empty_like(topk_w), torch.empty_like(ws)]
        strm = torch.cuda.Stream()
        others.append((strm, ([ctypes.c_void_p(t.data_ptr()) for t in a_s],
                              [ctypes.c_void_p(t.data_ptr()) for t in f_s]), a_s + f_s))
    if others:
        for strm, _, _ in others:
            strm.wait_stream(torch.cuda.current_stream())

        def step(i):  # noqa: F811
            launch(S * i, stream0)
            for j, (strm, bufs, _) in enumerate(others):
                launch(S * i + j + 1, ctypes.c_void_p(strm.cuda_stream), bufs)

    # unique experts per layer call (for algorithmic bytes), from the device's routing
    uniq = []
    for i in range(nsets):
        fwd(dref, aptr[0], None, lptr[i], wref[0], fixed[0], fixed[1], aptr[1], fixed[2], wsn, stream0)
        uniq.append(int(torch.unique(topk_idx).numel()))

    graphs = None
    if args.graph and others:
        raise SystemExit("--graph takes one stream")
    if args.graph:
        # one graph per logit-set offset; replays rotate through them
        ng = min(nsets, 8)
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(ng):
                launch(i, ctypes.c_void_p(side.cuda_stream))  # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for i in range(ng):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                launch(i, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            graphs.append(g)
        torch.cuda.synchronize()

        def step(i):  # noqa: F811
            graphs[i % len(graphs)].replay()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: timing {args.steps} steps of {nl} layer(s)"
          f"{' from HIP graphs' if graphs else ''}", file=sys.stderr, flush=True)
    loops = []
    for r in range(max(1, args.repeats)):
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(r * args.steps + i)
        torch.cuda.synchronize()
        loops.append(time.perf_counter() - t0)
    el = sorted(loops)[len(loops) // 2]
    ms = el * 1e3 / args.steps
    tokens_per_s = getattr(args, "job_tokens", wl.T) * S * args.steps / el

    # per-kernel HIP-event durations on the launch stream (separate pass of
    # launched steps; graph replays carry no events)
    moe_timing_start()
    for i in range(args.steps):
        launch(i, stream0)
    torch.cuda.synchronize()
    moe_timing_stop()
    # the path the library took: the grouped GEMM kernels ran, or the GEMV ones
    path = "prefill" if moe_timing_query("gg_gate_up")[0] > 0 else "decode"
    kname, srcs = DOMINANT[path]
    n_launch, tot_ms = moe_timing_query(kname)
    if n_launch == 0:
        raise RuntimeError(f"no timed launches of {kname}")
    kernel_us = tot_ms * 1e3 / n_launch
    eb = _expert_bytes(wl)
    act_b = 4 if wl.act == "f32" else 2
    mean_uniq = sum(uniq) / len(uniq)
    # the gate/up kernel's algorithmic work: the active experts' gate and up
    # weights read once, x read, h written; 2 FLOPs per MAC over T*k rows
    k_bytes = mean_uniq * eb["gate_up"] + wl.T * wl.d * act_b + wl.T * k * wl.f * act_b
    k_flops = 4.0 * wl.T * k * wl.d * wl.f
    # FP8 activations run on the scaled FP8 MFMA with MX-FP4 weights; with
    # NVFP4 weights they are carried as bf16 values on the bf16 MFMA
    scaled_fp8 = args.fp8 and wl.wfmt == "mxfp4"
    mfma_peak = FP8_PEAK_TFLOPS if scaled_fp8 else BF16_PEAK_TFLOPS
    if k_flops / k_bytes > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        bound, unit, peak = "mfma", "TFLOP/s", mfma_peak
        achieved = k_flops / (kernel_us * 1e-6) / 1e12
    else:
        bound, unit, peak = "hbm", "GB/s", HBM_PEAK_GBS
        achieved = k_bytes / (kernel_us * 1e-6) / 1e9
    layer_bytes = (mean_uniq * eb["total"] + 2 * wl.T * wl.d * act_b + wl.T * wl.E * 4 + wl.T * k * 8)
    layer_flops = 6.0 * wl.T * k * wl.d * wl.f
    # S independent requests per step, each streaming its own experts
    step_bytes, step_flops = S * nl * layer_bytes, S * nl * layer_flops
    t_floor = max(step_bytes / (HBM_PEAK_GBS * 1e9), step_flops / (mfma_peak * 1e12))
    digest = _source_digest(srcs)
    # counters are kept per path: the FP8 GEMMs are other kernels than the
    # bf16-activation ones of the same workload
    traffic = _traffic(kname, wl.name + ("_fp8" if args.fp8 else ""), digest) if nl == 1 else None
    breakdown = {}
    for kn in moe_timing_names():
        n, t = moe_timing_query(kn)
        if n:
            breakdown[kn] = round(t * 1e3 / n, 2)

    cfg = {"workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E, "k": k, "f": wl.f,
           "weights": wl.wfmt, "logit_sets": nsets, "mean_unique_experts": round(mean_uniq, 2)}
    if nl > 1:
        cfg["layers"] = nl
    if graphs:
        cfg["hip_graph"] = True
    if S > 1:
        cfg["streams"] = S
    if args.fp8:
        cfg["activations"] = "mxfp8"
    if args.expert_norm:
        cfg["expert_norm"] = "rms"
    rec = {
        "metric": METRIC, "value": round(tokens_per_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "repeats": len(loops), "ms_per_step_loops": [round(v * 1e3 / args.steps, 5) for v in loops],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8" if scaled_fp8 else ("bf16" if wl.act == "bf16" else "f32"), "data": "synthetic",
        "config": cfg,
        "roofline": {"bound": bound, "kernel": kname, "achieved": round(achieved, 1),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic, "kernel_us": round(kernel_us, 2),
                     "algorithmic_bytes_per_launch": int(k_bytes),
                     "algorithmic_flops_per_launch": k_flops},
        "step": {"algorithmic_bytes": int(step_bytes), "algorithmic_flops": step_flops,
                 "hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(step_flops / (ms * 1e-3) / 1e12 / mfma_peak, 4),
                 "attainable_frac": round(t_floor / (ms * 1e-3), 4),
                 "kernel_us": breakdown},
    }
    if with_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, x, ws_list[0], sets, args.cpu_seconds, args.fp8,
                                           args.expert_norm, chunk=args.cpu_tokens)
    else:
        rec["cpu_baseline"] = None
    return rec


def calibrate_counters():
    """Three plain 1 GiB device-to-device copies: what FETCH_SIZE and
    WRITE_SIZE read for them gives the factors that turn the counters into
    bytes (run under rocprofv3 --pmc with the copy kernel's name)."""
    import torch

    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied 3 x 1 GiB device to device", flush=True)


def run_workload(name, args):
    import torch

    from synth import WORKLOADS, gen_expert_weights

    base = WORKLOADS[name]
    assert not base.router, "bench workloads route by pre-drawn logits"
    if args.share:
        # One GPU's share at G = 8.  Expert parallelism: E/8 local experts
        # receive T*k/8 (token, expert) rows, each for one local expert.
        # Tensor parallelism over f: every expert, f/8 of its width.
        args.job_tokens = base.T
        if args.share == "ep8":
            base = dataclasses.replace(base, E=base.E // 8, k=1, T=max(1, base.T * base.k // 8),
                                       name=f"{base.name}_ep8_share")
        else:
            base = dataclasses.replace(base, f=base.f // 8, name=f"{base.name}_tp8_share")
        if args.T is not None or args.sweep:
            raise SystemExit("--share takes the workload's own T")
    dev = torch.device("cuda:0")
    print(f"[bench] generating {base.name} weights for {args.layers} layer(s)", file=sys.stderr, flush=True)
    # each layer's experts come from their own seed
    ws_list = [gen_expert_weights(dataclasses.replace(base, seed=base.seed + 7919 * i), dev)
               for i in range(args.layers)]
    if args.sweep:
        for T in [int(t) for t in args.sweep.split(",")]:
            wl = dataclasses.replace(base, T=T, name=f"{base.name}_T{T}")
            print(json.dumps(measure(wl, ws_list, args, with_cpu=False)), flush=True)
    else:
        wl = base
        if args.T is not None:
            wl = dataclasses.replace(base, T=args.T, name=f"{base.name}_T{args.T}")
        rec = measure(wl, ws_list, args, with_cpu=not args.no_cpu and args.layers == 1 and not args.share)
        if args.share:
            rec["config"]["share"] = args.share
            rec["config"]["job_tokens"] = args.job_tokens
        print(json.dumps(rec), flush=True)
    del ws_list
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_counters:
        calibrate_counters()
        return
    if args.layers < 1:
        raise SystemExit("--layers must be >= 1")
    names = [args.workload] if args.workload else list(DEFAULT_WORKLOADS)
    for name in names:
        run_workload(name, args)


if __name__ == "__main__":
    main()
