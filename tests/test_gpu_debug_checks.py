"""The bounds-checking debug build (libmoe_mi355x_dbg.so, -DMOE_DEBUG_CHECKS).

It runs in a child process (one library per process).  Valid layers on every
path record no violation and match the oracle.  Out-of-range indices passed
in from the host to the stage-wise entry points are recorded under their own
bit and clamped into range by the kernels, so every kernel still ends
normally; these calls are made only after the child has confirmed that the
debug build is the one loaded (the release build does not clamp).
"""

import json
import os
import subprocess
import sys

import pytest

from gpu_util import log, require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DBG = os.path.join(ROOT, "expert_ffn_layer_softmax_amd", "libmoe_mi355x_dbg.so")


def _child():
    """Runs in the child process, with the debug library loaded."""
    import zlib

    import torch

    import oracle
    from expert_ffn_layer_softmax_amd import (MoeError, moe_combine, moe_debug_check, moe_expert_ffn,
                                              moe_layer_forward, moe_permute, moe_route)
    from gpu_util import check_out, expert_getter, make_inputs, to_host_act
    from synth import Workload

    res = {}
    try:
        moe_debug_check()
    except MoeError as err:  # release build: stop before any out-of-range input
        res["debug_build"] = False
        res["error"] = str(err)
        return res
    res["debug_build"] = True

    # valid layers on every path: nothing recorded, outputs as the oracle's
    cases = [("t1_bf16", 1, 512, 32, 8, 256, "bf16", False), ("t1_mx", 1, 512, 32, 8, 256, "mxfp4", False),
             ("t5_nv", 5, 512, 32, 8, 256, "nvfp4", False), ("t40_bf16", 40, 256, 16, 4, 128, "bf16", False),
             ("t200_bf16", 200, 512, 16, 4, 384, "bf16", False), ("t150_mx", 150, 512, 8, 2, 384, "mxfp4", False),
             ("t100_nv", 100, 256, 8, 4, 256, "nvfp4", False), ("t100_mx_fp8", 100, 256, 8, 4, 512, "mxfp4", True),
             ("t100_nv_fp8", 100, 256, 8, 4, 512, "nvfp4", True)]
    for name, T, d, E, k, f, wfmt, fp8 in cases:
        wl = Workload(name, T=T, d=d, E=E, k=k, f=f, act="bf16", wfmt=wfmt,
                      seed=zlib.crc32(name.encode()) % 100000,
                      x_std=1.0, wg_std=d ** -0.5, wu_std=d ** -0.5, wd_std=f ** -0.5)
        x, w, _, logits = make_inputs(wl)
        out = moe_layer_forward(x, w, k, logits=logits, fp8=fp8)
        torch.cuda.synchronize()
        ref = oracle.layer(to_host_act(x), logits.cpu().numpy(), k, expert_getter(w, wfmt), E=E,
                           act_quant=oracle.quantize_mxfp8 if fp8 else None)
        check_out("debug_build_" + name, to_host_act(out["out"]), ref["out"], 5e-3,
                  token_tol=1e-2 if fp8 else None)
        res[name] = moe_debug_check()

    # stage-wise entry points with valid, then out-of-range, host inputs
    wl = Workload("stages", T=64, d=256, E=16, k=4, f=256, act="bf16", wfmt="bf16", seed=11,
                  x_std=1.0, wg_std=256 ** -0.5, wu_std=256 ** -0.5, wd_std=256 ** -0.5)
    x, w, _, logits = make_inputs(wl)
    idx, tw = moe_route(logits, wl.k)
    counts, offsets, sorted_src, dest_row = moe_permute(idx, wl.E)
    y = moe_expert_ffn(x, offsets, sorted_src, wl.k, w)
    moe_combine(y, dest_row, tw, x.dtype)
    torch.cuda.synchronize()
    res["stages_valid"] = moe_debug_check()
    Tk = wl.T * wl.k

    bad = dest_row.clone()
    bad[5] = Tk + 7
    bad[9] = -3
    moe_combine(y, bad, tw, x.dtype)
    moe_combine(y, bad, tw, x.dtype, expert_norm=True)
    torch.cuda.synchronize()
    res["dest_row"] = moe_debug_check()

    for T_sub in (64, 8):  # grouped GEMM path, then the GEMV path
        xs = x[:T_sub].contiguous()
        c2, o2, s2, _ = moe_permute(idx[:T_sub].contiguous(), wl.E)
        s_bad = s2.clone()
        s_bad[3] = T_sub * wl.k + 100
        moe_expert_ffn(xs, o2, s_bad, wl.k, w)
        torch.cuda.synchronize()
        res[f"sorted_src_T{T_sub}"] = moe_debug_check()

    i_bad = idx.clone()
    i_bad[2, 1] = wl.E + 5
    moe_permute(i_bad, wl.E)
    torch.cuda.synchronize()
    res["topk_idx"] = moe_debug_check()

    o_bad = offsets.clone()
    o_bad[-1] = Tk - 3  # does not end at T*k
    moe_expert_ffn(x, o_bad, sorted_src, wl.k, w)
    torch.cuda.synchronize()
    res["offsets"] = moe_debug_check()
    res["after"] = moe_debug_check()
    return res


def test_debug_checks_build():
    require_gpu()
    assert os.path.exists(DBG), "libmoe_mi355x_dbg.so is missing: run __graft_entry__.build()"
    env = dict(os.environ, MOE_MI355X_LIB=DBG)
    code = ("import json, sys; sys.path[:0] = [%r, %r]; import test_gpu_debug_checks as m; "
            "print('RESULT ' + json.dumps(m._child()), flush=True)") % (ROOT, os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-u", "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    log(r.stderr[-3000:])
    assert r.returncode == 0, f"child failed ({r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-3000:]}"
    line = [l for l in r.stdout.splitlines() if l.startswith("RESULT ")][-1]
    res = json.loads(line[len("RESULT "):])
    log(f"debug build: {res}")
    assert res["debug_build"], res
    for name in ("t1_bf16", "t1_mx", "t5_nv", "t40_bf16", "t200_bf16", "t150_mx", "t100_nv", "t100_mx_fp8",
                 "t100_nv_fp8", "stages_valid"):
        assert res[name] == 0, f"{name}: violations recorded on valid input ({res[name]})"
    assert res["dest_row"] == 1
    assert res["sorted_src_T64"] == 2 and res["sorted_src_T8"] == 2
    assert res["topk_idx"] == 32
    assert res["offsets"] == 16
    assert res["after"] == 0


def test_release_build_reports_no_checks():
    """The release library has no checks: moe_debug_check says so."""
    require_gpu()
    from expert_ffn_layer_softmax_amd import MoeError, moe_debug_check
    if os.environ.get("MOE_MI355X_LIB", "").endswith("_dbg.so"):
        pytest.skip("this process loaded the debug build")
    with pytest.raises(MoeError) as ei:
        moe_debug_check()
    assert ei.value.status == 2
