"""moe_layer_forward_noalloc (the library's own scratch, no workspace) against
moe_layer_forward (a caller's workspace): the same kernels on the same
inputs, so outputs, indices and weights must be bit-identical.  Calls come in
a row, each smaller than the one before, so a call that read what an earlier,
larger call left in the shared scratch would show."""

import zlib

import numpy as np
import pytest
import torch

from gpu_util import log, make_inputs, require_gpu
from synth import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def _same(a, b, what):
    assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else
                       a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int32) if b.dtype == torch.float32 else
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b), what


# (name, d, E, k, f, act, wfmt, token counts of the successive calls)
CASES = [
    ("bf16", 1024, 32, 8, 512, "bf16", "bf16", [200, 64, 16, 3, 1]),    # MFMA, GEMV, fused T=1
    ("mxfp4", 1024, 32, 8, 512, "bf16", "mxfp4", [150, 48, 5, 1]),      # routing inside gate/up at T=1
    ("nvfp4", 512, 16, 4, 256, "bf16", "nvfp4", [100, 2, 1]),
    ("f32", 256, 8, 2, 128, "f32", "f32", [40, 1]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry_point(case):
    from expert_ffn_layer_softmax_amd import moe_layer_forward, moe_layer_forward_noalloc
    name, d, E, k, f, act, wfmt, Ts = case
    wl = Workload(f"noalloc_{name}", T=max(Ts), d=d, E=E, k=k, f=f, act=act, wfmt=wfmt,
                  seed=zlib.crc32(name.encode()) % 100000,
                  x_std=1.0, wg_std=d ** -0.5, wu_std=d ** -0.5, wd_std=f ** -0.5)
    x_all, w, _, logits_all = make_inputs(wl)
    for T in Ts:
        log(f"noalloc {name} T={T}")
        x = x_all[:T].contiguous()
        logits = logits_all[:T].contiguous()
        ref = moe_layer_forward(x, w, k, logits=logits)
        got = moe_layer_forward_noalloc(x, w, k, logits=logits)
        torch.cuda.synchronize()
        _same(got["topk_idx"], ref["topk_idx"], f"{name} T={T}: topk_idx")
        _same(got["topk_w"], ref["topk_w"], f"{name} T={T}: topk_w")
        _same(got["out"], ref["out"], f"{name} T={T}: out")
        assert not np.isnan(got["out"].float().cpu().numpy()).any()


def test_noalloc_with_router_and_rejection():
    """In-path router logits (written to `logits`), then a shape whose
    workspace exceeds the scratch: rejected, and the scratch still serves the
    next call."""
    from expert_ffn_layer_softmax_amd import MoeError, moe_layer_forward, moe_layer_forward_noalloc
    wl = Workload("noalloc_router", T=37, d=512, E=64, k=8, f=256, act="bf16", wfmt="bf16", router=True,
                  seed=4711, x_std=1.0, wg_std=512 ** -0.5, wu_std=512 ** -0.5, wd_std=256 ** -0.5)
    x, w, w_r, _ = make_inputs(wl)
    ref = moe_layer_forward(x, w, wl.k, w_router=w_r)
    got = moe_layer_forward_noalloc(x, w, wl.k, w_router=w_r)
    torch.cuda.synchronize()
    _same(got["logits"], ref["logits"], "logits")
    _same(got["out"], ref["out"], "out")
    # 4096 tokens at d = 6144, E = 256, k = 8: y_sorted alone is 805 MB of
    # workspace (f = 32 keeps the weights small)
    big = torch.zeros(4096, 6144, dtype=torch.bfloat16, device="cuda")
    wsmall = dict(w_gate=torch.zeros(256, 32, 6144, dtype=torch.bfloat16, device="cuda"),
                  w_up=torch.zeros(256, 32, 6144, dtype=torch.bfloat16, device="cuda"),
                  w_down=torch.zeros(256, 6144, 32, dtype=torch.bfloat16, device="cuda"))
    lg = torch.zeros(4096, 256, dtype=torch.float32, device="cuda")
    with pytest.raises(MoeError) as ei:
        moe_layer_forward_noalloc(big, wsmall, 8, logits=lg)
    assert ei.value.status == 3
    del big, wsmall, lg
    got2 = moe_layer_forward_noalloc(x[:5].contiguous(), w, wl.k, w_router=w_r)
    ref2 = moe_layer_forward(x[:5].contiguous(), w, wl.k, w_router=w_r)
    torch.cuda.synchronize()
    _same(got2["out"], ref2["out"], "out after a rejected call")


@pytest.mark.parametrize("T,wfmt", [(1, "mxfp4"), (16, "bf16"), (100, "bf16"), (100, "mxfp4")])
def test_noalloc_under_graph_capture(T, wfmt):
    """The callers this entry point is for include code under HIP graph
    capture.  Captured once, the call replays to the eager result bit for
    bit, each replay after an eager call with other routing has rewritten
    the shared scratch and the outputs."""
    from expert_ffn_layer_softmax_amd import moe_layer_forward_noalloc
    log(f"noalloc graph T={T} {wfmt}")
    k = 8
    wl = Workload(f"noalloc_graph_{wfmt}", T=T, d=512, E=32, k=k, f=256, act="bf16", wfmt=wfmt, seed=97 + T,
                  x_std=1.0, wg_std=512 ** -0.5, wu_std=512 ** -0.5, wd_std=256 ** -0.5)
    x, w, _, logits = make_inputs(wl)
    other = torch.randn(T, wl.E, generator=torch.Generator().manual_seed(1000 + T)).cuda()
    eager = moe_layer_forward_noalloc(x, w, k, logits=logits)
    torch.cuda.synchronize()
    ref_out, ref_idx, ref_w = eager["out"].clone(), eager["topk_idx"].clone(), eager["topk_w"].clone()
    out = torch.empty_like(ref_out)
    idx = torch.empty_like(ref_idx)
    tw = torch.empty_like(ref_w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe_layer_forward_noalloc(x, w, k, logits=logits, topk_idx=idx, topk_w=tw, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe_layer_forward_noalloc(x, w, k, logits=logits, topk_idx=idx, topk_w=tw, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        moe_layer_forward_noalloc(x, w, k, logits=other, topk_idx=idx, topk_w=tw, out=out)
        torch.cuda.synchronize()
        assert not torch.equal(idx, ref_idx), "the eager call should route differently"
        g.replay()
        torch.cuda.synchronize()
        _same(idx, ref_idx, f"replay {rep}: topk_idx")
        _same(tw, ref_w, f"replay {rep}: topk_w")
        _same(out, ref_out, f"replay {rep}: out")
