"""GPU parity: every entry point of the HIP library against the oracle.

Routing (indices, counts, offsets, sorted_src, dest_row) must match bit for
bit given the device's own fp32 logits; routing weights to 1e-5 relative;
layer outputs to relative L2 <= 1e-5 (fp32) and 5e-3 (bf16, and 4-bit weights,
whose decoded values are exact in bf16), both over the whole output and for
every token's row on its own (FP8 activations: 1e-2 per token).
Shapes span several tiles with ragged tails; full-size decode and verify
workloads run in the launch configuration the bench times, and full-size
prefill is checked on every token that owns a row at an edge of the grouped
GEMM's row tiling.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (ACT_TOL, FP8_TOKEN_TOL, MXFP4_TOL, PrefetchGetter, check_out, check_routing,
                      expert_getter, log, make_inputs, record, rel_l2, require_gpu, run_layer_and_oracle,
                      stratified_tokens, to_host_act, token_rel_l2)
from synth import WORKLOADS, Workload, gen_expert_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def _tol(wl):
    return MXFP4_TOL if wl.wfmt in ("mxfp4", "nvfp4") else ACT_TOL[wl.act]


# --------------------------------------------------------------------- route
@pytest.mark.parametrize("T,E,k,mode", [
    (1, 256, 8, "normal"), (16, 256, 8, "normal"), (4096, 256, 8, "normal"),
    (37, 8, 2, "ties"), (64, 100, 7, "ties"), (33, 1000, 64, "normal"), (5, 1024, 1, "ties"),
    (9, 64, 64, "ties"), (11, 300, 16, "neginf"), (3, 1, 1, "normal"), (130, 129, 9, "neginf"),
])
def test_route(T, E, k, mode):
    from expert_ffn_layer_softmax_amd import moe_route
    log(f"route T={T} E={E} k={k} {mode}")
    g = torch.Generator().manual_seed(T * 1000 + E + k)
    if mode == "ties":
        l = torch.randint(0, 4, (T, E), generator=g).float()
    else:
        l = torch.randn(T, E, generator=g)
    if mode == "neginf":
        l[torch.rand(T, E, generator=g) < 0.3] = -float("inf")
        l[0, :] = -float("inf")
        l[1, : E // 2] = -float("inf")
        l[2, 0] = -0.0
        l[2, 1] = 0.0
    idx, w = moe_route(l.cuda(), k)
    torch.cuda.synchronize()
    ref_idx, ref_w = oracle.route(l.numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=1e-5, atol=1e-7)


# ------------------------------------------------------------------- permute
@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (16, 256, 8), (4096, 256, 8), (333, 1024, 3),
                                   (1000, 1, 1), (50, 7, 7), (2048, 64, 64), (129, 1000, 8),
                                   # a wave's chunk over several key groups, ragged at the end
                                   (8191, 256, 8), (4097, 1024, 8), (3001, 512, 5)])
def test_permute(T, E, k):
    from expert_ffn_layer_softmax_amd import moe_permute
    log(f"permute T={T} E={E} k={k}")
    g = torch.Generator().manual_seed(7 * T + E)
    # skewed: logits with a per-expert bias, top-k by sort
    logits = torch.randn(T, E, generator=g) + torch.randn(E, generator=g) * 1.5
    idx = torch.topk(logits, k, dim=1).indices.to(torch.int32).contiguous()
    counts, offsets, sorted_src, dest_row = moe_permute(idx.cuda(), E)
    torch.cuda.synchronize()
    rc, ro, rs, rd = oracle.permute(idx.numpy(), E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(sorted_src.cpu().numpy(), rs)
    assert np.array_equal(dest_row.cpu().numpy(), rd)


# ------------------------------------------------------------- small layers
SMALL = [
    # name, T, d, E, k, f, act, wfmt
    ("bf16_t1", 1, 256, 16, 4, 96, "bf16", "bf16"),
    ("bf16_t5", 5, 512, 32, 8, 160, "bf16", "bf16"),
    ("bf16_t16", 16, 1024, 64, 8, 352, "bf16", "bf16"),
    ("bf16_t17", 17, 256, 8, 2, 128, "bf16", "bf16"),
    ("bf16_t200", 200, 192, 12, 3, 224, "bf16", "bf16"),
    ("bf16_segd", 2, 9216, 4, 2, 64, "bf16", "bf16"),
    ("bf16_segf", 3, 64, 4, 2, 9216, "bf16", "bf16"),
    ("mx_t1", 1, 256, 16, 4, 96, "bf16", "mxfp4"),
    ("mx_t5", 5, 512, 32, 8, 160, "bf16", "mxfp4"),
    ("mx_t16", 16, 1024, 64, 8, 352, "bf16", "mxfp4"),
    ("mx_t40", 40, 256, 8, 2, 128, "bf16", "mxfp4"),
    ("mx_segd", 1, 33792, 2, 1, 32, "bf16", "mxfp4"),
    ("f32_t3", 3, 96, 5, 5, 32, "f32", "f32"),
    ("f32_t64", 64, 128, 16, 4, 64, "f32", "f32"),
    ("f32_segd", 2, 4160, 3, 2, 32, "f32", "f32"),
    ("bf16_t1_k16", 1, 512, 64, 16, 224, "bf16", "bf16"),
    ("bf16_t1_k20", 1, 256, 32, 20, 64, "bf16", "bf16"),
    ("f32_t1", 1, 128, 8, 3, 64, "f32", "f32"),
    ("mx_t1_bigf", 1, 64, 4, 2, 8192, "bf16", "mxfp4"),
    # single token, 4-bit, the balanced gate/up and ring down+combine kernels:
    # 40 and 88 chunks per row (partial last chunk slot), d % 12 != 0 (partial
    # last block of 12 output rows), 64 slots, 256 chunks per gate/up row
    ("mx_t1_ring", 1, 1280, 16, 8, 2816, "bf16", "mxfp4"),
    ("nv_t1_ring", 1, 1280, 16, 6, 1408, "bf16", "nvfp4"),
    ("mx_t1_k64", 1, 256, 64, 64, 128, "bf16", "mxfp4"),
    ("mx_t1_bigd", 1, 8192, 8, 2, 256, "bf16", "mxfp4"),
    ("nv_t1_bigd", 1, 8192, 8, 3, 384, "bf16", "nvfp4"),
    # routing inside the single-token gate/up kernel at 2, 8 and 16 logits per lane
    ("mx_t1_e128", 1, 256, 128, 8, 128, "bf16", "mxfp4"),
    ("nv_t1_e512", 1, 256, 512, 4, 128, "bf16", "nvfp4"),
    ("mx_t1_e1024", 1, 256, 1024, 16, 256, "bf16", "mxfp4"),
    ("bf16_t1_bigf", 1, 64, 4, 2, 16384, "bf16", "bf16"),
    ("bf16_t47", 47, 320, 16, 4, 192, "bf16", "bf16"),          # largest T on the GEMV path
    ("bf16_longrow_t2", 2, 3584, 8, 2, 96, "bf16", "bf16"),      # rows in quarters, 2 chunks/lane
    ("f32_longrow_t3", 3, 2048, 8, 2, 64, "f32", "f32"),         # fp32 rows in quarters
    ("mx_t47", 47, 320, 16, 4, 192, "bf16", "mxfp4"),
    # grouped MFMA GEMM path (T >= 48, d and f multiples of 64)
    ("gg_bf16_t48", 48, 256, 8, 2, 128, "bf16", "bf16"),
    ("gg_bf16_t300", 300, 512, 16, 4, 384, "bf16", "bf16"),
    ("gg_bf16_hot", 600, 384, 4, 2, 256, "bf16", "bf16"),      # ~300 rows/expert: 3 m-tiles
    ("gg_bf16_ntail", 64, 640, 6, 3, 128, "bf16", "bf16"),     # down N=640: partial n-tile
    ("gg_bf16_oddk", 70, 320, 6, 2, 192, "bf16", "bf16"),      # odd K-step counts
    ("gg_bf16_ktail", 120, 352, 8, 2, 352, "bf16", "bf16"),    # K % 64 == 32 on both GEMMs
    ("gg_bf16_ktail_t48", 48, 160, 4, 2, 96, "bf16", "bf16"),  # 2.5 and 1.5 K-steps
    ("gg_mx_t100", 100, 256, 8, 4, 256, "bf16", "mxfp4"),
    ("gg_mx_hot", 700, 512, 5, 2, 384, "bf16", "mxfp4"),
    ("gg_mx_ntail", 90, 640, 6, 2, 256, "bf16", "mxfp4"),      # down N=640: partial n-tile
    ("gg_mx_oddk", 80, 320, 6, 2, 192, "bf16", "mxfp4"),       # K % 128 != 0 on both GEMMs
    ("gg_mx_gtail", 150, 512, 6, 2, 320, "bf16", "mxfp4"),     # gate/up N=320: partial n-tile
    ("gg_mx_ktail", 120, 352, 8, 2, 352, "bf16", "mxfp4"),     # K % 64 == 32 on both GEMMs
    ("gg_mx_ktail_t48", 48, 96, 4, 2, 160, "bf16", "mxfp4"),   # 1.5 and 2.5 K-steps
    # MX-FP4 tiles of 129..256 rows (K % 256 == 0)
    ("gg_mx_big", 640, 512, 8, 2, 512, "bf16", "mxfp4"),       # ~160 rows/expert, both GEMMs
    ("gg_mx_big_hot", 900, 256, 3, 2, 768, "bf16", "mxfp4"),   # ~600 rows/expert: 256 + 256 + rest
    ("gg_mx_big_gtail", 520, 512, 4, 2, 320, "bf16", "mxfp4"), # gate/up N=320: partial n-tile
    ("gg_mx_big_dtail", 520, 640, 4, 2, 512, "bf16", "mxfp4"), # down N=640: partial n-tile
    # NVFP4: 16-element E4M3 blocks and fp32 matrix scales
    ("nv_t1", 1, 256, 16, 4, 96, "bf16", "nvfp4"),
    ("nv_t5", 5, 512, 32, 8, 160, "bf16", "nvfp4"),
    ("nv_t16", 16, 1024, 64, 8, 352, "bf16", "nvfp4"),
    ("nv_t40", 40, 256, 8, 2, 128, "bf16", "nvfp4"),
    ("nv_segd", 1, 33792, 2, 1, 32, "bf16", "nvfp4"),
    ("nv_t1_bigf", 1, 64, 4, 2, 8192, "bf16", "nvfp4"),
    ("nv_oddk_t100", 100, 320, 6, 2, 192, "bf16", "nvfp4"),     # K % 256 != 0: GEMV at any T
    ("gg_nv_t100", 100, 256, 8, 4, 256, "bf16", "nvfp4"),
    ("gg_nv_hot", 700, 512, 5, 2, 512, "bf16", "nvfp4"),
    ("gg_nv_tails", 150, 768, 6, 2, 512, "bf16", "nvfp4"),      # partial n-tiles on both GEMMs
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_layer_small(case):
    name, T, d, E, k, f, act, wfmt = case
    log(f"layer {name}")
    wl = Workload(name, T=T, d=d, E=E, k=k, f=f, act=act, wfmt=wfmt, seed=zlib.crc32(name.encode()) % 100000,
                  x_std=1.0, wg_std=d ** -0.5, wu_std=d ** -0.5, wd_std=f ** -0.5)
    x, w, w_r, logits = make_inputs(wl)
    got, ref, _ = run_layer_and_oracle(wl, x, w, w_r, logits)
    check_out(name, got, ref["out"], _tol(wl))


@pytest.mark.parametrize("name", ["tiny_fp32", "tiny_fp32_stress"])
def test_layer_tiny_fp32_with_router(name):
    wl = WORKLOADS[name]
    log(f"layer {name}")
    x, w, w_r, logits = make_inputs(wl)
    got, ref, _ = run_layer_and_oracle(wl, x, w, w_r, logits)
    check_out(name, got, ref["out"], 1e-5)


# bf16 layers with the router GEMV in the path: logits within 1e-5 of the
# oracle's, routing bit-exact on the device's own logits
ROUTER_BF16 = [
    # name, T, d, E, k, f
    ("router_bf16_t1", 1, 6144, 256, 8, 256),      # the real router shape, single token
    ("router_bf16_t16", 16, 6144, 256, 8, 256),
    ("router_bf16_t37", 37, 512, 64, 8, 256),
    ("router_bf16_t300", 300, 320, 24, 6, 128),    # grouped GEMM path
]


@pytest.mark.parametrize("case", ROUTER_BF16, ids=[c[0] for c in ROUTER_BF16])
def test_layer_bf16_router(case):
    name, T, d, E, k, f = case
    log(f"layer {name}")
    wl = Workload(name, T=T, d=d, E=E, k=k, f=f, act="bf16", wfmt="bf16", router=True,
                  seed=zlib.crc32(name.encode()) % 100000,
                  x_std=1.0, wg_std=d ** -0.5, wu_std=d ** -0.5, wd_std=f ** -0.5)
    x, w, w_r, logits = make_inputs(wl)
    assert w_r is not None and w_r.dtype == torch.bfloat16 and logits is None
    got, ref, res = run_layer_and_oracle(wl, x, w, w_r, logits)
    lg = res["logits"].cpu().numpy().astype(np.float64)
    lerr = rel_l2(lg, oracle.router_logits(to_host_act(x), to_host_act(w_r)))
    record(name + ":logits", rel_l2=lerr, tol=1e-5)
    check_out(name, got, ref["out"], 5e-3)


def test_layer_k_equals_E_uniform_is_dense_mixture():
    """k=E with equal logits: the device output equals (1/E) sum_e FFN_e."""
    wl = Workload("dense_mix", T=4, d=128, E=8, k=8, f=64, act="f32", wfmt="f32", seed=99,
                  x_std=1.0, wg_std=0.1, wu_std=0.1, wd_std=0.1)
    x, w, _, _ = make_inputs(wl)
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    res = moe_layer_forward(x, w, 8, logits=torch.zeros(4, 8, device="cuda"))
    torch.cuda.synchronize()
    xh = to_host_act(x)
    get = expert_getter(w, "f32")
    dense = sum(oracle.swiglu_expert(xh, *get(e)) for e in range(8)) / 8
    check_out("dense_mix", to_host_act(res["out"]), dense, 1e-5)


def test_determinism_and_t0():
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    wl = Workload("det", T=16, d=512, E=32, k=8, f=160, act="bf16", wfmt="bf16", seed=5)
    x, w, _, logits = make_inputs(wl)
    a = moe_layer_forward(x, w, 8, logits=logits)["out"].clone()
    b = moe_layer_forward(x, w, 8, logits=logits)["out"].clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    wl2 = Workload("det2", T=300, d=256, E=16, k=4, f=96, act="bf16", wfmt="mxfp4", seed=6)
    x, w, _, logits = make_inputs(wl2)
    a = moe_layer_forward(x, w, 4, logits=logits)["out"].clone()
    b = moe_layer_forward(x, w, 4, logits=logits)["out"].clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # T = 0 is a no-op
    e = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    r = moe_layer_forward(e, w, 4, logits=torch.empty(0, 16, device="cuda"))
    assert r["out"].shape == (0, 256)


@pytest.mark.parametrize("wfmt,k,f,d", [("bf16", 8, 352, 1024), ("mxfp4", 8, 352, 1024), ("nvfp4", 8, 352, 1024),
                                        ("f32", 4, 352, 1024), ("bf16", 16, 352, 1024), ("bf16", 8, 2816, 1024),
                                        ("f32", 4, 1024, 1024), ("bf16", 12, 2048, 1024),
                                        ("mxfp4", 8, 2816, 1024), ("nvfp4", 6, 1408, 1024),
                                        ("mxfp4", 4, 4096, 1024),
                                        # bf16 rows split four ways, routing inside the gate/up kernel
                                        ("bf16", 8, 704, 4096), ("bf16", 16, 352, 6144),
                                        ("bf16", 3, 128, 3104)])
def test_single_token_fused_path_equals_stagewise(wfmt, k, f, d):
    """The single-token layer (fused down+combine) is bit-identical to
    route -> permute -> expert_ffn -> combine called one by one, for short
    and full-width down rows and for k up to 16."""
    from expert_ffn_layer_softmax_amd import (moe_combine, moe_expert_ffn, moe_layer_forward,
                                              moe_permute, moe_route)
    act = "f32" if wfmt == "f32" else "bf16"
    wl = Workload("t1eq", T=1, d=d, E=32, k=k, f=f, act=act, wfmt=wfmt, seed=31 + k,
                  x_std=1.0, wg_std=d ** -0.5, wu_std=d ** -0.5, wd_std=f ** -0.5)
    x, w, _, logits = make_inputs(wl)
    fused = moe_layer_forward(x, w, k, logits=logits)["out"]
    idx, tw = moe_route(logits, k)
    counts, offsets, sorted_src, dest_row = moe_permute(idx, wl.E)
    y = moe_expert_ffn(x, offsets, sorted_src, k, w)
    staged = moe_combine(y, dest_row, tw, x.dtype)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16) if act == "bf16" else fused.view(torch.int32),
                       staged.view(torch.int16) if act == "bf16" else staged.view(torch.int32))


# ------------------------------------------------- FP8 activations (MXFP8)
# Both sides quantise x and h to MXFP8; they differ by fp32 vs fp64
# accumulation and, rarely, an FP8 rounding decision that the accumulation
# difference moves across a boundary, so the bf16 tolerance applies.
FP8_CASES = [
    # name, T, d, E, k, f, weights (MX-FP4: scaled MFMA; NVFP4: bf16 MFMA on
    # MXFP8-valued activations, the pages' own FP8 + NVFP4 pairing)
    ("fp8_t1", 1, 256, 16, 4, 256, "mxfp4"),
    ("fp8_t16", 16, 512, 32, 8, 256, "mxfp4"),
    ("fp8_t100", 100, 256, 8, 4, 512, "mxfp4"),
    ("fp8_hot", 700, 512, 5, 2, 512, "mxfp4"),       # several m-tiles per expert
    ("fp8_tails", 150, 768, 6, 2, 256, "mxfp4"),     # 3 down n-tiles, ragged m-tiles
    ("fp8nv_t1", 1, 256, 16, 4, 256, "nvfp4"),
    ("fp8nv_t16", 16, 512, 32, 8, 256, "nvfp4"),
    ("fp8nv_t100", 100, 256, 8, 4, 512, "nvfp4"),
    ("fp8nv_hot", 700, 512, 5, 2, 512, "nvfp4"),
    ("fp8nv_tails", 150, 768, 6, 2, 768, "nvfp4"),   # partial n-tiles on both GEMMs
]


@pytest.mark.parametrize("case", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_layer_fp8_activations(case):
    name, T, d, E, k, f, wfmt = case
    log(f"fp8 layer {name}")
    wl = Workload(name, T=T, d=d, E=E, k=k, f=f, act="bf16", wfmt=wfmt,
                  seed=zlib.crc32(name.encode()) % 100000,
                  x_std=1.0, wg_std=d ** -0.5, wu_std=d ** -0.5, wd_std=f ** -0.5)
    x, w, w_r, logits = make_inputs(wl)
    got, ref, _ = run_layer_and_oracle(wl, x, w, w_r, logits, fp8=True)
    check_out(name, got, ref["out"], 5e-3, token_tol=FP8_TOKEN_TOL)
    # the FP8 rounding is real: the bf16-activation result differs by about 2-4 %
    plain = oracle.layer(to_host_act(x), logits.cpu().numpy(), k, expert_getter(w, wfmt), E=E)
    sep = rel_l2(plain["out"], ref["out"])
    log(f"  bf16-activation reference differs by {sep:.3e}")
    assert sep > 5e-3


# ------------------------------------------- RMS-normalised expert outputs
# MOE_FLAG_EXPERT_NORM on every path: the fused single-token kernel is
# bypassed, the GEMV and grouped-GEMM paths feed the normalising combine.
NORM_CASES = [
    # name, T, d, E, k, f, act, wfmt, fp8
    ("norm_t1_bf16", 1, 512, 32, 8, 160, "bf16", "bf16", False),
    ("norm_t1_f32", 1, 128, 8, 3, 64, "f32", "f32", False),
    ("norm_t1_mx", 1, 512, 32, 8, 256, "bf16", "mxfp4", False),          # routing inside gate/up
    ("norm_t1_bf16_long", 1, 4096, 16, 4, 256, "bf16", "bf16", False),   # rows split four ways
    ("norm_t16_mx", 16, 512, 32, 8, 256, "bf16", "mxfp4", False),
    ("norm_t40_nv", 40, 256, 8, 2, 128, "bf16", "nvfp4", False),
    ("norm_gg_bf16", 300, 512, 16, 4, 384, "bf16", "bf16", False),
    ("norm_gg_mx_k20", 90, 640, 32, 20, 256, "bf16", "mxfp4", False),   # 5 slots per wave
    ("norm_fp8", 100, 256, 8, 4, 512, "bf16", "mxfp4", True),
    ("norm_fp8_nv", 100, 256, 8, 4, 512, "bf16", "nvfp4", True),
]


@pytest.mark.parametrize("case", NORM_CASES, ids=[c[0] for c in NORM_CASES])
def test_layer_expert_norm(case):
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    name, T, d, E, k, f, act, wfmt, fp8 = case
    log(f"expert-norm layer {name}")
    wl = Workload(name, T=T, d=d, E=E, k=k, f=f, act=act, wfmt=wfmt,
                  seed=zlib.crc32(name.encode()) % 100000,
                  x_std=1.0, wg_std=d ** -0.5, wu_std=d ** -0.5, wd_std=f ** -0.5)
    x, w, _, logits = make_inputs(wl)
    res = moe_layer_forward(x, w, k, logits=logits, fp8=fp8, expert_norm=True)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    check_routing(res, lg, k, E)
    aq = oracle.quantize_mxfp8 if fp8 else None
    get = expert_getter(w, wfmt)
    ref = oracle.layer(to_host_act(x), lg, k, get, E=E, act_quant=aq, expert_norm=True)
    plain = oracle.layer(to_host_act(x), lg, k, get, E=E, act_quant=aq)
    check_out(name, to_host_act(res["out"]), ref["out"],
              1e-5 if act == "f32" else 5e-3 if wfmt == "bf16" or fp8 else _tol(wl),
              token_tol=FP8_TOKEN_TOL if fp8 else None)
    sep = rel_l2(plain["out"], ref["out"])
    log(f"  unnormalised reference differs by {sep:.3e}")
    assert sep > 0.1


@pytest.mark.parametrize("act,d,k,T", [("f32", 64, 1, 37), ("f32", 320, 6, 37), ("bf16", 6144, 8, 37),
                                       ("bf16", 1024, 64, 37), ("f32", 704, 5, 300),
                                       ("bf16", 6144, 8, 260), ("bf16", 1024, 12, 300),
                                       ("f32", 8448, 4, 20), ("f32", 8448, 4, 256),
                                       ("bf16", 64, 1, 400)])
def test_combine_expert_norm_entry_point(act, d, k, T):
    """moe_combine with the flag on the device's own y_sorted, against the
    oracle's fp64 combine within the fp32 error bound of the norm and sum.
    Cases cover the register-resident kernel (T >= 256, k <= 8, d <= 8192;
    256 and 1024 threads) and the two-pass kernel (T < 256, or k > 8, or
    d > 8192; 1024 and 256 threads)."""
    from expert_ffn_layer_softmax_amd import moe_combine, moe_permute, moe_route
    E = max(k, 8)
    g = torch.Generator().manual_seed(d + k + T)
    logits = torch.randn(T, E, generator=g).cuda()
    idx, tw = moe_route(logits, k)
    _, _, _, dest_row = moe_permute(idx, E)
    # rows of very different scales (the norm removes them) and one zero row
    scale = torch.exp2(torch.randint(-20, 20, (T * k, 1), generator=g).float())
    y = torch.randn(T * k, d, generator=g) * scale
    y[3] = 0.0
    y = y.cuda()
    dt = torch.float32 if act == "f32" else torch.bfloat16
    out = moe_combine(y, dest_row, tw, dt, expert_norm=True)
    torch.cuda.synchronize()
    yh = y.cpu().numpy().astype(np.float64)
    rd = dest_row.cpu().numpy()
    twh = tw.cpu().numpy().astype(np.float64)
    rout = oracle.combine(yh, rd, twh, expert_norm=True)
    got = to_host_act(out)
    # per-row weight w/r: sum of squares of at most d/64 sequential terms per
    # lane, a 6-level wave tree and at most 16 wave partials (all terms >= 0),
    # a root and a division; then the fp32 sum of k products, and for bf16 one
    # rounding
    mag = oracle.combine(np.abs(yh), rd, np.abs(twh), expert_norm=True)
    u = 2.0 ** -24
    bound = ((k + 1) + (d / 64 + 6 + 16) / 2 + 3) * u * mag + 1e-30
    if act == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(rout)
    assert np.all(np.abs(got - rout) <= bound), float(np.max(np.abs(got - rout) / bound))


# ------------------------------------------------- load and shape extremes
EXTREMES = [
    # name, T, d, E, k, f, wfmt, logits: "hot" (every token picks the same k
    # experts), "rand"
    ("all_to_k_experts_bf16", 4096, 256, 64, 8, 128, "bf16", "hot"),    # 32 m-tiles per expert
    ("all_to_k_experts_mx", 4096, 256, 64, 8, 128, "mxfp4", "hot"),
    ("one_expert_bf16", 300, 256, 1, 1, 128, "bf16", "rand"),           # E = k = 1
    ("one_expert_mx", 300, 256, 1, 1, 256, "mxfp4", "rand"),
    ("k_is_E_64", 100, 128, 64, 64, 64, "bf16", "rand"),                # largest k: dense mixture
    ("min_gemm_shape", 64, 64, 4, 2, 64, "bf16", "rand"),               # d = f = 64 on the MFMA path
    ("many_tokens_small", 20000, 64, 16, 2, 64, "bf16", "rand"),
    ("many_experts_gg_bf16", 256, 256, 1024, 8, 256, "bf16", "rand"),   # ~2 rows per expert: 1024 tiny m-tiles
    ("many_experts_gg_mx", 256, 256, 1024, 8, 256, "mxfp4", "rand"),
]


@pytest.mark.parametrize("case", EXTREMES, ids=[c[0] for c in EXTREMES])
def test_routing_and_shape_extremes(case):
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    name, T, d, E, k, f, wfmt, mode = case
    log(f"extreme {name}")
    wl = Workload(name, T=T, d=d, E=E, k=k, f=f, act="bf16", wfmt=wfmt,
                  seed=zlib.crc32(name.encode()) % 100000,
                  x_std=1.0, wg_std=d ** -0.5, wu_std=d ** -0.5, wd_std=f ** -0.5)
    x, w, _, logits = make_inputs(wl)
    if mode == "hot":
        hot = torch.tensor([3, 17, 29, 30, 41, 50, 58, 63][:k], device=logits.device)
        logits[:, hot] += 100.0
    res = moe_layer_forward(x, w, k, logits=logits)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    check_routing(res, lg, k, E)
    if mode == "hot":
        assert set(np.unique(res["topk_idx"].cpu().numpy()).tolist()) == set(hot.cpu().tolist())
    ref = oracle.layer(to_host_act(x), lg, k, expert_getter(w, wfmt), E=E)
    check_out(name, to_host_act(res["out"]), ref["out"], 5e-3 if wfmt == "bf16" else MXFP4_TOL)


@pytest.mark.parametrize("wfmt", ["mxfp4", "bf16"])
def test_tile_height_edges(wfmt):
    """Experts with exactly 1, 128, 129, 256, 257 and 383 rows (k = 1, each
    token sent to a chosen expert in shuffled order): the boundaries between
    one and two 128-row m-tiles and between the MX-FP4 tiles of up to 128
    and of 129..256 rows."""
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    counts = [128, 129, 256, 257, 1, 383]
    E, k, d, f = len(counts), 1, 512, 512
    T = sum(counts)
    name = f"tile_edges_{wfmt}"
    log(f"tile edges {wfmt}: counts {counts}")
    wl = Workload(name, T=T, d=d, E=E, k=k, f=f, act="bf16", wfmt=wfmt, seed=zlib.crc32(name.encode()) % 100000,
                  x_std=1.0, wg_std=d ** -0.5, wu_std=d ** -0.5, wd_std=f ** -0.5)
    x, w, _, logits = make_inputs(wl)
    target = np.repeat(np.arange(E), counts)
    np.random.default_rng(5).shuffle(target)
    logits[torch.arange(T, device=logits.device), torch.from_numpy(target).to(logits.device)] += 100.0
    res = moe_layer_forward(x, w, k, logits=logits)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    check_routing(res, lg, k, E)
    assert np.bincount(res["topk_idx"].cpu().numpy().ravel(), minlength=E).tolist() == counts
    ref = oracle.layer(to_host_act(x), lg, k, expert_getter(w, wfmt), E=E)
    check_out(name, to_host_act(res["out"]), ref["out"], 5e-3 if wfmt == "bf16" else MXFP4_TOL)


def _random_fp4_weights(wfmt, E, d, f, seed):
    """Expert weights whose bytes cover the format's domain: codes uniform
    over all 16 nibbles; NVFP4 block scales uniform over every E4M3 byte but
    the two NaNs (so zero, subnormal, negative and the largest scales occur),
    matrix scales in [0.25, 4); MX-FP4 scales uniform over E8M0 bytes
    110..144 (2^-17 .. 2^17: a wide range with no fp32 overflow in the
    layer)."""
    g = torch.Generator().manual_seed(seed)
    shapes = dict(gate=(E, f, d), up=(E, f, d), down=(E, d, f))
    w = {}
    for n, (a, b, K) in shapes.items():
        w["w_" + n] = torch.randint(0, 256, (a, b, K // 2), generator=g, dtype=torch.uint8)
        if wfmt == "nvfp4":
            r = torch.randint(0, 254, (a, b, K // 16), generator=g, dtype=torch.int32)
            w["s_" + n] = (r + (r >= 0x7F).to(torch.int32)).to(torch.uint8).view(torch.float8_e4m3fn)
            w["t_" + n] = 0.25 + 3.75 * torch.rand(a, generator=g)
        else:
            w["s_" + n] = torch.randint(110, 145, (a, b, K // 32), generator=g, dtype=torch.uint8)
    return {key: v.cuda() for key, v in w.items()}


@pytest.mark.parametrize("wfmt,T", [("nvfp4", 1), ("nvfp4", 16), ("nvfp4", 200),
                                    ("mxfp4", 1), ("mxfp4", 16), ("mxfp4", 200)])
def test_fp4_scale_byte_domain(wfmt, T):
    """4-bit weights over the whole code and scale domain (not only what the
    quantiser of the synthetic weights produces), on the single-token kernels,
    the GEMV path and the grouped MFMA path (T = 200, K % 256 == 0)."""
    name = f"scale_domain_{wfmt}_T{T}"
    log(name)
    d, f, E, k = 512, 512, 8, 2
    wl = Workload(name, T=T, d=d, E=E, k=k, f=f, act="bf16", wfmt=wfmt, seed=zlib.crc32(name.encode()) % 100000,
                  x_std=1.0)
    w = _random_fp4_weights(wfmt, E, d, f, wl.seed)
    if wfmt == "nvfp4":
        s8 = torch.cat([w["s_" + n].view(torch.uint8).flatten() for n in ("gate", "up", "down")]).cpu()
        present = set(torch.unique(s8).tolist())
        assert 0x7F not in present and 0xFF not in present and len(present) == 254
    x, w, _, logits = make_inputs(wl, weights=w)
    got, ref, _ = run_layer_and_oracle(wl, x, w, None, logits)
    check_out(name, got, ref["out"], MXFP4_TOL)


@pytest.mark.parametrize("wfmt,T,fp8", [("bf16", 16, False), ("bf16", 200, False), ("mxfp4", 16, False),
                                        ("mxfp4", 200, False), ("nvfp4", 200, False), ("mxfp4", 200, True)])
def test_nan_token_is_isolated(wfmt, T, fp8):
    """Tokens are independent: a NaN in one token's activations makes that
    token's whole output NaN and leaves every other token as the oracle
    computes it, on the GEMV and the grouped MFMA paths (where other rows of
    the NaN token's tiles, and padding rows copied from it, share its
    blocks)."""
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    name = f"nan_token_{wfmt}_T{T}{'_fp8' if fp8 else ''}"
    log(name)
    d, f, E, k = 512, 512, 8, 4
    wl = Workload(name, T=T, d=d, E=E, k=k, f=f, act="bf16", wfmt=wfmt, seed=zlib.crc32(name.encode()) % 100000,
                  x_std=1.0, wg_std=d ** -0.5, wu_std=d ** -0.5, wd_std=f ** -0.5)
    x, w, _, logits = make_inputs(wl)
    bad = T // 3
    x[bad, 17] = float("nan")
    res = moe_layer_forward(x, w, k, logits=logits, fp8=fp8)
    torch.cuda.synchronize()
    out = to_host_act(res["out"])
    assert np.isnan(out[bad]).all(), "the NaN token's output is not all NaN"
    keep = np.array([t for t in range(T) if t != bad])
    assert not np.isnan(out[keep]).any(), "NaN reached another token"
    lg = logits.cpu().numpy()
    check_routing(res, lg, k, E)
    ref = oracle.layer(to_host_act(x)[keep], lg[keep], k, expert_getter(w, wfmt), E=E,
                       act_quant=oracle.quantize_mxfp8 if fp8 else None)
    check_out(name, out[keep], ref["out"], MXFP4_TOL if wfmt != "bf16" else 5e-3,
              token_tol=FP8_TOKEN_TOL if fp8 else None)


@pytest.mark.parametrize("T", [1, 64])
def test_mx_nan_scale_propagates(T):
    """An E8M0 scale byte of 255 is NaN (OCP MX): the output columns that use
    that weight block are NaN on the device as in the oracle, and all other
    values still match.  T=1 takes the GEMV kernels, T=64 the grouped GEMM."""
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    wl = Workload(f"mx_nan_t{T}", T=T, d=256, E=4, k=2, f=256, act="bf16", wfmt="mxfp4", seed=77 + T,
                  x_std=1.0, wg_std=256 ** -0.5, wu_std=256 ** -0.5, wd_std=256 ** -0.5)
    x, w, _, logits = make_inputs(wl)
    logits[:, 1] += 50.0  # every token uses expert 1
    w["s_down"][1, 7, 3] = 255  # W_down row 7 (output column 7), K-block 3
    res = moe_layer_forward(x, w, wl.k, logits=logits)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    check_routing(res, lg, wl.k, wl.E)
    with np.errstate(invalid="ignore"):
        ref = oracle.layer(to_host_act(x), lg, wl.k, expert_getter(w, "mxfp4"), E=wl.E)["out"]
    got = to_host_act(res["out"])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(ref[:, 7]).all() and not np.isnan(np.delete(ref, 7, axis=1)).any()
    cols = ~np.isnan(ref).any(axis=0)
    check_out(f"mx_nan_t{T}", got[:, cols], ref[:, cols], MXFP4_TOL)


# ------------------------------------------------------------ HIP graphs
@pytest.mark.parametrize("T,wfmt", [(1, "bf16"), (16, "bf16"), (100, "bf16"), (100, "mxfp4"),
                                    (100, "nvfp4"), (100, "mxfp4_fp8"), (100, "nvfp4_fp8")])
def test_hip_graph_replay(T, wfmt):
    """A captured layer replays to the eager result, bit for bit, after eager
    calls with other routing have rewritten the same workspace and outputs."""
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    log(f"graph T={T} {wfmt}")
    fp8 = wfmt.endswith("_fp8")
    wfmt = wfmt[:-4] if fp8 else wfmt
    k = 8
    wl = Workload("graph", T=T, d=512, E=32, k=k, f=256, act="bf16", wfmt=wfmt, seed=71 + T,
                  x_std=1.0, wg_std=512 ** -0.5, wu_std=512 ** -0.5, wd_std=256 ** -0.5)
    x, w, _, logits = make_inputs(wl)
    other_logits = torch.randn(T, wl.E, generator=torch.Generator().manual_seed(T)).cuda()
    eager = moe_layer_forward(x, w, k, logits=logits, fp8=fp8)
    ref_out, ref_idx = eager["out"].clone(), eager["topk_idx"].clone()
    ws = eager["workspace"]
    out = torch.empty_like(ref_out)
    idx = torch.empty_like(ref_idx)
    tw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe_layer_forward(x, w, k, logits=logits, topk_idx=idx, topk_w=tw, out=out, workspace=ws, fp8=fp8)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe_layer_forward(x, w, k, logits=logits, topk_idx=idx, topk_w=tw, out=out, workspace=ws, fp8=fp8)
    torch.cuda.synchronize()
    for _ in range(3):
        moe_layer_forward(x, w, k, logits=other_logits, topk_idx=idx, topk_w=tw, out=out, workspace=ws, fp8=fp8)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))


# --------------------------------------------------- individual entry points
@pytest.mark.parametrize("wfmt,T", [("bf16", 7), ("bf16", 64), ("mxfp4", 23), ("nvfp4", 64), ("f32", 9)])
def test_stagewise_entry_points(wfmt, T):
    from expert_ffn_layer_softmax_amd import moe_combine, moe_expert_ffn, moe_permute, moe_route
    act = "f32" if wfmt == "f32" else "bf16"
    wl = Workload("stages", T=T, d=320, E=24, k=6, f=192, act=act, wfmt=wfmt, seed=T,
                  x_std=1.0, wg_std=320 ** -0.5, wu_std=320 ** -0.5, wd_std=192 ** -0.5)
    log(f"stages {wfmt} T={T}")
    x, w, _, logits = make_inputs(wl)
    idx, tw = moe_route(logits, wl.k)
    counts, offsets, sorted_src, dest_row = moe_permute(idx, wl.E)
    y = moe_expert_ffn(x, offsets, sorted_src, wl.k, w)
    out = moe_combine(y, dest_row, tw, x.dtype)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    ridx, rw = oracle.route(lg, wl.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    rc, ro, rs, rd = oracle.permute(ridx, wl.E)
    assert np.array_equal(offsets.cpu().numpy(), ro) and np.array_equal(sorted_src.cpu().numpy(), rs)
    assert np.array_equal(dest_row.cpu().numpy(), rd) and np.array_equal(counts.cpu().numpy(), rc)
    xh = to_host_act(x)
    ry = oracle.expert_ffn(xh, ro, rs, wl.k, expert_getter(w, wfmt))
    yh = y.cpu().numpy().astype(np.float64)
    check_out(f"stages_{wfmt}_T{T}:y_sorted", yh, ry, _tol(wl))   # every row of y_sorted
    # combine alone: fp32 sum of the device's own y_sorted, rounded once
    twh = tw.cpu().numpy().astype(np.float64)
    rout = oracle.combine(yh, rd, twh)
    got = to_host_act(out)
    # fp32 accumulation of k products: |err| <= (k+1) u32 sum_j |w_j y_j|;
    # bf16 output adds one rounding, |err| <= 2^-8 |value|
    mag = oracle.combine(np.abs(yh), rd, np.abs(twh))
    bound = (wl.k + 1) * 2.0 ** -24 * mag
    if act == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(rout)
    assert np.all(np.abs(got - rout) <= bound)


# ------------------------------------------------------- full-size workloads
@pytest.fixture(scope="module")
def full_bf16_weights():
    wl = WORKLOADS["decode_bf16"]
    log("generating full bf16 expert weights (26.6 GB)")
    w = gen_expert_weights(wl, "cuda")
    torch.cuda.synchronize()
    yield w
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("logit_set", [0, 17, 63])
def test_decode_bf16_full(full_bf16_weights, logit_set):
    wl = WORKLOADS["decode_bf16"]
    log(f"decode_bf16 full, logit set {logit_set}")
    x, w, w_r, logits = make_inputs(wl, weights=full_bf16_weights, logit_set=logit_set)
    got, ref, _ = run_layer_and_oracle(wl, x, w, w_r, logits)
    check_out(f"decode_bf16_full_set{logit_set}", got, ref["out"], 5e-3)


def test_verify_bf16_full(full_bf16_weights):
    wl = WORKLOADS["verify_bf16"]
    log("verify_bf16 full (T=16)")
    x, w, w_r, logits = make_inputs(wl, weights=full_bf16_weights, logit_set=5)
    got, ref, _ = run_layer_and_oracle(wl, x, w, w_r, logits)
    log(f"  unique experts={int((ref['counts'] > 0).sum())}")
    check_out("verify_bf16_full", got, ref["out"], 5e-3)


def _oracle_on_tokens(x, lg, k, w, wfmt, E, S, act_quant=None, expert_norm=False):
    """oracle.layer on the tokens S (the layer is per-token independent), with
    the experts those tokens use decoded ahead on host threads."""
    idx, _ = oracle.route(lg[S], k)
    get = PrefetchGetter(expert_getter(w, wfmt), sorted(set(idx.ravel().tolist())))
    try:
        return oracle.layer(to_host_act(x)[S], lg[S], k, get, E=E, act_quant=act_quant,
                            expert_norm=expert_norm)
    finally:
        get.close()


@pytest.mark.parametrize("name", ["prefill_bf16", "prefill_mxfp4", "prefill_nvfp4", "prefill_mxfp4_fp8",
                                  "prefill_nvfp4_fp8"])
def test_prefill_full_stratified(name, full_bf16_weights):
    """T=4096 with skewed load, in the bench's launch configuration: routing
    checked in full; outputs on every token that owns the first or last row
    of an expert's segment or a row either side of an m-tile boundary (so
    every expert's ragged last m-tile), plus random tokens, each over all d
    columns (every column-tile edge)."""
    fp8 = name.endswith("_fp8")
    wl = WORKLOADS[name[:-4] if fp8 else name]
    log(f"{name} full (T=4096), stratified tokens")
    w = full_bf16_weights if wl.wfmt == "bf16" else gen_expert_weights(wl, "cuda")
    x, w, w_r, logits = make_inputs(wl, weights=w)
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    res = moe_layer_forward(x, w, wl.k, logits=logits, fp8=fp8)
    torch.cuda.synchronize()
    lg = res["logits"].cpu().numpy()
    idx, _ = check_routing(res, lg, wl.k, wl.E)
    counts = np.bincount(idx.ravel(), minlength=wl.E)
    log(f"  expert load: min {counts.min()} mean {counts.mean():.0f} max {counts.max()}")
    S = stratified_tokens(idx, wl.E)
    log(f"  {S.size} tokens cover {int((counts > 0).sum())} experts' segment edges")
    ref = _oracle_on_tokens(x, lg, wl.k, w, wl.wfmt, wl.E, S,
                            act_quant=oracle.quantize_mxfp8 if fp8 else None)
    got = to_host_act(res["out"])[S]
    check_out(name + "_full", got, ref["out"],
              MXFP4_TOL if wl.wfmt in ("mxfp4", "nvfp4") and not fp8 else 5e-3, tokens=S,
              token_tol=FP8_TOKEN_TOL if fp8 else None)
    if wl.wfmt != "bf16":
        del w
        torch.cuda.empty_cache()


@pytest.mark.parametrize("wfmt", ["bf16", "mxfp4"])
def test_prefill_tp8_shard_width_stratified(wfmt):
    """One GPU's tensor-parallel share at G = 8: f = 2816/8 = 352, a K tail of
    32 in the down projection and a 96-column n-tile in gate/up, at T=4096."""
    base = WORKLOADS["prefill_bf16"]
    wl = Workload(f"prefill_{wfmt}_f352", T=base.T, d=base.d, E=base.E, k=base.k, f=352, act="bf16",
                  wfmt=wfmt, seed=base.seed + 11, logit_sets=1, bias_std=base.bias_std,
                  x_std=1.0, wg_std=base.d ** -0.5, wu_std=base.d ** -0.5, wd_std=352 ** -0.5)
    log(f"prefill {wfmt} f=352 (T=4096), stratified tokens")
    x, w, _, logits = make_inputs(wl)
    from expert_ffn_layer_softmax_amd import moe_layer_forward, moe_timing_query, moe_timing_start, \
        moe_timing_stop
    moe_timing_start()
    res = moe_layer_forward(x, w, wl.k, logits=logits)
    torch.cuda.synchronize()
    moe_timing_stop()
    assert moe_timing_query("gg_down")[0] == 1, "the grouped GEMM path must take f = 352"
    lg = res["logits"].cpu().numpy()
    idx, _ = check_routing(res, lg, wl.k, wl.E)
    S = stratified_tokens(idx, wl.E)
    ref = _oracle_on_tokens(x, lg, wl.k, w, wfmt, wl.E, S)
    check_out(wl.name, to_host_act(res["out"])[S], ref["out"], 5e-3 if wfmt == "bf16" else MXFP4_TOL,
              tokens=S)
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode_mxfp4", "decode_nvfp4"])
def test_decode_fp4_full(name):
    wl = WORKLOADS[name]
    log(f"generating full {wl.wfmt} expert weights")
    w = gen_expert_weights(wl, "cuda")
    for s in (0, 9):
        x, w, w_r, logits = make_inputs(wl, weights=w, logit_set=s)
        got, ref, _ = run_layer_and_oracle(wl, x, w, w_r, logits)
        check_out(f"{name}_full_set{s}", got, ref["out"], MXFP4_TOL)
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode_mxfp4", "prefill_bf16"])
def test_ep8_share(name):
    """One GPU's expert-parallel share at G = 8, as the bench's ep8 share times
    it: E/8 = 32 local experts, each of the T*k/8 dispatched rows routed to one
    of them (k = 1), at the real d and f; decode in full, prefill on the
    stratified tokens."""
    import dataclasses
    base = WORKLOADS[name]
    wl = dataclasses.replace(base, E=base.E // 8, k=1, T=max(1, base.T * base.k // 8),
                             name=f"{name}_ep8_share", logit_sets=1)
    log(f"{wl.name}: T={wl.T} E={wl.E} k=1 d={wl.d} f={wl.f} {wl.wfmt}")
    x, w, w_r, logits = make_inputs(wl)
    if wl.T <= 16:
        got, ref, res = run_layer_and_oracle(wl, x, w, w_r, logits)
        check_out(wl.name, got, ref["out"], _tol(wl))
    else:
        from expert_ffn_layer_softmax_amd import moe_layer_forward
        res = moe_layer_forward(x, w, wl.k, logits=logits)
        torch.cuda.synchronize()
        lg = res["logits"].cpu().numpy()
        idx, _ = check_routing(res, lg, wl.k, wl.E)
        S = stratified_tokens(idx, wl.E)
        ref = _oracle_on_tokens(x, lg, wl.k, w, wl.wfmt, wl.E, S)
        check_out(wl.name, to_host_act(res["out"])[S], ref["out"], _tol(wl), tokens=S)
    del w, res
    torch.cuda.empty_cache()


def test_prefill_expert_norm_full_stratified(full_bf16_weights):
    """T=4096 with MOE_FLAG_EXPERT_NORM: the grouped GEMMs feed the
    register-resident normalising combine at the real d and k."""
    from expert_ffn_layer_softmax_amd import moe_layer_forward
    wl = WORKLOADS["prefill_bf16"]
    log("prefill_bf16 full (T=4096) with per-expert RMS normalisation, stratified tokens")
    x, w, _, logits = make_inputs(wl, weights=full_bf16_weights)
    res = moe_layer_forward(x, w, wl.k, logits=logits, expert_norm=True)
    torch.cuda.synchronize()
    lg = res["logits"].cpu().numpy()
    idx, _ = check_routing(res, lg, wl.k, wl.E)
    S = stratified_tokens(idx, wl.E, extra=4)[::3]   # a third of them: two oracle passes
    ref = _oracle_on_tokens(x, lg, wl.k, w, wl.wfmt, wl.E, S, expert_norm=True)
    plain = oracle.combine(ref["y_sorted"], ref["dest_row"], ref["w"])
    check_out("prefill_bf16_expert_norm_full", to_host_act(res["out"])[S], ref["out"], 5e-3, tokens=S)
    sep = rel_l2(plain, ref["out"])
    log(f"  unnormalised combine differs by {sep:.3e}")
    assert sep > 0.1


# ---------------------------------------------------- MXFP8 quantisation
@pytest.mark.parametrize("rows,K", [(1, 32), (5, 256), (4096, 6144), (333, 2816), (64, 96)])
def test_quantize_mxfp8_bit_exact(rows, K):
    """The FP8 path's activation quantisation is byte work: the device's E4M3
    codes and E8M0 scales, decoded, equal oracle.quantize_mxfp8 of the same
    bf16 input exactly (NaN where the oracle has NaN).  Inputs span 2^-30 ..
    2^30 per block, with zero blocks, NaN elements, bf16 subnormals and values
    on rounding ties."""
    from expert_ffn_layer_softmax_amd import moe_quantize_mxfp8
    g = torch.Generator().manual_seed(rows * 7 + K)
    v = torch.randn(rows, K, generator=g)
    # one power-of-two magnitude per 32-element block
    v = v * torch.exp2(torch.randint(-30, 30, (rows, K // 32), generator=g).float()).repeat_interleave(32, dim=1)
    if rows * K >= 256:
        v.view(-1)[::97] = float("nan")
        v[0, :32] = 0.0                                     # an all-zero block
        v.view(-1)[5::211] = 2.0 ** -130                    # bf16 subnormals among normals
        if K >= 64:
            # a block whose scale is 2^0 (amax 256): 1 + 1/16 is the tie of
            # E4M3 neighbours 1 and 1.125, 3 + 1/8 that of 3 and 3.25 (both
            # round to the even neighbour)
            v[-1, 32:64] = torch.tensor([256.0] + [1.0 + 1.0 / 16] * 15 + [3.0 + 1.0 / 8] * 16)
        if rows >= 2 and K >= 64:
            # a block of bf16 subnormals only: amax 2^-129, scale clamped to 2^-126
            v[1, 32:64] = (torch.arange(32) - 16).float() * 2.0 ** -133
    x = v.to(torch.bfloat16).cuda()
    q, sc = moe_quantize_mxfp8(x)
    torch.cuda.synchronize()
    xh = to_host_act(x)
    got = (oracle.decode_e4m3(q.cpu().numpy()).reshape(rows, K // 32, 32)
           * oracle.decode_e8m0(sc.cpu().numpy())[..., None]).reshape(rows, K)
    ref = oracle.quantize_mxfp8(xh)
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"NaN positions differ ({nan_g.sum()} vs {nan_r.sum()})"
    assert np.array_equal(got[~nan_g], ref[~nan_r]), \
        f"{int((got[~nan_g] != ref[~nan_r]).sum())} of {got.size} quantised values differ"
    record(f"quantize_mxfp8_{rows}x{K}", mismatches=0, values=int(got.size))
