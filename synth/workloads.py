"""Workload shapes and seeded generators.

The pages measure whole models on real prompts (single-request decode, 4K-token
prefill, 4 concurrent requests, speculative verification) which cannot be
reproduced here.  A layer's cost depends only on the token count and on where
the router sends the tokens, so each workload below is a synthetic stand-in
with that shape: activations and weights ~ N(0, 0.02^2), router logits
~ N(0, 1) (uniform expected load), plus a fixed per-expert bias ~ N(0, 0.5^2)
for the skewed prefill load.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    f: int
    act: str            # "f32" | "bf16"
    wfmt: str           # "f32" | "bf16" | "mxfp4" | "nvfp4"
    router: bool = False        # logits computed from x and W_r inside the layer
    logit_sets: int = 1         # pre-generated logit sets, rotated per call
    bias_std: float = 0.0       # per-expert logit bias (skewed load)
    x_std: float = 0.02
    wg_std: float = 0.02
    wu_std: float = 0.02
    wd_std: float = 0.02
    seed: int = 20261202
    notes: str = field(default="", compare=False)


D, F, E_, K_ = 6144, 2816, 256, 8

WORKLOADS = {
    # Tiny fp32 layer with an in-path router GEMV.
    "tiny_fp32": Workload("tiny_fp32", T=16, d=64, E=8, k=2, f=128, act="f32", wfmt="f32",
                          router=True, seed=20261203),
    # Same shape with unit-variance activations and 1/fan-in weights, so that
    # SiLU works in its nonlinear range (at std 0.02 it is almost linear).
    "tiny_fp32_stress": Workload("tiny_fp32_stress", T=16, d=64, E=8, k=2, f=128, act="f32",
                                 wfmt="f32", router=True, x_std=1.0, wg_std=64 ** -0.5,
                                 wu_std=64 ** -0.5, wd_std=128 ** -0.5, seed=20261213),
    # Single-request decode: one token.
    "decode_bf16": Workload("decode_bf16", T=1, d=D, E=E_, k=K_, f=F, act="bf16", wfmt="bf16",
                            logit_sets=64, seed=20261204),
    # Speculative verify: 4 concurrent requests x 4 draft tokens.
    "verify_bf16": Workload("verify_bf16", T=16, d=D, E=E_, k=K_, f=F, act="bf16", wfmt="bf16",
                            logit_sets=64, seed=20261205),
    # 4K-token prompt with skewed expert load.
    "prefill_bf16": Workload("prefill_bf16", T=4096, d=D, E=E_, k=K_, f=F, act="bf16",
                             wfmt="bf16", bias_std=0.5, seed=20261206),
    # Block-scaled 4-bit experts (E2M1 values, one E8M0 scale per 32 elements).
    "decode_mxfp4": Workload("decode_mxfp4", T=1, d=D, E=E_, k=K_, f=F, act="bf16",
                             wfmt="mxfp4", logit_sets=64, seed=20261207),
    "prefill_mxfp4": Workload("prefill_mxfp4", T=4096, d=D, E=E_, k=K_, f=F, act="bf16",
                              wfmt="mxfp4", bias_std=0.5, seed=20261207),
    # The pages' own 4-bit format: E2M1 values, one E4M3 scale per 16 elements
    # and one fp32 scale per weight matrix.
    "decode_nvfp4": Workload("decode_nvfp4", T=1, d=D, E=E_, k=K_, f=F, act="bf16",
                             wfmt="nvfp4", logit_sets=64, seed=20261208),
    "prefill_nvfp4": Workload("prefill_nvfp4", T=4096, d=D, E=E_, k=K_, f=F, act="bf16",
                              wfmt="nvfp4", bias_std=0.5, seed=20261208),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def gen_x(T: int, d: int, act: str, seed: int, device="cpu", std: float = 0.02):
    g = _gen(seed * 7 + 1, device)
    x = torch.randn(T, d, generator=g, device=device, dtype=torch.float32) * std
    return x.to(_torch_dtype(act))


def gen_router(E: int, d: int, act: str, seed: int, device="cpu", std: float = 0.02):
    g = _gen(seed * 7 + 2, device)
    w = torch.randn(E, d, generator=g, device=device, dtype=torch.float32) * std
    return w.to(_torch_dtype(act))


def gen_logits(T: int, E: int, seed: int, device="cpu", sets: int = 1, bias_std: float = 0.0):
    """fp32 router logits ``[sets][T][E]`` ~ N(0,1) plus a fixed per-expert bias."""
    g = _gen(seed * 7 + 3, device)
    z = torch.randn(sets, T, E, generator=g, device=device, dtype=torch.float32)
    if bias_std:
        b = torch.randn(E, generator=g, device=device, dtype=torch.float32) * bias_std
        z = z + b
    return z


# E2M1 magnitudes in code order and the midpoints between neighbours.  Used
# only to encode generated weights; decoding lives in the oracle and the
# library, each with its own code.
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def quantize_mxfp4(w: torch.Tensor):
    """OCP MX quantisation of ``w[..., K]`` (K % 32 == 0) to MX-FP4.

    Shared exponent per 32-element block: floor(log2(amax)) - 2 (E2M1's largest
    exponent is 2), stored as E8M0 clamped to [1, 254].  Elements are rounded
    to the nearest E2M1 value (ties to the even code) and saturated at +-6.
    Returns ``(codes uint8[..., K/2], scales uint8[..., K/32])`` with element
    2i in the low nibble of byte i.
    """
    K = w.shape[-1]
    assert K % 32 == 0
    wf = w.to(torch.float32)
    blocks = wf.reshape(*wf.shape[:-1], K // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    tiny = torch.finfo(torch.float32).tiny
    e = torch.floor(torch.log2(torch.clamp(amax, min=tiny))) - 2
    s = torch.clamp(e + 127, 1, 254)
    scale = torch.exp2(s - 127)
    v = blocks / scale[..., None]
    code = _e2m1_codes(v).to(torch.uint8).reshape(*wf.shape[:-1], K)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), s.to(torch.uint8).contiguous()


def _e2m1_codes(v: torch.Tensor) -> torch.Tensor:
    """Nearest E2M1 code (ties to the even code, saturating at +-6) for each
    value of ``v``, with the sign in bit 3."""
    mag = v.abs()
    mids = torch.tensor(_E2M1_MID, dtype=torch.float32, device=v.device)
    code = torch.bucketize(mag, mids, right=False)
    tie = (mag[..., None] == mids).any(dim=-1)
    code = torch.where(tie & (code % 2 == 1), code + 1, code)
    code = torch.clamp(code, max=7)
    return code | torch.where(torch.signbit(v), 8, 0)


def quantize_nvfp4(w: torch.Tensor):
    """NVFP4 quantisation of one matrix ``w[..., K]`` (K % 16 == 0).

    Tensor scale ts = amax|w| / (6 * 448) (fp32; 1 for an all-zero matrix), so
    every block scale fits E4M3.  Block scale per 16 elements: amax / 6 / ts,
    cast to E4M3 (round to nearest even).  Elements: w / (scale * ts) rounded
    to the nearest E2M1 value (ties to the even code), saturating at +-6.
    Returns ``(codes uint8[..., K/2], scales uint8[..., K/16] (E4M3 bytes),
    ts float)`` with element 2i in the low nibble of byte i.
    """
    K = w.shape[-1]
    assert K % 16 == 0
    wf = w.to(torch.float32)
    amax = float(wf.abs().max())
    ts = torch.tensor(amax / (6.0 * 448.0) if amax > 0 else 1.0, dtype=torch.float32).item()
    blocks = wf.reshape(*wf.shape[:-1], K // 16, 16)
    bs = (blocks.abs().amax(dim=-1) / 6.0 / ts).clamp(max=448.0)
    bs8 = bs.to(torch.float8_e4m3fn)
    bsv = bs8.to(torch.float32)
    denom = (bsv * ts)[..., None]
    v = torch.where(denom > 0, blocks / torch.where(denom > 0, denom, 1.0), torch.zeros_like(blocks))
    code = _e2m1_codes(v).to(torch.uint8).reshape(*wf.shape[:-1], K)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), bs8.view(torch.uint8).contiguous(), ts


def gen_expert_weights(wl: Workload, device="cpu", experts=None):
    """Stacked expert weights, reduction dimension innermost.

    bf16/f32: ``w_gate, w_up: [E][f][d]``, ``w_down: [E][d][f]``.
    mxfp4: uint8 codes ``[E][f][d/2]``, ``[E][d][f/2]`` and E8M0 scales
    ``[E][f][d/32]``, ``[E][d][f/32]`` under ``s_gate, s_up, s_down``.
    nvfp4: the same codes, E4M3 scales (dtype float8_e4m3fn) ``[E][f][d/16]``,
    ``[E][d][f/16]`` and fp32 matrix scales ``[E]`` under ``t_gate, t_up, t_down``.
    Expert e is drawn from its own seed, so any subset can be regenerated.
    """
    E, d, f = wl.E, wl.d, wl.f
    experts = range(E) if experts is None else experts
    n = len(experts)
    if wl.wfmt == "nvfp4":
        out = dict(
            w_gate=torch.empty(n, f, d // 2, dtype=torch.uint8, device=device),
            w_up=torch.empty(n, f, d // 2, dtype=torch.uint8, device=device),
            w_down=torch.empty(n, d, f // 2, dtype=torch.uint8, device=device),
            s_gate=torch.empty(n, f, d // 16, dtype=torch.float8_e4m3fn, device=device),
            s_up=torch.empty(n, f, d // 16, dtype=torch.float8_e4m3fn, device=device),
            s_down=torch.empty(n, d, f // 16, dtype=torch.float8_e4m3fn, device=device),
            t_gate=torch.empty(n, dtype=torch.float32, device=device),
            t_up=torch.empty(n, dtype=torch.float32, device=device),
            t_down=torch.empty(n, dtype=torch.float32, device=device),
        )
    elif wl.wfmt == "mxfp4":
        out = dict(
            w_gate=torch.empty(n, f, d // 2, dtype=torch.uint8, device=device),
            w_up=torch.empty(n, f, d // 2, dtype=torch.uint8, device=device),
            w_down=torch.empty(n, d, f // 2, dtype=torch.uint8, device=device),
            s_gate=torch.empty(n, f, d // 32, dtype=torch.uint8, device=device),
            s_up=torch.empty(n, f, d // 32, dtype=torch.uint8, device=device),
            s_down=torch.empty(n, d, f // 32, dtype=torch.uint8, device=device),
        )
    else:
        dt = _torch_dtype(wl.wfmt)
        out = dict(
            w_gate=torch.empty(n, f, d, dtype=dt, device=device),
            w_up=torch.empty(n, f, d, dtype=dt, device=device),
            w_down=torch.empty(n, d, f, dtype=dt, device=device),
        )
    for i, e in enumerate(experts):
        g = _gen(wl.seed * 1000003 + 17 * e + 11, device)
        wg = torch.randn(f, d, generator=g, device=device) * wl.wg_std
        wu = torch.randn(f, d, generator=g, device=device) * wl.wu_std
        wd = torch.randn(d, f, generator=g, device=device) * wl.wd_std
        if wl.wfmt == "nvfp4":
            for name, w in (("gate", wg), ("up", wu), ("down", wd)):
                c, s, t = quantize_nvfp4(w)
                out["w_" + name][i] = c
                out["s_" + name][i] = s.view(torch.float8_e4m3fn)
                out["t_" + name][i] = t
        elif wl.wfmt == "mxfp4":
            for name, w in (("gate", wg), ("up", wu), ("down", wd)):
                c, s = quantize_mxfp4(w)
                out["w_" + name][i] = c
                out["s_" + name][i] = s
        else:
            out["w_gate"][i] = wg
            out["w_up"][i] = wu
            out["w_down"][i] = wd
        del wg, wu, wd
    return out
