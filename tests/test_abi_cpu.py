"""The C-ABI library without a GPU: it loads, exports every entry point that
include/moe.h declares, and its host-side validation returns the documented
status codes before any device call (so these run on a CPU-only machine)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


@pytest.fixture(scope="module")
def m():
    import expert_ffn_layer_softmax_amd as mod
    mod.load()
    return mod


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(m):
    names = _declared()
    assert "moe_layer_forward" in names and len(names) >= 12
    for n in names:
        assert hasattr(m.lib, n), f"{n} declared in moe.h but not exported"


def test_python_binding_names_match_abi(m):
    for n in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
              "moe_workspace_size", "moe_status_string"):
        assert callable(getattr(m, n))


def _dims(m, T=4, d=64, E=8, k=2, f=32, act=1, w=1, flags=0):
    return m._lib.MoeDims(T, d, E, k, f, act, w, flags)


def _ws(m, dims):
    out = ctypes.c_size_t(0)
    st = m.lib.moe_workspace_size(ctypes.byref(dims), ctypes.byref(out))
    return st, out.value


def test_workspace_size_validation(m):
    assert _ws(m, _dims(m))[0] == OK
    assert _ws(m, _dims(m))[1] > 0
    assert _ws(m, _dims(m, k=9))[0] == INVALID          # k > E
    assert _ws(m, _dims(m, k=0))[0] == INVALID
    assert _ws(m, _dims(m, T=-1))[0] == INVALID
    assert _ws(m, _dims(m, d=48))[0] == UNSUPPORTED     # d % 32
    assert _ws(m, _dims(m, f=40))[0] == UNSUPPORTED
    assert _ws(m, _dims(m, E=2000, k=2))[0] == UNSUPPORTED
    assert _ws(m, _dims(m, E=100, k=65))[0] == UNSUPPORTED
    assert _ws(m, _dims(m, act=0, w=1))[0] == UNSUPPORTED   # f32 act, bf16 weights
    assert _ws(m, _dims(m, act=1, w=0))[0] == UNSUPPORTED
    assert _ws(m, _dims(m, act=2, w=2))[0] == UNSUPPORTED   # MX-FP4 activations
    assert _ws(m, _dims(m, act=5))[0] == INVALID
    assert _ws(m, _dims(m, act=1, w=3))[0] == OK            # NVFP4 weights
    assert _ws(m, _dims(m, act=3, w=3))[0] == UNSUPPORTED   # NVFP4 activations
    assert _ws(m, _dims(m, act=1, w=4))[0] == INVALID
    # FP8 activations: MX-FP4 weights, bf16 activations, d and f multiples of 256
    assert _ws(m, _dims(m, d=256, f=512, w=2, flags=1))[0] == OK
    assert _ws(m, _dims(m, d=256, f=512, w=2, flags=4))[0] == INVALID   # unknown bit
    # RMS-normalised combine: any supported pair, alone or with FP8 activations
    assert _ws(m, _dims(m, flags=2))[0] == OK
    assert _ws(m, _dims(m, d=256, f=512, w=2, flags=3))[0] == OK
    assert _ws(m, _dims(m, flags=2))[1] == _ws(m, _dims(m))[1]
    assert _ws(m, _dims(m, d=256, f=512, w=1, flags=1))[0] == UNSUPPORTED   # bf16 weights
    assert _ws(m, _dims(m, d=256, f=512, w=3, flags=1))[0] == OK            # NVFP4 weights
    assert _ws(m, _dims(m, d=256, f=320, w=3, flags=1))[0] == UNSUPPORTED   # f % 256
    assert _ws(m, _dims(m, d=320, f=512, w=2, flags=1))[0] == UNSUPPORTED   # d % 256
    # the FP8 workspace holds the MXFP8 activations instead of the bf16 h
    T, k, d, f = 64, 8, 256, 512
    w8 = _ws(m, _dims(m, T=T, d=d, E=16, k=k, f=f, w=2, flags=1))[1]
    w16 = _ws(m, _dims(m, T=T, d=d, E=16, k=k, f=f, w=2))[1]
    assert w8 - w16 >= T * d + T * d // 32 + T * k * f // 32 - T * k * f - 4 * 256
    # with NVFP4 weights the FP8 workspace adds the rounded x (bf16) to the bf16 h
    n8 = _ws(m, _dims(m, T=T, d=d, E=16, k=k, f=f, w=3, flags=1))[1]
    n16 = _ws(m, _dims(m, T=T, d=d, E=16, k=k, f=f, w=3))[1]
    assert n8 - n16 >= T * d * 2
    assert m.lib.moe_workspace_size(None, None) == INVALID


def test_workspace_grows_with_tokens(m):
    small = _ws(m, _dims(m, T=1, d=6144, E=256, k=8, f=2816))[1]
    big = _ws(m, _dims(m, T=4096, d=6144, E=256, k=8, f=2816))[1]
    # h (bf16) and y_sorted (fp32) for T*k rows dominate
    assert big >= 4096 * 8 * (2816 * 2 + 6144 * 4)
    assert small < big


FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: every call below is rejected
MISALIGNED = ctypes.c_void_p(0x10004)


def test_route_validation(m):
    L = m.lib
    assert L.moe_route(None, 0, 8, 2, None, None, None) == OK          # T == 0
    assert L.moe_route(None, 4, 8, 2, None, None, None) == INVALID
    assert L.moe_route(FAKE, 4, 8, 9, FAKE, FAKE, None) == INVALID      # k > E
    assert L.moe_route(FAKE, 4, 2000, 2, FAKE, FAKE, None) == UNSUPPORTED
    assert L.moe_route(FAKE, 4, 256, 65, FAKE, FAKE, None) == UNSUPPORTED
    assert L.moe_route(MISALIGNED, 4, 8, 2, FAKE, FAKE, None) == INVALID
    assert L.moe_route(FAKE, -1, 8, 2, FAKE, FAKE, None) == INVALID


def test_permute_validation(m):
    L = m.lib
    assert L.moe_permute(None, 0, 8, 2, None, None, None, None, None) == OK
    assert L.moe_permute(FAKE, 3, 8, 2, FAKE, None, FAKE, FAKE, None) == INVALID
    assert L.moe_permute(FAKE, 3, 8, 2, FAKE, FAKE, FAKE, MISALIGNED, None) == INVALID
    assert L.moe_permute(FAKE, 3, 1025, 2, FAKE, FAKE, FAKE, FAKE, None) == UNSUPPORTED


def _w(m, mx=False, bad=None, t=False):
    vals = [FAKE.value] * 3 + ([FAKE.value] * 3 if mx else [None] * 3) + ([FAKE.value] * 3 if t else [None] * 3)
    if bad is not None:
        vals[bad[0]] = bad[1]
    return m._lib.MoeExpertWeights(*vals)


def test_layer_forward_validation(m):
    L = m.lib
    dims = _dims(m)
    st, need = _ws(m, dims)
    args = lambda d, w, ws=FAKE, wsb=need: (ctypes.byref(d), FAKE, None, FAKE, ctypes.byref(w), FAKE,
                                           FAKE, FAKE, ws, wsb, None)
    assert L.moe_layer_forward(*args(dims, _w(m), wsb=need - 1)) == WS_SMALL
    assert L.moe_layer_forward(*args(dims, _w(m, bad=(1, None)))) == INVALID
    assert L.moe_layer_forward(*args(dims, _w(m, mx=True))) == INVALID      # scales with bf16
    mxd = _dims(m, w=2)
    assert L.moe_layer_forward(*args(mxd, _w(m), wsb=_ws(m, mxd)[1])) == INVALID  # no scales
    assert L.moe_layer_forward(*args(dims, _w(m), ws=ctypes.c_void_p(0x10010))) == INVALID
    assert L.moe_layer_forward(*args(_dims(m, d=40), _w(m))) == UNSUPPORTED
    assert L.moe_layer_forward(*args(_dims(m, T=0), _w(m))) == OK
    # NVFP4: block scales and fp32 matrix scales both required; matrix scales
    # only with NVFP4
    nvd = _dims(m, w=3)
    nvn = _ws(m, nvd)[1]
    assert L.moe_layer_forward(*args(nvd, _w(m, mx=True), wsb=nvn)) == INVALID       # no t_*
    assert L.moe_layer_forward(*args(nvd, _w(m, t=True), wsb=nvn)) == INVALID        # no s_*
    assert L.moe_layer_forward(*args(nvd, _w(m, mx=True, t=True, bad=(7, MISALIGNED.value)),
                                     wsb=nvn)) == INVALID
    assert L.moe_layer_forward(*args(mxd, _w(m, mx=True, t=True), wsb=_ws(m, mxd)[1])) == INVALID
    assert L.moe_layer_forward(*args(dims, _w(m, t=True))) == INVALID
    assert L.moe_layer_forward(None, None, None, None, None, None, None, None, None, 0, None) == INVALID


def test_expert_ffn_and_combine_validation(m):
    L = m.lib
    dims = _dims(m)
    _, need = _ws(m, dims)
    w = _w(m)
    assert L.moe_expert_ffn(ctypes.byref(dims), FAKE, FAKE, FAKE, ctypes.byref(w), FAKE, FAKE,
                            need - 256, None) == WS_SMALL
    assert L.moe_expert_ffn(ctypes.byref(dims), None, FAKE, FAKE, ctypes.byref(w), FAKE, FAKE,
                            need, None) == INVALID
    assert L.moe_combine(ctypes.byref(dims), FAKE, FAKE, FAKE, None, None) == INVALID
    assert L.moe_combine(ctypes.byref(dims), FAKE, MISALIGNED, FAKE, FAKE, None) == INVALID
    assert L.moe_combine(ctypes.byref(_dims(m, T=0)), None, None, None, None, None) == OK


def test_status_strings(m):
    for code in range(5):
        assert m.moe_status_string(code)
    assert m.moe_status_string(99) == "unknown status"


def test_timing_query_validation(m):
    assert m.lib.moe_timing_query(None, None, None) == INVALID
    assert m.lib.moe_timing_names(None, 0) == INVALID


def test_quantize_mxfp8_validation(m):
    L = m.lib
    assert L.moe_quantize_mxfp8(None, 0, 64, None, None, None) == OK           # rows == 0
    assert L.moe_quantize_mxfp8(FAKE, 4, 48, FAKE, FAKE, None) == UNSUPPORTED  # K % 32
    assert L.moe_quantize_mxfp8(FAKE, 4, 0, FAKE, FAKE, None) == INVALID
    assert L.moe_quantize_mxfp8(FAKE, -1, 64, FAKE, FAKE, None) == INVALID
    assert L.moe_quantize_mxfp8(FAKE, 4, 64, None, FAKE, None) == INVALID
    assert L.moe_quantize_mxfp8(MISALIGNED, 4, 64, FAKE, FAKE, None) == INVALID
    assert L.moe_quantize_mxfp8(FAKE, 4, 64, MISALIGNED, FAKE, None) == INVALID
    assert L.moe_quantize_mxfp8(FAKE, 1 << 40, 64, FAKE, FAKE, None) == UNSUPPORTED


def test_layer_forward_noalloc_validation(m):
    """The allocation-free entry point validates as moe_layer_forward does and
    rejects shapes whose workspace exceeds its 64 MiB scratch, all before any
    device call."""
    L = m.lib
    args = lambda d, w: (ctypes.byref(d), FAKE, None, FAKE, ctypes.byref(w), FAKE, FAKE, FAKE, None)
    assert L.moe_layer_forward_noalloc(*args(_dims(m, T=0), _w(m))) == OK
    assert L.moe_layer_forward_noalloc(*args(_dims(m, d=40), _w(m))) == UNSUPPORTED
    assert L.moe_layer_forward_noalloc(*args(_dims(m), _w(m, bad=(1, None)))) == INVALID
    assert L.moe_layer_forward_noalloc(*args(_dims(m), _w(m, mx=True))) == INVALID
    assert L.moe_layer_forward_noalloc(None, None, None, None, None, None, None, None, None) == INVALID
    big = _dims(m, T=278, d=6144, E=256, k=8, f=2816)
    fits = _dims(m, T=277, d=6144, E=256, k=8, f=2816)
    assert _ws(m, fits)[1] <= 64 << 20 < _ws(m, big)[1]
    assert L.moe_layer_forward_noalloc(*args(big, _w(m))) == WS_SMALL
    prefill = _dims(m, T=4096, d=6144, E=256, k=8, f=2816)
    assert L.moe_layer_forward_noalloc(*args(prefill, _w(m))) == WS_SMALL


def test_debug_check_entry_point(m):
    """moe_debug_check validates its pointer; a release build has no checks."""
    L = m.lib
    assert L.moe_debug_check(None) == INVALID
    v = ctypes.c_uint32(7)
    assert L.moe_debug_check(ctypes.byref(v)) == UNSUPPORTED
    assert v.value == 0
