"""ctypes binding of ``libmoe_mi355x.so`` (C ABI: ``include/moe.h``).

Each function takes torch tensors, checks device/dtype/shape/contiguity,
passes raw device pointers plus the current HIP stream to the C entry point
of the same name, and raises ``MoeError`` on any non-OK status.  Outputs that
are not supplied are allocated with torch (device memory is torch's job).
"""

from __future__ import annotations

import ctypes
import os

import torch  # loaded first: the library then binds to torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_MI355X_LIB may name another build of the same library (e.g. a tuning
# variant); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK = 0
MOE_DTYPE_F32, MOE_DTYPE_BF16, MOE_DTYPE_MXFP4, MOE_DTYPE_NVFP4 = 0, 1, 2, 3


class MoeDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("f", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class MoeExpertWeights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("t_gate", ctypes.c_void_p), ("t_up", ctypes.c_void_p), ("t_down", ctypes.c_void_p)]


_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_P = ctypes.POINTER
_SIGS = {
    "moe_workspace_size": [_P(MoeDims), _P(_sz)],
    "moe_route": [_vp, _i32, _i32, _i32, _vp, _vp, _vp],
    "moe_permute": [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp],
    "moe_expert_ffn": [_P(MoeDims), _vp, _vp, _vp, _P(MoeExpertWeights), _vp, _vp, _sz, _vp],
    "moe_combine": [_P(MoeDims), _vp, _vp, _vp, _vp, _vp],
    "moe_layer_forward": [_P(MoeDims), _vp, _vp, _vp, _P(MoeExpertWeights), _vp, _vp, _vp, _vp,
                          _sz, _vp],
    "moe_timing_start": [],
    "moe_timing_stop": [],
    "moe_timing_query": [ctypes.c_char_p, _P(_i32), _P(ctypes.c_double)],
    "moe_timing_names": [ctypes.c_char_p, _sz],
    "moe_last_device_error": [],
    "moe_quantize_mxfp8": [_vp, ctypes.c_int64, _i32, _vp, _vp, _vp],
    "moe_layer_forward_noalloc": [_P(MoeDims), _vp, _vp, _vp, _P(MoeExpertWeights), _vp, _vp, _vp, _vp],
    "moe_debug_check": [_P(ctypes.c_uint32)],
}


class _Library:
    """``libmoe_mi355x.so``, opened on first use.

    Importing the package needs no built library (so a fresh checkout can run
    the build); the first call into the library opens it and raises
    ImportError if it has not been built.  There is no CPU fallback.
    """

    def __init__(self):
        self._cdll = None

    def _open(self):
        if self._cdll is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build the HIP library first "
                    "(python -m expert_ffn_layer_softmax_amd.build); there is no CPU fallback")
            cdll = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
            for name, args in _SIGS.items():
                fn = getattr(cdll, name)
                fn.argtypes = args
                fn.restype = ctypes.c_int32
            cdll.moe_status_string.argtypes = [ctypes.c_int32]
            cdll.moe_status_string.restype = ctypes.c_char_p
            self._cdll = cdll
        return self._cdll

    def __getattr__(self, name):
        if name.startswith("_"):
            raise AttributeError(name)
        return getattr(self._open(), name)


lib = _Library()


def load():
    """Open the library now (raises ImportError if it is not built)."""
    return lib._open()


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = moe_status_string(status)
        if status == 4:
            msg += f" (hipError {lib.moe_last_device_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


def moe_status_string(status: int) -> str:
    return lib.moe_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (the library has no CPU path)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_ACT = {torch.float32: MOE_DTYPE_F32, torch.bfloat16: MOE_DTYPE_BF16}


MOE_FLAG_FP8_ACTIVATIONS = 1
MOE_FLAG_EXPERT_NORM = 2


def _dims(T, d, E, k, f, act, wfmt, flags=0) -> MoeDims:
    return MoeDims(T, d, E, k, f, act, wfmt, flags)


def _weights(w: dict, E, d, f, wfmt, device) -> MoeExpertWeights:
    if wfmt == MOE_DTYPE_NVFP4:
        _need(w["w_gate"], "w_gate", torch.uint8, (E, f, d // 2), device)
        _need(w["w_up"], "w_up", torch.uint8, (E, f, d // 2), device)
        _need(w["w_down"], "w_down", torch.uint8, (E, d, f // 2), device)
        for n, shape in (("s_gate", (E, f, d // 16)), ("s_up", (E, f, d // 16)), ("s_down", (E, d, f // 16))):
            _need(w[n].view(torch.uint8), n, torch.uint8, shape, device)
        for n in ("t_gate", "t_up", "t_down"):
            _need(w[n], n, torch.float32, (E,), device)
        return MoeExpertWeights(*(w[n].data_ptr() for n in
                                  ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                                   "t_gate", "t_up", "t_down")))
    if wfmt == MOE_DTYPE_MXFP4:
        _need(w["w_gate"], "w_gate", torch.uint8, (E, f, d // 2), device)
        _need(w["w_up"], "w_up", torch.uint8, (E, f, d // 2), device)
        _need(w["w_down"], "w_down", torch.uint8, (E, d, f // 2), device)
        _need(w["s_gate"], "s_gate", torch.uint8, (E, f, d // 32), device)
        _need(w["s_up"], "s_up", torch.uint8, (E, f, d // 32), device)
        _need(w["s_down"], "s_down", torch.uint8, (E, d, f // 32), device)
        return MoeExpertWeights(*(w[n].data_ptr() for n in
                                  ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")))
    dt = torch.float32 if wfmt == MOE_DTYPE_F32 else torch.bfloat16
    _need(w["w_gate"], "w_gate", dt, (E, f, d), device)
    _need(w["w_up"], "w_up", dt, (E, f, d), device)
    _need(w["w_down"], "w_down", dt, (E, d, f), device)
    return MoeExpertWeights(w["w_gate"].data_ptr(), w["w_up"].data_ptr(), w["w_down"].data_ptr(),
                            None, None, None)


def _wfmt(w: dict) -> int:
    if w.get("t_gate") is not None:
        return MOE_DTYPE_NVFP4
    if "s_gate" in w and w["s_gate"] is not None:
        return MOE_DTYPE_MXFP4
    return MOE_DTYPE_F32 if w["w_gate"].dtype == torch.float32 else MOE_DTYPE_BF16


def _wshape(w: dict, wfmt: int):
    E, f, dd = w["w_gate"].shape
    return E, (dd * 2 if wfmt in (MOE_DTYPE_MXFP4, MOE_DTYPE_NVFP4) else dd), f


def moe_workspace_size(T, d, E, k, f, act_dtype, w_dtype, flags=0) -> int:
    out = _sz(0)
    _check(lib.moe_workspace_size(ctypes.byref(_dims(T, d, E, k, f, act_dtype, w_dtype, flags)),
                                  ctypes.byref(out)), "moe_workspace_size")
    return out.value


def moe_route(logits, k, topk_idx=None, topk_w=None):
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    if topk_idx is None:
        topk_idx = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), logits.device)
    _need(topk_w, "topk_w", torch.float32, (T, k), logits.device)
    _check(lib.moe_route(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_w), _stream(logits)),
           "moe_route")
    return topk_idx, topk_w


def moe_permute(topk_idx, E, counts=None, offsets=None, sorted_src=None, dest_row=None):
    _need(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    sorted_src = torch.empty(T * k, dtype=torch.int32, device=dev) if sorted_src is None else sorted_src
    dest_row = torch.empty(T * k, dtype=torch.int32, device=dev) if dest_row is None else dest_row
    _need(counts, "counts", torch.int32, (E,), dev)
    _need(offsets, "offsets", torch.int32, (E + 1,), dev)
    _need(sorted_src, "sorted_src", torch.int32, (T * k,), dev)
    _need(dest_row, "dest_row", torch.int32, (T * k,), dev)
    _check(lib.moe_permute(_ptr(topk_idx), T, E, k, _ptr(counts), _ptr(offsets), _ptr(sorted_src),
                           _ptr(dest_row), _stream(topk_idx)), "moe_permute")
    return counts, offsets, sorted_src, dest_row


def _workspace(dims: MoeDims, device, workspace):
    need = _sz(0)
    _check(lib.moe_workspace_size(ctypes.byref(dims), ctypes.byref(need)), "moe_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=device)
    _need(workspace, "workspace", torch.uint8, None, device)
    return workspace


def moe_expert_ffn(x, offsets, sorted_src, k, weights: dict, y_sorted=None, workspace=None, fp8=False):
    """Grouped SwiGLU expert FFN.  ``fp8=True`` sets MOE_FLAG_FP8_ACTIVATIONS
    (MXFP8 activations on the scaled MFMA; MX-FP4 weights)."""
    _need(x, "x")
    if x.dtype not in _ACT:
        raise TypeError("x must be float32 or bfloat16")
    T, d = x.shape
    wfmt = _wfmt(weights)
    E, _, f = _wshape(weights, wfmt)
    dev = x.device
    _need(offsets, "offsets", torch.int32, (E + 1,), dev)
    _need(sorted_src, "sorted_src", torch.int32, (T * k,), dev)
    dims = _dims(T, d, E, k, f, _ACT[x.dtype], wfmt, _flags(fp8))
    w = _weights(weights, E, d, f, wfmt, dev)
    if y_sorted is None:
        y_sorted = torch.empty(T * k, d, dtype=torch.float32, device=dev)
    _need(y_sorted, "y_sorted", torch.float32, (T * k, d), dev)
    ws = _workspace(dims, dev, workspace)
    _check(lib.moe_expert_ffn(ctypes.byref(dims), _ptr(x), _ptr(offsets), _ptr(sorted_src),
                              ctypes.byref(w), _ptr(y_sorted), _ptr(ws), ws.numel(), _stream(x)),
           "moe_expert_ffn")
    return y_sorted


def _flags(fp8=False, expert_norm=False):
    return (MOE_FLAG_FP8_ACTIVATIONS if fp8 else 0) | (MOE_FLAG_EXPERT_NORM if expert_norm else 0)


def moe_combine(y_sorted, dest_row, topk_w, out_dtype, out=None, expert_norm=False):
    _need(y_sorted, "y_sorted", torch.float32)
    T, k = topk_w.shape
    d = y_sorted.shape[1]
    dev = y_sorted.device
    _need(dest_row, "dest_row", torch.int32, (T * k,), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    if out is None:
        out = torch.empty(T, d, dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, (T, d), dev)
    dims = _dims(T, d, max(k, 1), k, 32, _ACT[out_dtype],
                 MOE_DTYPE_F32 if out_dtype == torch.float32 else MOE_DTYPE_BF16,
                 _flags(expert_norm=expert_norm))
    _check(lib.moe_combine(ctypes.byref(dims), _ptr(y_sorted), _ptr(dest_row), _ptr(topk_w),
                           _ptr(out), _stream(y_sorted)), "moe_combine")
    return out


def moe_layer_forward(x, weights: dict, k, logits=None, w_router=None, topk_idx=None, topk_w=None,
                      out=None, workspace=None, fp8=False, expert_norm=False):
    """Whole layer.  Give ``w_router`` to compute the logits in-path (they are
    written to ``logits``, allocated if None), or ``logits`` to route by them.
    ``fp8=True`` sets MOE_FLAG_FP8_ACTIVATIONS (MXFP8 activations on the scaled
    MFMA; MX-FP4 weights); ``expert_norm=True`` sets MOE_FLAG_EXPERT_NORM
    (each expert's output row RMS-normalised before the combine)."""
    _need(x, "x")
    if x.dtype not in _ACT:
        raise TypeError("x must be float32 or bfloat16")
    T, d = x.shape
    wfmt = _wfmt(weights)
    E, _, f = _wshape(weights, wfmt)
    dev = x.device
    if w_router is None and logits is None:
        raise ValueError("give logits or w_router")
    if w_router is not None:
        _need(w_router, "w_router", x.dtype, (E, d), dev)
        if logits is None:
            logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    _need(logits, "logits", torch.float32, (T, E), dev)
    topk_idx = torch.empty(T, k, dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    topk_w = torch.empty(T, k, dtype=torch.float32, device=dev) if topk_w is None else topk_w
    out = torch.empty(T, d, dtype=x.dtype, device=dev) if out is None else out
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    _need(out, "out", x.dtype, (T, d), dev)
    dims = _dims(T, d, E, k, f, _ACT[x.dtype], wfmt, _flags(fp8, expert_norm))
    w = _weights(weights, E, d, f, wfmt, dev)
    ws = _workspace(dims, dev, workspace)
    _check(lib.moe_layer_forward(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(logits),
                                 ctypes.byref(w), _ptr(topk_idx), _ptr(topk_w), _ptr(out), _ptr(ws),
                                 ws.numel(), _stream(x)), "moe_layer_forward")
    return dict(out=out, logits=logits, topk_idx=topk_idx, topk_w=topk_w, workspace=ws)


def moe_quantize_mxfp8(x, q=None, scales=None):
    """MXFP8 codes and E8M0 block scales of bf16 ``x[rows][K]`` (the FP8
    path's activation quantisation, exposed for checking)."""
    _need(x, "x", torch.bfloat16)
    rows, K = x.shape
    dev = x.device
    q = torch.empty(rows, K, dtype=torch.uint8, device=dev) if q is None else q
    scales = torch.empty(rows, K // 32, dtype=torch.uint8, device=dev) if scales is None else scales
    _need(q, "q", torch.uint8, (rows, K), dev)
    _need(scales, "scales", torch.uint8, (rows, K // 32), dev)
    _check(lib.moe_quantize_mxfp8(_ptr(x), rows, K, _ptr(q), _ptr(scales), _stream(x)),
           "moe_quantize_mxfp8")
    return q, scales


def moe_layer_forward_noalloc(x, weights: dict, k, logits=None, w_router=None, topk_idx=None,
                              topk_w=None, out=None, fp8=False, expert_norm=False):
    """moe_layer_forward on the library's own scratch (no workspace; the C
    call allocates nothing).  Outputs not supplied are allocated here, by
    torch, before the call."""
    _need(x, "x")
    if x.dtype not in _ACT:
        raise TypeError("x must be float32 or bfloat16")
    T, d = x.shape
    wfmt = _wfmt(weights)
    E, _, f = _wshape(weights, wfmt)
    dev = x.device
    if w_router is None and logits is None:
        raise ValueError("give logits or w_router")
    if w_router is not None:
        _need(w_router, "w_router", x.dtype, (E, d), dev)
        if logits is None:
            logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    _need(logits, "logits", torch.float32, (T, E), dev)
    topk_idx = torch.empty(T, k, dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    topk_w = torch.empty(T, k, dtype=torch.float32, device=dev) if topk_w is None else topk_w
    out = torch.empty(T, d, dtype=x.dtype, device=dev) if out is None else out
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    _need(out, "out", x.dtype, (T, d), dev)
    dims = _dims(T, d, E, k, f, _ACT[x.dtype], wfmt, _flags(fp8, expert_norm))
    w = _weights(weights, E, d, f, wfmt, dev)
    _check(lib.moe_layer_forward_noalloc(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(logits),
                                         ctypes.byref(w), _ptr(topk_idx), _ptr(topk_w), _ptr(out),
                                         _stream(x)), "moe_layer_forward_noalloc")
    return dict(out=out, logits=logits, topk_idx=topk_idx, topk_w=topk_w)


def moe_debug_check() -> int:
    """Bounds-check violations recorded by a debug build since the last call
    (bit mask, see include/moe.h); raises MoeError on a release build."""
    v = ctypes.c_uint32(0)
    _check(lib.moe_debug_check(ctypes.byref(v)), "moe_debug_check")
    return v.value


def moe_timing_start():
    _check(lib.moe_timing_start(), "moe_timing_start")


def moe_timing_stop():
    _check(lib.moe_timing_stop(), "moe_timing_stop")


def moe_timing_query(kernel: str):
    n = _i32(0)
    ms = ctypes.c_double(0.0)
    _check(lib.moe_timing_query(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)), "moe_timing_query")
    return n.value, ms.value


def moe_timing_names():
    buf = ctypes.create_string_buffer(4096)
    _check(lib.moe_timing_names(buf, 4096), "moe_timing_names")
    return [s for s in buf.value.decode().split(",") if s]
