"""Plain, slow, fp64 CPU definition of one Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library.  It shares
no code, table or helper with the HIP path and imports nothing from it.

What the layer computes, and where it comes from
-------------------------------------------------
* Expert count and fan-out: every decoder layer of Muse Spark is a
  Mixture-of-Experts layer that picks 8 of its 256 experts per token
  (SGLang-TorchTPU on TPU v7 page, "Introduction").  E and k are parameters.
* Per-expert outputs are normalised and then combined (TensorSharp Muse Spark
  report, "Performance" section, ko and zh-hans pages).  The pages give no
  formula.  Reading adopted: the normalisation is the routing weight, i.e. a
  softmax over all E router logits renormalised over the k selected experts,
  and the combine is the weighted sum of the selected experts' outputs.
* The pages tie accuracy drift to bf16 reduction of per-expert partial results
  (TensorSharp report, "Answer quality" section), so this definition keeps
  every value in fp64 and never rounds.
* Expert FFN: SwiGLU, ``W_down (silu(W_gate x) * (W_up x))`` with
  ``silu(z) = z * sigmoid(z)``, no biases (the pages are silent; this is the
  plain reading of a gated-SiLU expert).
* Top-k selection compares the fp32 logits themselves; ties go to the lower
  expert index; the k slots are ordered by descending logit (ties: lower index).

Storage convention (the reduction dimension is innermost):
``w_gate, w_up: [E][f][d]``, ``w_down: [E][d][f]``, router ``w_r: [E][d]``.
bf16 values are passed as their raw ``uint16`` bit patterns and MX-FP4 weights
as ``uint8`` codes (two E2M1 values per byte, even element in the low nibble)
plus ``uint8`` E8M0 scales, one per 32 consecutive elements along the
reduction dimension.  NVFP4 weights (the pages' own 4-bit expert format:
SGLang-TorchTPU on TPU v7 page, "Results") use the same codes with one E4M3
scale byte per 16 consecutive elements and one fp32 scale per weight matrix.

Every function below is pinned by ``tests/test_oracle_*.py`` against brute
force, closed forms, invariants or library routines; none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Input decoding (exact: every bf16, E2M1 and E8M0 value is an fp64 value)
# ----------------------------------------------------------------------------

# E2M1 magnitudes indexed by the three low bits of a code (1 sign, 2 exponent
# bits with bias 1, 1 mantissa bit; exponent field 0 is the subnormal 0.5*m).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64.  A bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_e8m0(s: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> fp64 power of two 2**(s-127); 0xFF is NaN."""
    s = np.asarray(s, dtype=np.int64)
    out = np.ldexp(1.0, s - 127).astype(np.float64)
    return np.where(s == 255, np.nan, out)


def decode_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MX-FP4 block-scaled weights -> fp64.

    ``codes[..., K/2]`` holds two E2M1 values per byte (element 2i in the low
    nibble, 2i+1 in the high nibble); ``scales[..., K/32]`` holds one E8M0
    scale for each run of 32 consecutive elements along the last axis.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes & 0x0F
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    mag = E2M1_VALUES[nib & 0x7]
    val = np.where(nib & 0x8, -mag, mag)
    K = val.shape[-1]
    assert K % 32 == 0, "MX-FP4 rows must hold whole 32-element blocks"
    blocks = val.reshape(*val.shape[:-1], K // 32, 32)
    sc = decode_e8m0(scales)
    assert sc.shape == blocks.shape[:-1], (sc.shape, blocks.shape)
    return (blocks * sc[..., None]).reshape(val.shape)


def decode_e4m3(b: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 bytes -> fp64.  1 sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2**-6; there
    are no infinities and S.1111.111 is NaN (largest finite value 448)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = b >> 7
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where(sign == 1, -mag, mag)
    return np.where((e == 0xF) & (m == 0x7), np.nan, val)


def decode_nvfp4(codes: np.ndarray, scales: np.ndarray, tensor_scale) -> np.ndarray:
    """NVFP4 block-scaled weights -> fp64.

    ``codes[..., K/2]`` as in MX-FP4 (element 2i in the low nibble);
    ``scales[..., K/16]`` holds one E4M3 byte for each run of 16 consecutive
    elements along the last axis; ``tensor_scale`` is the matrix's fp32 scale.
    value = E2M1(code) * E4M3(scale) * tensor_scale.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes & 0x0F
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    mag = E2M1_VALUES[nib & 0x7]
    val = np.where(nib & 0x8, -mag, mag)
    K = val.shape[-1]
    assert K % 16 == 0, "NVFP4 rows must hold whole 16-element blocks"
    blocks = val.reshape(*val.shape[:-1], K // 16, 16)
    sc = decode_e4m3(scales)
    assert sc.shape == blocks.shape[:-1], (sc.shape, blocks.shape)
    return (blocks * sc[..., None]).reshape(val.shape) * float(np.float32(tensor_scale))


# ----------------------------------------------------------------------------
# Router
# ----------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_i x[t, i] * w_r[e, i]  (fp64).

    A router is implied by the per-layer choice of 8 of 256 experts
    (SGLang-TorchTPU page, "Introduction"); the pages do not describe it.
    """
    x = np.asarray(x, dtype=np.float64)
    w_r = np.asarray(w_r, dtype=np.float64)
    return x @ w_r.T


def route(logits: np.ndarray, k: int):
    """Top-k selection and renormalised softmax weights.

    ``idx[t, :]``: the k experts with the largest logits, ordered by
    descending logit, equal logits ordered by ascending expert index (so the
    lower index wins a tie at the selection boundary).  Logits are compared as
    given (fp32 values; -0.0 equals +0.0; -inf is allowed; NaN is not).

    ``w[t, j] = p[idx[t, j]] / sum_j' p[idx[t, j']]`` with ``p = softmax(l)``
    over all E experts.  When every logit of a token is -inf the softmax is
    undefined; the limit of equal logits is taken and each slot gets 1/k.
    """
    l = np.asarray(logits)
    assert l.ndim == 2
    assert not np.isnan(l).any(), "NaN logits are outside the layer's domain"
    T, E = l.shape
    assert 1 <= k <= E
    lf = l.astype(np.float64)  # exact for fp32 inputs
    # Stable sort on (-logit, index): lexsort's last key is the primary key.
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -lf), axis=-1)
    idx = order[:, :k].astype(np.int32)

    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        row = lf[t]
        m = row.max()
        if m == -np.inf:
            w[t] = 1.0 / k
            continue
        p = np.exp(row - m)
        p /= p.sum()                       # softmax over all E experts
        sel = p[idx[t]]
        w[t] = sel / sel.sum()             # renormalised over the k selected
    return idx, w


# ----------------------------------------------------------------------------
# Permutation of (token, slot) pairs by expert
# ----------------------------------------------------------------------------

def permute(idx: np.ndarray, E: int):
    """Group the T*k (token, slot) pairs by expert.

    The flat id of pair (t, j) is ``q = t*k + j``.  ``sorted_src`` lists the
    flat ids sorted by expert, ties kept in flat-id order (a stable sort).
    ``counts[e]`` is the number of pairs routed to e, ``offsets`` its exclusive
    prefix sum with ``offsets[E] = T*k``, and ``dest_row`` the inverse
    permutation: ``sorted_src[dest_row[q]] == q``.
    """
    key = np.asarray(idx, dtype=np.int64).ravel()
    assert ((key >= 0) & (key < E)).all()
    counts = np.bincount(key, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_src = np.argsort(key, kind="stable").astype(np.int32)
    dest_row = np.empty_like(sorted_src)
    dest_row[sorted_src] = np.arange(key.size, dtype=np.int32)
    return counts, offsets, sorted_src, dest_row


# ----------------------------------------------------------------------------
# Expert FFN and combine
# ----------------------------------------------------------------------------

def _silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------
# FP8 activations (the pages run the experts with FP8 compute: SGLang-TorchTPU
# on TPU v7 page, "Results").  Reading: OCP MX-style FP8, i.e. E4M3 elements
# with one E8M0 scale per 32 consecutive elements along the reduction
# dimension, applied to the two activation operands of the expert FFN (x before
# the gate/up products, h before the down product).
# ----------------------------------------------------------------------------

def round_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest OCP FP8 E4M3 value (ties to even mantissa), saturating at +-448.
    Normal values 2**e * (1 + m/8) for e >= -6, subnormals m * 2**-9."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                      # below 2**-6 the spacing stays 2**-9
    quantum = np.ldexp(1.0, (e - 3).astype(np.int64))
    q = np.round(a / quantum) * quantum          # numpy rounds half to even
    q = np.minimum(q, 448.0)
    return np.where(v < 0, -q, q)


def quantize_mxfp8(v: np.ndarray) -> np.ndarray:
    """The values an MXFP8 encoding of ``v[..., K]`` (K % 32 == 0) decodes to.
    Per 32-element block: shared exponent s = floor(log2 amax) - 8 (E4M3's
    largest exponent), clamped to the E8M0 range [-126, 127]; elements are
    v / 2**s rounded to E4M3 (saturating at +-448); an all-zero block stays 0.
    A NaN element stays NaN and takes no part in amax (the pages say nothing
    of NaN; this keeps it visible in the outputs it reaches).  Infinite
    elements are outside the domain."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % 32 == 0, "MXFP8 rows must hold whole 32-element blocks"
    b = v.reshape(*v.shape[:-1], K // 32, 32)
    amax = np.where(np.isnan(b), 0.0, np.abs(b)).max(axis=-1)
    s = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8
    s = np.clip(s, -126, 127)
    scale = np.ldexp(1.0, s.astype(np.int64))[..., None]
    return (round_e4m3(b / scale) * scale).reshape(v.shape)


def swiglu_expert(xs: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
                  act_quant=None) -> np.ndarray:
    """One expert applied to rows ``xs[n, d]``; ``wg, wu: [f][d]``, ``wd: [d][f]``.
    ``act_quant`` (e.g. ``quantize_mxfp8``) is applied to the rows and to h
    before the products that read them."""
    q = (lambda a: a) if act_quant is None else act_quant
    xs = q(xs)
    g = xs @ wg.T
    u = xs @ wu.T
    h = q(_silu(g) * u)
    return h @ wd.T


def expert_ffn(x, offsets, sorted_src, k, get_expert, act_quant=None):
    """``y_sorted[r] = FFN_e(x[sorted_src[r] // k])`` for r in expert e's segment.

    ``get_expert(e)`` returns the fp64 ``(w_gate[e], w_up[e], w_down[e])``; it
    is only called for experts with at least one routed pair.
    """
    x = np.asarray(x, dtype=np.float64)
    offsets = np.asarray(offsets)
    sorted_src = np.asarray(sorted_src)
    E = offsets.size - 1
    d = x.shape[1]
    y = np.zeros((sorted_src.size, d), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        wg, wu, wd = get_expert(e)
        tok = sorted_src[r0:r1] // k
        y[r0:r1] = swiglu_expert(x[tok], wg, wu, wd, act_quant)
    return y


# Per-expert output normalisation, the second reading of "per-expert outputs
# are normalised, then combined" (TensorSharp Muse Spark report, "Performance"
# section; the pages give no formula).  Reading taken: each selected expert's
# output row is divided by its root mean square over d, with EXPERT_NORM_EPS
# inside the root (the plain parameter-free RMS normalisation), before the
# weighted sum.  It makes the combine nonlinear in the expert outputs.
EXPERT_NORM_EPS = 1e-6


def combine(y_sorted, dest_row, w, expert_norm: bool = False):
    """``out[t] = sum_j w[t, j] * n(y_sorted[dest_row[t*k + j]])`` (fp64, no
    rounding); n is the identity, or the RMS normalisation if ``expert_norm``."""
    w = np.asarray(w, dtype=np.float64)
    T, k = w.shape
    dest = np.asarray(dest_row).reshape(T, k)
    out = np.zeros((T, y_sorted.shape[1]), dtype=np.float64)
    for j in range(k):
        rows = y_sorted[dest[:, j]]
        if expert_norm:
            rows = rows / np.sqrt(np.mean(rows * rows, axis=1, keepdims=True) + EXPERT_NORM_EPS)
        out += w[:, j:j + 1] * rows
    return out


def layer(x, logits, k, get_expert, E=None, w_r=None, act_quant=None, expert_norm=False):
    """Whole layer.  If ``w_r`` is given the logits are computed from it
    (``logits`` is then ignored); otherwise ``logits`` are used as given.
    ``act_quant`` quantises the expert FFN's activation operands (FP8 mode);
    ``expert_norm`` RMS-normalises each expert output before the combine.
    Returns a dict with every intermediate."""
    x = np.asarray(x, dtype=np.float64)
    if w_r is not None:
        logits = router_logits(x, w_r)
    logits = np.asarray(logits)
    E = logits.shape[1] if E is None else E
    idx, w = route(logits, k)
    counts, offsets, sorted_src, dest_row = permute(idx, E)
    y = expert_ffn(x, offsets, sorted_src, k, get_expert, act_quant)
    out = combine(y, dest_row, w, expert_norm)
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                sorted_src=sorted_src, dest_row=dest_row, y_sorted=y, out=out)


def dense_layer(x, logits, k, get_expert):
    """Second formulation for tiny shapes: every expert on every token, mixed
    by the gate matrix ``G[t, e]`` (the renormalised weight if e is selected
    for t, else 0).  It shares ``route`` but none of the permute/combine
    bookkeeping."""
    x = np.asarray(x, dtype=np.float64)
    logits = np.asarray(logits)
    T, E = logits.shape
    idx, w = route(logits, k)
    G = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        G[t, idx[t]] = w[t]
    out = np.zeros_like(x)
    for e in range(E):
        wg, wu, wd = get_expert(e)
        out += G[:, e:e + 1] * swiglu_expert(x, wg, wu, wd)
    return out
