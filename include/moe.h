/*
 * moe.h -- C ABI of a gfx950 (MI355X) library for the forward pass of one
 * Mixture-of-Experts decoder layer: router softmax and top-k selection,
 * grouping of (token, slot) pairs by expert, a grouped SwiGLU expert FFN over
 * bf16, MX-FP4 or NVFP4 weights with fp32 accumulation, and the weighted
 * combine.
 *
 * The layer is the one the Muse Spark pages describe: every decoder layer is
 * a Mixture-of-Experts layer that sends each token to 8 of its 256 experts
 * (SGLang-TorchTPU on TPU v7 page, "Introduction"), whose selected expert
 * outputs are normalised and then combined (TensorSharp Muse Spark report,
 * "Performance" section).  E, k, d and f are parameters here.
 *
 * Conventions shared by every entry point
 *  - Every buffer pointer is a DEVICE pointer (HIP global memory), row-major,
 *    contiguous and at least 16-byte aligned; the workspace 256-byte aligned.
 *  - The caller owns every buffer and keeps it alive until the work queued on
 *    `stream` has finished.  The library allocates no device memory, keeps no
 *    pointer after returning and never synchronises the stream.
 *  - All work is queued asynchronously on `stream` (a hipStream_t; NULL means
 *    the default stream).  Calls are reentrant.
 *  - Arguments are validated on the host before any HIP call; a call that
 *    returns anything but MOE_OK has queued no work.  Errors are returned as
 *    moe_status_t, never raised or aborted across the ABI.  MOE_ERR_DEVICE
 *    means a HIP launch failed; moe_last_device_error() then holds the
 *    hipError_t value for the calling thread.
 *  - T == 0 is a valid no-op (pointers are then not inspected).
 *  - Results are deterministic: identical inputs give bit-identical outputs
 *    (no floating-point atomics anywhere).
 *
 * Stored layouts (the reduction dimension is innermost):
 *    x                 [T][d]          act dtype (fp32 or bf16)
 *    router w_r        [E][d]          act dtype
 *    logits            [T][E]          fp32
 *    w_gate, w_up      [E][f][d]       w dtype
 *    w_down            [E][d][f]       w dtype
 *    MX-FP4 weights:   codes uint8 [E][f][d/2] / [E][d][f/2], two E2M1 values
 *                      per byte, element 2i in the low nibble; E8M0 scales
 *                      uint8 [E][f][d/32] / [E][d][f/32], one per 32
 *                      consecutive elements along the reduction dimension.
 *                      The kernels form each weight, code * 2^(s-127), in
 *                      bf16: scale bytes s <= 252 keep it finite; s = 255
 *                      (NaN) propagates.
 *    NVFP4 weights:    the same codes; OCP FP8 E4M3 scales uint8 [E][f][d/16]
 *                      / [E][d][f/16], one per 16 consecutive elements along
 *                      the reduction dimension; fp32 scales t_gate, t_up,
 *                      t_down [E], one per weight matrix.  A weight is
 *                      E2M1(code) * E4M3(scale) * t (the 4-bit expert format
 *                      the pages run: SGLang-TorchTPU on TPU v7 page,
 *                      "Results").  E4M3 NaN bytes (0x7F, 0xFF) are outside
 *                      the domain.
 *    topk_idx, topk_w  [T][k]          int32 / fp32
 *    y_sorted          [T*k][d]        fp32
 *    out               [T][d]          act dtype
 *
 * Supported shapes: 1 <= E <= 1024, 1 <= k <= min(E, 64), d and f positive
 * multiples of 32, T*k < 2^31.  Supported (act, weight) dtype pairs:
 * (F32, F32), (BF16, BF16), (BF16, MXFP4), (BF16, NVFP4); others give
 * MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_MI355X_H_
#define MOE_MI355X_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,    /* NULL/misaligned pointer, bad size      */
  MOE_ERR_UNSUPPORTED = 2,         /* valid but unsupported shape or dtypes  */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < moe_workspace_size  */
  MOE_ERR_DEVICE = 4               /* a HIP call failed                     */
} moe_status_t;

typedef enum {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1,
  MOE_DTYPE_MXFP4 = 2,
  MOE_DTYPE_NVFP4 = 3
} moe_dtype_t;

/* Compute options (moe_dims_t.flags).
 *  MOE_FLAG_FP8_ACTIVATIONS: run the expert products with FP8 activations,
 *    the pages' production precision ("FP8 compute" with 4-bit expert
 *    weights: SGLang-TorchTPU on TPU v7 page, "Results", which pairs FP8
 *    compute with NVFP4 expert weights).  x and h are quantised to MXFP8
 *    (OCP FP8 E4M3 values, one E8M0 scale per 32 elements along the
 *    reduction dimension: scale 2^(floor(log2 amax) - 8), elements rounded to
 *    nearest even and saturated at +-448; h from its fp32 value).  With
 *    MX-FP4 weights the products run on the gfx950 scaled MFMA (E8M0 block
 *    scales on both operands).  With NVFP4 weights, whose E4M3 block scales
 *    that instruction does not take, the quantised activations are carried
 *    as their exact bf16 values and multiplied on bf16 MFMA with fp32 sums,
 *    which computes the same products (exact for block scales >= 2^-124).
 *    Requires act BF16, weights MXFP4 or NVFP4, d and f multiples of 256
 *    (else MOE_ERR_UNSUPPORTED); x, out and every other buffer keep their
 *    layouts.  Applies at every T (the grouped MFMA path is then used for
 *    decode too).  Results are defined with the quantised activations; they
 *    differ from the bf16 path by the FP8 rounding (about 2-4 % relative). */
/*  MOE_FLAG_EXPERT_NORM: divide each selected expert's output row by its
 *    root mean square over d, sqrt(mean(y^2) + 1e-6), before the weighted
 *    sum.  The report that describes the combine (TensorSharp Muse Spark
 *    report, "Performance" section) says the per-expert outputs are
 *    normalised before they are combined but gives no formula; the default
 *    reads that as the routing-weight normalisation, this flag as an RMS
 *    normalisation of each expert's output row.  It makes the combine
 *    nonlinear in the expert outputs.  Honoured by moe_combine and
 *    moe_layer_forward (which then skips the fused single-token down+combine
 *    kernel); other entry points ignore it. */
enum { MOE_FLAG_FP8_ACTIVATIONS = 1, MOE_FLAG_EXPERT_NORM = 2 };

/* Layer shape.  T tokens of hidden size d, E experts of FFN width f, each
 * token routed to k experts.  act_dtype / w_dtype hold moe_dtype_t values;
 * flags holds MOE_FLAG_* bits (0 for the default bf16/fp32 compute). */
typedef struct {
  int32_t T, d, E, k, f;
  int32_t act_dtype;
  int32_t w_dtype;
  int32_t flags;
} moe_dims_t;

/* Stacked expert weights (device pointers, layouts above).  s_* are the
 * block-scale arrays of the 4-bit dtypes (E8M0 for MX-FP4, E4M3 for NVFP4)
 * and t_* the NVFP4 per-matrix fp32 scales; each must be NULL for the dtypes
 * that do not use it. */
typedef struct {
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const uint8_t* s_gate;
  const uint8_t* s_up;
  const uint8_t* s_down;
  const float* t_gate;
  const float* t_up;
  const float* t_down;
} moe_expert_weights_t;

typedef void* moe_stream_t; /* a hipStream_t */

/* Bytes of scratch device memory moe_layer_forward needs for `dims` (also
 * enough for moe_expert_ffn).  Host-only; no device work. */
moe_status_t moe_workspace_size(const moe_dims_t* dims, size_t* bytes);

/* Router top-k and weights (the selection of k of E experts per token:
 * SGLang-TorchTPU page, "Introduction"; the normalised weights the report's
 * "Performance" section combines by).  For each token t:
 *   topk_idx[t][0..k) = the k largest logits[t][:], in descending order of
 *     logit; equal logits ordered by ascending expert index, so a tie at the
 *     selection boundary goes to the lower index.  -0.0 equals +0.0; -inf is
 *     a valid logit; NaN is outside the domain (results unspecified).
 *   topk_w[t][j] = softmax over all E logits, renormalised over the selected
 *     k, computed in fp32 as exp(l_j - l_0) / sum_j' exp(l_j' - l_0); equal
 *     logits (also when all are -inf) contribute 1.
 * Inputs: logits [T][E] fp32.  Outputs: topk_idx [T][k], topk_w [T][k]. */
moe_status_t moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                       int32_t* topk_idx, float* topk_w, moe_stream_t stream);

/* Group the T*k (token, slot) pairs by expert (a stable counting sort of
 * flat ids q = t*k + j by topk_idx.flat[q]).  Each token is sent to k of the
 * E experts (8 of 256 in the pages' model: SGLang-TorchTPU on TPU v7 page,
 * "Introduction"), so every expert computes on the rows routed to it; this
 * call lays those rows out expert by expert for the grouped expert FFN and
 * records where each pair landed for the combine.
 *   counts[E]        pairs routed to each expert
 *   offsets[E+1]     exclusive prefix sum of counts, offsets[E] = T*k
 *   sorted_src[T*k]  flat ids ordered by expert, ascending q within an expert
 *   dest_row[T*k]    inverse: sorted_src[dest_row[q]] == q
 * topk_idx values must lie in [0, E); out-of-range ids are clamped (the
 * outputs are then unspecified but no out-of-bounds access happens). */
moe_status_t moe_permute(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_src,
                         int32_t* dest_row, moe_stream_t stream);

/* Grouped SwiGLU expert FFN.  For every row r of expert e's segment
 * [offsets[e], offsets[e+1]) with token t = sorted_src[r] / k:
 *   h = silu(w_gate[e] x[t]) * (w_up[e] x[t]),  silu(z) = z / (1 + exp(-z))
 *   y_sorted[r] = w_down[e] h
 * All products accumulate in fp32 (the pages tie accuracy drift to bf16
 * reduction of per-expert partial results: TensorSharp report, "Answer
 * quality" section).  h is held in the act dtype in the workspace.
 * x [T][d] act dtype; y_sorted [T*k][d] fp32 output. */
moe_status_t moe_expert_ffn(const moe_dims_t* dims, const void* x, const int32_t* offsets,
                            const int32_t* sorted_src, const moe_expert_weights_t* weights,
                            float* y_sorted, void* workspace, size_t workspace_bytes,
                            moe_stream_t stream);

/* Weighted combine (TensorSharp report, "Performance" section: the selected
 * experts' normalised outputs are combined):
 *   out[t] = sum_{j<k} topk_w[t][j] * y_sorted[dest_row[t*k + j]]
 * summed in fp32 in slot order and rounded once to the act dtype (bf16:
 * round to nearest even).  With MOE_FLAG_EXPERT_NORM each row is first
 * divided by r = sqrt(sum_i y_i^2 / d + 1e-6), the sum of squares taken in
 * fp32. */
moe_status_t moe_combine(const moe_dims_t* dims, const float* y_sorted, const int32_t* dest_row,
                         const float* topk_w, void* out, moe_stream_t stream);

/* The whole layer: [router logits] -> route -> permute -> expert FFN ->
 * combine, i.e. the forward pass of one Mixture-of-Experts decoder layer that
 * sends each token to k of its E experts (SGLang-TorchTPU on TPU v7 page,
 * "Introduction") and combines the selected experts' outputs after their
 * normalisation (TensorSharp Muse Spark report, "Performance" section):
 *   out[t] = sum_{j<k} topk_w[t][j] * FFN_{topk_idx[t][j]}(x[t])
 * with the routing of moe_route, the FFN of moe_expert_ffn and the sum of
 * moe_combine.  If w_router is non-NULL, logits[T][E] = x . w_router^T (fp32
 * accumulation) is written to `logits`; otherwise `logits` is read as input.
 * topk_idx / topk_w receive the routing.  For T == 1 (k <= 16, no
 * MOE_FLAG_* set) the down projection is fused with the combine; the per-token sum keeps slot order
 * and the combine's arithmetic, so the result equals the stage-wise path bit
 * for bit.
 * workspace must hold moe_workspace_size(dims) bytes. */
moe_status_t moe_layer_forward(const moe_dims_t* dims, const void* x, const void* w_router,
                               float* logits, const moe_expert_weights_t* weights,
                               int32_t* topk_idx, float* topk_w, void* out, void* workspace,
                               size_t workspace_bytes, moe_stream_t stream);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with no workspace argument.
 * Its scratch is a device array owned by the library, 64 MiB per GPU
 * (moe_workspace_size(dims) must not exceed 67108864 bytes, else
 * MOE_ERR_WORKSPACE_TOO_SMALL, returned before any device work: enough for
 * single-token decode and small batches at d = 6144, E = 256, k = 8,
 * f = 2816, i.e. T <= 277, not for long prefill).  Each GPU holds its copy
 * until the process ends; the first call on a device looks it up with that
 * device current.  Every call on one GPU uses the same scratch, so calls that
 * overlap on one GPU (several host threads, or several streams whose work
 * overlaps) race; calls on one stream are ordered and safe.  Allocates
 * nothing, on the host or the device. */
moe_status_t moe_layer_forward_noalloc(const moe_dims_t* dims, const void* x, const void* w_router,
                                       float* logits, const moe_expert_weights_t* weights,
                                       int32_t* topk_idx, float* topk_w, void* out,
                                       moe_stream_t stream);

/* MXFP8 quantisation of bf16 activations, the first step of the FP8-compute
 * path (MOE_FLAG_FP8_ACTIVATIONS; "FP8 compute" with 4-bit expert weights:
 * SGLang-TorchTPU on TPU v7 page, "Results").  For each run of 32
 * consecutive elements of a row of x (bf16 [rows][K], K a positive multiple
 * of 32):
 *   scales[r][b] = E8M0 byte of 2^(floor(log2 amax) - 8), amax the largest
 *                  magnitude of the block's non-NaN elements, kept in [1, 254]
 *   q[r][32b + i] = OCP FP8 E4M3 byte of x / 2^(scales[r][b] - 127), rounded
 *                  to nearest even and saturated at +-448; NaN stays NaN.
 * So each block decodes to E4M3(q) * 2^(s - 127).  An all-zero block gives
 * zero codes (its scale byte is then 1).  Infinite inputs are outside the
 * domain.  q is uint8 [rows][K], scales uint8 [rows][K/32]; x and q must be
 * 16-byte aligned.  rows == 0 is a no-op. */
moe_status_t moe_quantize_mxfp8(const void* x, int64_t rows, int32_t K, uint8_t* q,
                                uint8_t* scales, moe_stream_t stream);

/* Bounds checks of a debug build (compiled with -DMOE_DEBUG_CHECKS:
 * `python -m expert_ffn_layer_softmax_amd.build --debug-checks` makes
 * libmoe_mi355x_dbg.so).  In such a build every kernel checks each index it
 * reads from memory before using it as an address -- dest_row and sorted_src
 * values against [0, T*k), expert ids against [0, E), topk_idx against
 * [0, E) in moe_permute, and moe_expert_ffn's offsets for ascending from 0
 * to T*k -- and an index out of range is clamped into range (the access
 * stays in bounds; the results are then wrong) and recorded.  This call
 * returns the OR of the recorded bits since the previous call, and clears
 * them: 1 dest_row, 2 sorted_src, 4 expert id, 8 segment rows, 16 offsets,
 * 32 topk_idx.  Call it after the work to check has finished (it reads the
 * flags synchronously, on the null stream).  Release builds check nothing
 * and return MOE_ERR_UNSUPPORTED with *violations = 0. */
moe_status_t moe_debug_check(uint32_t* violations);

/* Static, NUL-terminated description of a status code. */
const char* moe_status_string(moe_status_t status);

/* hipError_t of the last MOE_ERR_DEVICE returned on the calling thread. */
int32_t moe_last_device_error(void);

/* Per-kernel timing with HIP events, for measurement tools.  While enabled,
 * every kernel the library launches is bracketed by a pair of events recorded
 * on the launch stream (at most 8192 launches are recorded; later ones are
 * not).  moe_timing_start clears earlier records and enables; moe_timing_stop
 * disables.  moe_timing_query waits for the recorded events and returns, for
 * the kernel named `kernel` (e.g. "gemv_gate_up"), the number of recorded
 * launches and their summed duration in milliseconds; call it after the
 * launches it should cover have returned.  moe_timing_names writes the
 * distinct recorded kernel names, comma separated, into buf.  All four are
 * thread-safe. */
moe_status_t moe_timing_start(void);
moe_status_t moe_timing_stop(void);
moe_status_t moe_timing_query(const char* kernel, int32_t* launches, double* total_ms);
moe_status_t moe_timing_names(char* buf, size_t buf_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H_ */
