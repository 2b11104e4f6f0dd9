// C ABI: argument validation, workspace plan, path selection and launches.
// Every check runs on the host before the first HIP call, so a rejected call
// queues no work.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "moe.h"
#include "internal.h"

namespace moe {

namespace {

thread_local int32_t g_last_device_error = 0;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------------ timing --
// `enabled` is read without the lock on every launch (the common, disabled
// case); everything else is guarded by `mu`.  `generation` counts
// moe_timing_start calls, so a launch whose slot was handed out before a
// restart does not record into a slot that now belongs to another launch.
constexpr int kMaxTimed = 8192;
struct TimerState {
  std::mutex mu;
  std::atomic<bool> enabled{false};
  bool created = false;
  std::vector<hipEvent_t> ev0, ev1;
  std::vector<std::string> names;
  int used = 0;
  unsigned generation = 0;
};
TimerState& timer() {
  static TimerState t;
  return t;
}

}  // namespace

LaunchTimer::LaunchTimer(const char* name, hipStream_t s) : name_(name), s_(s), slot_(-1), gen_(0) {
  TimerState& t = timer();
  if (!t.enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(t.mu);
  if (!t.enabled.load(std::memory_order_relaxed) || t.used >= kMaxTimed) return;
  slot_ = t.used++;
  gen_ = t.generation;
  t.names[slot_] = name;
  (void)hipEventRecord(t.ev0[slot_], s);
}

LaunchTimer::~LaunchTimer() {
  if (slot_ < 0) return;
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  if (t.generation == gen_) (void)hipEventRecord(t.ev1[slot_], s_);
}

WsLayout ws_layout(const Dims& dm) {
  WsLayout L{};
  const size_t Tk = (size_t)dm.Tk();
  const size_t E = (size_t)dm.E;
  const size_t max_mtiles = Tk / kGemmBM + (Tk < E ? Tk : E) + 1;
  const size_t act = dm.act == kF32 ? 4 : 2;
  size_t o = 0;
  L.counts = o;      o = align_up(o + E * 4);
  L.offsets = o;     o = align_up(o + (E + 1) * 4);
  L.sorted_src = o;  o = align_up(o + Tk * 4);
  L.dest_row = o;    o = align_up(o + Tk * 4);
  L.active = o;      o = align_up(o + E * 4);
  L.num_active = o;  o = align_up(o + 4);
  L.slot_info = o;   o = align_up(o + E * 16);
  L.mtiles = o;      o = align_up(o + max_mtiles * kMtileInts * 4);
  L.num_mtiles = o;  o = align_up(o + 4);
  // FP8 activations: with MX-FP4 weights x and h travel as MXFP8 codes and
  // scales; with NVFP4 weights as bf16 values on the MXFP8 grid
  const bool f8mx = dm.fp8 && dm.wfmt == kMXFP4;
  const bool f8nv = dm.fp8 && dm.wfmt == kNVFP4;
  L.h = o;           o = align_up(o + (f8mx ? 0 : Tk * (size_t)dm.f * act));
  L.y_sorted = o;    o = align_up(o + Tk * (size_t)dm.d * 4);
  const size_t T = (size_t)dm.T;
  L.xq = o;          o = align_up(o + (f8mx ? T * dm.d : f8nv ? T * dm.d * 2 : 0));
  L.xs = o;          o = align_up(o + (f8mx ? T * dm.d / 32 : 0));
  L.hq = o;          o = align_up(o + (f8mx ? Tk * dm.f : 0));
  L.hs = o;          o = align_up(o + (f8mx ? Tk * dm.f / 32 : 0));
  L.total = o;
  return L;
}

namespace {

Plan plan_at(void* ws, const WsLayout& L) {
  char* b = static_cast<char*>(ws);
  Plan p;
  p.counts = reinterpret_cast<int*>(b + L.counts);
  p.offsets = reinterpret_cast<int*>(b + L.offsets);
  p.sorted_src = reinterpret_cast<int*>(b + L.sorted_src);
  p.dest_row = reinterpret_cast<int*>(b + L.dest_row);
  p.active = reinterpret_cast<int*>(b + L.active);
  p.num_active = reinterpret_cast<int*>(b + L.num_active);
  p.slot_info = reinterpret_cast<int*>(b + L.slot_info);
  p.mtiles = reinterpret_cast<int*>(b + L.mtiles);
  p.num_mtiles = reinterpret_cast<int*>(b + L.num_mtiles);
  return p;
}

moe_status_t device_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_device_error = (int32_t)e;
  return MOE_ERR_DEVICE;
}

bool routing_shape_ok(int T, int E, int k) {
  return T >= 0 && E >= 1 && E <= 1024 && k >= 1 && k <= E && k <= 64 &&
         (long long)T * k < (1ll << 31);
}

moe_status_t check_dims(const moe_dims_t* d, Dims* out) {
  if (!d) return MOE_ERR_INVALID_ARGUMENT;
  if (d->T < 0 || d->d <= 0 || d->f <= 0 || d->E <= 0 || d->k <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (d->k > d->E) return MOE_ERR_INVALID_ARGUMENT;
  if (d->act_dtype < 0 || d->act_dtype > 3 || d->w_dtype < 0 || d->w_dtype > 3)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!routing_shape_ok(d->T, d->E, d->k)) return MOE_ERR_UNSUPPORTED;
  if (d->d % 32 != 0 || d->f % 32 != 0) return MOE_ERR_UNSUPPORTED;
  const bool pair_ok = (d->act_dtype == MOE_DTYPE_F32 && d->w_dtype == MOE_DTYPE_F32) ||
                       (d->act_dtype == MOE_DTYPE_BF16 && d->w_dtype == MOE_DTYPE_BF16) ||
                       (d->act_dtype == MOE_DTYPE_BF16 && d->w_dtype == MOE_DTYPE_MXFP4) ||
                       (d->act_dtype == MOE_DTYPE_BF16 && d->w_dtype == MOE_DTYPE_NVFP4);
  if (!pair_ok) return MOE_ERR_UNSUPPORTED;
  if (d->flags & ~(MOE_FLAG_FP8_ACTIVATIONS | MOE_FLAG_EXPERT_NORM)) return MOE_ERR_INVALID_ARGUMENT;
  Dims dm{d->T, d->d, d->E, d->k, d->f, d->act_dtype, d->w_dtype};
  dm.fp8 = (d->flags & MOE_FLAG_FP8_ACTIVATIONS) != 0;
  dm.expert_norm = (d->flags & MOE_FLAG_EXPERT_NORM) != 0;
  if (dm.fp8 && !fp8_path_ok(dm)) return MOE_ERR_UNSUPPORTED;
  *out = dm;
  return MOE_OK;
}

moe_status_t check_weights(const moe_expert_weights_t* w, const Dims& dm, Weights* out) {
  if (!w || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down))
    return MOE_ERR_INVALID_ARGUMENT;
  if (is_fp4(dm.wfmt)) {
    if (!w->s_gate || !w->s_up || !w->s_down) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(w->s_gate) || !aligned16(w->s_up) || !aligned16(w->s_down))
      return MOE_ERR_INVALID_ARGUMENT;
  } else if (w->s_gate || w->s_up || w->s_down) {
    return MOE_ERR_INVALID_ARGUMENT;
  }
  if (dm.wfmt == kNVFP4) {
    if (!w->t_gate || !w->t_up || !w->t_down) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(w->t_gate) || !aligned16(w->t_up) || !aligned16(w->t_down))
      return MOE_ERR_INVALID_ARGUMENT;
  } else if (w->t_gate || w->t_up || w->t_down) {
    return MOE_ERR_INVALID_ARGUMENT;
  }
  *out = Weights{w->w_gate, w->w_up, w->w_down, w->s_gate, w->s_up, w->s_down,
                 w->t_gate, w->t_up, w->t_down};
  return MOE_OK;
}

// Expert FFN on a prepared plan (offsets, sorted_src, active list).
hipError_t run_expert_ffn(const Dims& dm, const void* x, const Plan& p, const Weights& w,
                          char* ws, const WsLayout& L, float* y_sorted, hipStream_t s) {
  if (dm.fp8 && dm.wfmt == kNVFP4) {
    // x rounded to the MXFP8 grid (bf16); gate/up rounds h the same way
    void* xq = ws + L.xq;
    void* h = ws + L.h;
    hipError_t e = launch_round_mxfp8(x, dm.T, dm.d, xq, s);
    if (e == hipSuccess) e = launch_gg_gate_up(dm, xq, p, w, h, s);
    if (e == hipSuccess) e = launch_gg_down(dm, h, p, w, y_sorted, s);
    return e;
  }
  if (dm.fp8) {
    uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.xq);
    uint8_t* xs = reinterpret_cast<uint8_t*>(ws + L.xs);
    uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.hq);
    uint8_t* hs = reinterpret_cast<uint8_t*>(ws + L.hs);
    hipError_t e = launch_quantize_mxfp8(x, dm.T, dm.d, xq, xs, s);
    if (e == hipSuccess) e = launch_gg_f8_gate_up(dm, xq, xs, p, w, hq, hs, s);
    if (e == hipSuccess) e = launch_gg_f8_down(dm, hq, hs, p, w, y_sorted, s);
    return e;
  }
  void* h = ws + L.h;
  if (grouped_gemm_ok(dm)) {
    hipError_t e = launch_gg_gate_up(dm, x, p, w, h, s);
    if (e != hipSuccess) return e;
    return launch_gg_down(dm, h, p, w, y_sorted, s);
  }
  hipError_t e = launch_gemv_gate_up(dm, x, p, w, h, s);
  if (e != hipSuccess) return e;
  return launch_gemv_down(dm, h, p, w, y_sorted, s);
}

// Validation shared by the whole-layer entry points (all but the workspace).
moe_status_t check_layer_args(const moe_dims_t* dims, const void* x, const void* w_router,
                              const float* logits, const moe_expert_weights_t* weights,
                              const int32_t* topk_idx, const float* topk_w, const void* out, Dims* dm,
                              Weights* w) {
  moe_status_t st = check_dims(dims, dm);
  if (st != MOE_OK) return st;
  if (dm->T == 0) return MOE_OK;
  if ((st = check_weights(weights, *dm, w)) != MOE_OK) return st;
  if (!x || !logits || !topk_idx || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(logits) || !aligned16(topk_idx) || !aligned16(topk_w) ||
      !aligned16(out) || (w_router && !aligned16(w_router)))
    return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

// The whole layer on a validated call and a workspace of L.total bytes.
hipError_t run_layer(const Dims& dm, const Weights& w, const void* x, const void* w_router, float* logits,
                     int32_t* topk_idx, float* topk_w, void* out, char* ws, const WsLayout& L,
                     hipStream_t s) {
  Plan p = plan_at(ws, L);
  void* h = ws + L.h;
  float* y_sorted = reinterpret_cast<float*>(ws + L.y_sorted);

  hipError_t e = hipSuccess;
  if (w_router) e = launch_router_logits(x, w_router, logits, dm.T, dm.d, dm.E, dm.act, s);
  if (!dm.fp8 && gemv_down_combine_t1_ok(dm)) {
    // single token: one-wave route+plan, gate/up GEMV (4-bit: one kernel for
    // both), down GEMV + combine (fused unless the expert outputs are
    // normalised first)
    if (gemv_gate_up_t1_routed_ok(dm)) {
      if (e == hipSuccess)
        e = launch_gemv_gate_up_t1_routed(dm, logits, x, p, w, h, topk_idx, topk_w, s);
    } else {
      if (e == hipSuccess) e = launch_route_plan_t1(logits, dm.E, dm.k, topk_idx, topk_w, p, s);
      if (e == hipSuccess) e = launch_gemv_gate_up(dm, x, p, w, h, s);
    }
    if (!dm.expert_norm) {
      if (e == hipSuccess)
        e = launch_gemv_down_combine_t1(dm, h, p, topk_idx, topk_w, w, out, s);
    } else {
      if (e == hipSuccess) e = launch_gemv_down(dm, h, p, w, y_sorted, s);
      if (e == hipSuccess) e = launch_combine(dm, y_sorted, p.dest_row, topk_w, out, s);
    }
    return e;
  }
  if (dm.T <= kDecodeMaxT) {
    if (e == hipSuccess)
      e = launch_route_permute_small(logits, dm.T, dm.E, dm.k, topk_idx, topk_w, p, s);
  } else {
    if (e == hipSuccess) e = launch_route_topk(logits, dm.T, dm.E, dm.k, topk_idx, topk_w, s);
    if (e == hipSuccess) e = launch_permute(topk_idx, dm.T, dm.E, dm.k, p, true, s);
  }
  if (e == hipSuccess) e = run_expert_ffn(dm, x, p, w, ws, L, y_sorted, s);
  if (e == hipSuccess) e = launch_combine(dm, y_sorted, p.dest_row, topk_w, out, s);
  return e;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status_t moe_workspace_size(const moe_dims_t* dims, size_t* bytes) {
  Dims dm;
  moe_status_t st = check_dims(dims, &dm);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  *bytes = ws_layout(dm).total;
  return MOE_OK;
}

moe_status_t moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_idx,
                       float* topk_w, moe_stream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
  if (!routing_shape_ok(T, E, k)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(logits) || !aligned16(topk_idx) || !aligned16(topk_w))
    return MOE_ERR_INVALID_ARGUMENT;
  return device_status(launch_route_topk(logits, T, E, k, topk_idx, topk_w, (hipStream_t)stream));
}

moe_status_t moe_permute(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_src,
                         int32_t* dest_row, moe_stream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
  if (!routing_shape_ok(T, E, k)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !counts || !offsets || !sorted_src || !dest_row) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(topk_idx) || !aligned16(counts) || !aligned16(offsets) || !aligned16(sorted_src) ||
      !aligned16(dest_row))
    return MOE_ERR_INVALID_ARGUMENT;
  Plan p{counts, offsets, sorted_src, dest_row, nullptr, nullptr, nullptr, nullptr, nullptr};
  return device_status(launch_permute(topk_idx, T, E, k, p, false, (hipStream_t)stream));
}

moe_status_t moe_expert_ffn(const moe_dims_t* dims, const void* x, const int32_t* offsets,
                            const int32_t* sorted_src, const moe_expert_weights_t* weights,
                            float* y_sorted, void* workspace, size_t workspace_bytes,
                            moe_stream_t stream) {
  Dims dm;
  moe_status_t st = check_dims(dims, &dm);
  if (st != MOE_OK) return st;
  if (dm.T == 0) return MOE_OK;
  Weights w;
  if ((st = check_weights(weights, dm, &w)) != MOE_OK) return st;
  if (!x || !offsets || !sorted_src || !y_sorted || !workspace) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(offsets) || !aligned16(sorted_src) || !aligned16(y_sorted) ||
      (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  const WsLayout L = ws_layout(dm);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = (hipStream_t)stream;
  Plan p = plan_at(workspace, L);
  p.offsets = const_cast<int*>(offsets);
  p.sorted_src = const_cast<int*>(sorted_src);
  hipError_t e = launch_plan_from_offsets(offsets, dm.E, (int)dm.Tk(), p, s);
  if (e == hipSuccess)
    e = run_expert_ffn(dm, x, p, w, static_cast<char*>(workspace), L, y_sorted, s);
  return device_status(e);
}

moe_status_t moe_combine(const moe_dims_t* dims, const float* y_sorted, const int32_t* dest_row,
                         const float* topk_w, void* out, moe_stream_t stream) {
  Dims dm;
  moe_status_t st = check_dims(dims, &dm);
  if (st != MOE_OK) return st;
  if (dm.T == 0) return MOE_OK;
  if (!y_sorted || !dest_row || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y_sorted) || !aligned16(dest_row) || !aligned16(topk_w) || !aligned16(out))
    return MOE_ERR_INVALID_ARGUMENT;
  return device_status(launch_combine(dm, y_sorted, dest_row, topk_w, out, (hipStream_t)stream));
}

moe_status_t moe_layer_forward(const moe_dims_t* dims, const void* x, const void* w_router,
                               float* logits, const moe_expert_weights_t* weights,
                               int32_t* topk_idx, float* topk_w, void* out, void* workspace,
                               size_t workspace_bytes, moe_stream_t stream) {
  Dims dm;
  Weights w;
  moe_status_t st = check_layer_args(dims, x, w_router, logits, weights, topk_idx, topk_w, out, &dm, &w);
  if (st != MOE_OK || dm.T == 0) return st;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  const WsLayout L = ws_layout(dm);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return device_status(run_layer(dm, w, x, w_router, logits, topk_idx, topk_w, out,
                                 static_cast<char*>(workspace), L, (hipStream_t)stream));
}

moe_status_t moe_layer_forward_noalloc(const moe_dims_t* dims, const void* x, const void* w_router,
                                       float* logits, const moe_expert_weights_t* weights,
                                       int32_t* topk_idx, float* topk_w, void* out,
                                       moe_stream_t stream) {
  Dims dm;
  Weights w;
  moe_status_t st = check_layer_args(dims, x, w_router, logits, weights, topk_idx, topk_w, out, &dm, &w);
  if (st != MOE_OK || dm.T == 0) return st;
  const WsLayout L = ws_layout(dm);
  if (L.total > kScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* scratch = nullptr;
  hipError_t e = scratch_for_current_device(&scratch);
  if (e != hipSuccess) return device_status(e);
  return device_status(run_layer(dm, w, x, w_router, logits, topk_idx, topk_w, out,
                                 static_cast<char*>(scratch), L, (hipStream_t)stream));
}

moe_status_t moe_quantize_mxfp8(const void* x, int64_t rows, int32_t K, uint8_t* q,
                                uint8_t* scales, moe_stream_t stream) {
  if (rows < 0 || K <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (K % 32 != 0) return MOE_ERR_UNSUPPORTED;
  // one thread per 32-element block: at most 2^31 threads in the grid
  if (rows > ((int64_t)1 << 31) / (K / 32)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(q)) return MOE_ERR_INVALID_ARGUMENT;
  return device_status(launch_quantize_mxfp8(x, rows, K, q, scales, (hipStream_t)stream));
}

moe_status_t moe_debug_check(uint32_t* violations) {
  if (!violations) return MOE_ERR_INVALID_ARGUMENT;
  *violations = 0;
#ifdef MOE_DEBUG_CHECKS
  unsigned f = 0;
  hipError_t e = dbg_take_route(&f);
  if (e == hipSuccess) e = dbg_take_permute(&f);
  if (e == hipSuccess) e = dbg_take_gemv(&f);
  if (e == hipSuccess) e = dbg_take_combine(&f);
  if (e == hipSuccess) e = dbg_take_grouped_gemm(&f);
  *violations = f;
  return device_status(e);
#else
  return MOE_ERR_UNSUPPORTED;
#endif
}

const char* moe_status_string(moe_status_t status) {
  // A C caller may pass any int; in C++ loading an enum outside its declared
  // values is undefined, so the argument's bits are read as an int first.
  int32_t code = 0;
  static_assert(sizeof(status) == sizeof(code), "moe_status_t is an int");
  std::memcpy(&code, &status, sizeof code);
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_DEVICE: return "HIP device error";
  }
  return "unknown status";
}

int32_t moe_last_device_error(void) { return g_last_device_error; }

moe_status_t moe_timing_start(void) {
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  if (!t.created) {
    t.ev0.resize(kMaxTimed);
    t.ev1.resize(kMaxTimed);
    t.names.resize(kMaxTimed);
    for (int i = 0; i < kMaxTimed; ++i) {
      hipError_t e0 = hipEventCreate(&t.ev0[i]);
      hipError_t e1 = hipEventCreate(&t.ev1[i]);
      if (e0 != hipSuccess || e1 != hipSuccess) return device_status(e0 != hipSuccess ? e0 : e1);
    }
    t.created = true;
  }
  t.used = 0;
  ++t.generation;
  t.enabled.store(true, std::memory_order_relaxed);
  return MOE_OK;
}

moe_status_t moe_timing_stop(void) {
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  t.enabled.store(false, std::memory_order_relaxed);
  return MOE_OK;
}

moe_status_t moe_timing_query(const char* kernel, int32_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) return MOE_ERR_INVALID_ARGUMENT;
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  int n = 0;
  double ms = 0.0;
  for (int i = 0; i < t.used; ++i) {
    if (t.names[i] != kernel) continue;
    hipError_t e = hipEventSynchronize(t.ev1[i]);
    if (e != hipSuccess) return device_status(e);
    float v = 0.f;
    e = hipEventElapsedTime(&v, t.ev0[i], t.ev1[i]);
    if (e != hipSuccess) return device_status(e);
    ms += v;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return MOE_OK;
}

moe_status_t moe_timing_names(char* buf, size_t buf_bytes) {
  if (!buf || buf_bytes == 0) return MOE_ERR_INVALID_ARGUMENT;
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  std::vector<std::string> seen;
  std::string all;
  for (int i = 0; i < t.used; ++i) {
    bool dup = false;
    for (auto& s : seen) dup |= (s == t.names[i]);
    if (dup) continue;
    seen.push_back(t.names[i]);
    if (!all.empty()) all += ",";
    all += t.names[i];
  }
  if (all.size() + 1 > buf_bytes) return MOE_ERR_INVALID_ARGUMENT;
  for (size_t i = 0; i < all.size(); ++i) buf[i] = all[i];
  buf[all.size()] = '\0';
  return MOE_OK;
}

}  // extern "C"
