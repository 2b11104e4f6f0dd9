// Host-side internals shared by the launchers and the C ABI: workspace plan,
// launch parameters and the per-kernel event timer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Storage formats, numbered as moe_dtype_t.
enum Fmt : int { kF32 = 0, kBF16 = 1, kMXFP4 = 2, kNVFP4 = 3 };

// The two 4-bit weight formats share codes and kernels; they differ in the
// block scales (E8M0 per 32 elements vs E4M3 per 16 plus an fp32 scale per
// matrix).
constexpr bool is_fp4(int wf) { return wf == kMXFP4 || wf == kNVFP4; }

// Rows per m-tile of the grouped MFMA GEMMs; the tile list in the workspace
// is sized for this value.  Each m-tile entry holds kMtileInts ints:
// expert, first row, rows in the tile, index of the expert's first m-tile,
// number of m-tiles of the expert, 3 unused.
constexpr int kGemmBM = 128;
constexpr int kMtileInts = 8;

// Largest T routed and permuted by the single-workgroup decode kernel.
constexpr int kDecodeMaxT = 16;

// Smallest T that takes the grouped MFMA GEMMs (bf16 activations).  Below it
// the GEMV kernels stream each active expert's weights once per layer and are
// faster; measured at d=6144, E=256, k=8, f=2816 on MI355X: T=32 GEMV 2.64 ms
// vs MFMA 2.83 ms, T=64 GEMV 3.90 ms vs MFMA 3.71 ms (bf16 weights; MX-FP4
// crosses over between the same T).
constexpr int kGemmMinT = 48;

struct Dims {
  int T, d, E, k, f, act, wfmt;
  bool fp8 = false;          // MXFP8 activations on the scaled MFMA
  bool expert_norm = false;  // RMS-normalise each expert output before the combine
  long long Tk() const { return (long long)T * k; }
};

struct Weights {
  const void *wg, *wu, *wd;
  const uint8_t *sg, *su, *sd;  // 4-bit block scales
  const float *tg, *tu, *td;    // NVFP4 matrix scales [E]
};

// Workspace layout (byte offsets, each 256-aligned).
struct WsLayout {
  size_t counts, offsets, sorted_src, dest_row, active, num_active, slot_info, mtiles, num_mtiles;
  size_t h, y_sorted;
  size_t xq, xs, hq, hs;  // FP8 activations: x and h as MXFP8 (values, E8M0 scales)
  size_t total;
};
WsLayout ws_layout(const Dims& dm);

// Routing plan pointers in the workspace (device).
struct Plan {
  int* counts;
  int* offsets;
  int* sorted_src;
  int* dest_row;
  int* active;      // [E] experts with at least one routed pair, ascending
  int* num_active;  // [1]
  int* slot_info;   // [E][4] per active slot: expert, first row, rows, 0
  int* mtiles;      // [kMtileInts * max_mtiles] m-tile entries (see kMtileInts)
  int* num_mtiles;  // [1]
};

// Library-owned scratch (scratch.hip) for moe_layer_forward_noalloc: its
// size, and the current device's copy, looked up on the first call per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_for_current_device(void** ptr);

// Debug builds: each kernel file's bounds-check flag word, OR-ed into *flags
// and cleared (synchronous).  No-ops in release builds.
hipError_t dbg_take_route(unsigned* flags);
hipError_t dbg_take_permute(unsigned* flags);
hipError_t dbg_take_gemv(unsigned* flags);
hipError_t dbg_take_combine(unsigned* flags);
hipError_t dbg_take_grouped_gemm(unsigned* flags);

// Per-kernel event timing (abi.cpp).  Bracket every launch with it.
struct LaunchTimer {
  LaunchTimer(const char* name, hipStream_t s);
  ~LaunchTimer();
  const char* name_;
  hipStream_t s_;
  int slot_;
  unsigned gen_;  // timing generation the slot was taken in
};

// Launchers: each queues one kernel on `s` and returns hipGetLastError().
hipError_t launch_router_logits(const void* x, const void* w_r, float* logits, int T, int d,
                                int E, int act, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int* topk_idx,
                             float* topk_w, hipStream_t s);
// Route and permute in one workgroup for T <= kDecodeMaxT (T*k <= 1024).
hipError_t launch_route_permute_small(const float* logits, int T, int E, int k, int* topk_idx,
                                      float* topk_w, const Plan& p, hipStream_t s);
// T == 1: one wave routes the token and writes the whole plan.
hipError_t launch_route_plan_t1(const float* logits, int E, int k, int* topk_idx, float* topk_w,
                                const Plan& p, hipStream_t s);
hipError_t launch_permute(const int* topk_idx, int T, int E, int k, const Plan& p,
                          bool with_lists, hipStream_t s);
hipError_t launch_plan_from_offsets(const int* offsets, int E, int Tk, const Plan& p, hipStream_t s);
hipError_t launch_gemv_gate_up(const Dims& dm, const void* x, const Plan& p, const Weights& w,
                               void* h, hipStream_t s);
hipError_t launch_gemv_down(const Dims& dm, const void* h, const Plan& p, const Weights& w,
                            float* y_sorted, hipStream_t s);
// T == 1 with 4-bit weights: routing (as launch_route_plan_t1, whose outputs
// and plan it writes) folded into the gate/up GEMV, saving a launch.
bool gemv_gate_up_t1_routed_ok(const Dims& dm);
hipError_t launch_gemv_gate_up_t1_routed(const Dims& dm, const float* logits, const void* x,
                                         const Plan& p, const Weights& w, void* h, int* topk_idx,
                                         float* topk_w, hipStream_t s);
// T == 1 (k <= 16, one segment per row): down projection and weighted
// combine in one kernel, writing `out` directly.
bool gemv_down_combine_t1_ok(const Dims& dm);
hipError_t launch_gemv_down_combine_t1(const Dims& dm, const void* h, const Plan& p,
                                       const int* topk_idx, const float* topk_w,
                                       const Weights& w, void* out, hipStream_t s);
// Grouped MFMA GEMMs for many tokens per expert (bf16 or MX-FP4 weights,
// bf16 activations).  gate/up: h = silu(x W_g^T) * (x W_u^T); down: y = h W_d^T.
bool grouped_gemm_ok(const Dims& dm);
size_t grouped_gemm_max_mtiles(const Dims& dm);
hipError_t launch_gg_gate_up(const Dims& dm, const void* x, const Plan& p, const Weights& w,
                             void* h, hipStream_t s);
// FP8 activations (MXFP8): with MX-FP4 weights on the scaled MFMA, with NVFP4
// weights as bf16 values on bf16 MFMA.
bool fp8_path_ok(const Dims& dm);
hipError_t launch_quantize_mxfp8(const void* x, long long rows, int K, uint8_t* q, uint8_t* qs,
                                 hipStream_t s);
// bf16 x rounded to the MXFP8 grid, kept as bf16 (FP8 activations with NVFP4
// weights: the gate/up GEMM then rounds h the same way, from fp32).
hipError_t launch_round_mxfp8(const void* x, long long rows, int K, void* y, hipStream_t s);
hipError_t launch_gg_f8_gate_up(const Dims& dm, const uint8_t* xq, const uint8_t* xs, const Plan& p,
                                const Weights& w, uint8_t* hq, uint8_t* hs, hipStream_t s);
hipError_t launch_gg_f8_down(const Dims& dm, const uint8_t* hq, const uint8_t* hs, const Plan& p,
                             const Weights& w, float* y_sorted, hipStream_t s);
hipError_t launch_gg_down(const Dims& dm, const void* h, const Plan& p, const Weights& w,
                          float* y_sorted, hipStream_t s);
hipError_t launch_combine(const Dims& dm, const float* y_sorted, const int* dest_row,
                          const float* topk_w, void* out, hipStream_t s);

}  // namespace moe
