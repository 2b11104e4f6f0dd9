// Router: logits GEMV (optional in-path stage) and top-k with renormalised
// softmax weights (selection rule: route_dev.h).
#include "device.h"
#include "internal.h"
#include "route_dev.h"

namespace moe {
namespace {

// logits[t][e] = sum_i x[t][i] * w_r[e][i], fp32 accumulation.
// One block of 4 waves per token; each wave takes experts e = wave, wave+4, ...
template <int ACT>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ xv,
                                                            const void* __restrict__ wv,
                                                            float* __restrict__ logits, int T,
                                                            int d, int E) {
  const int t = blockIdx.x;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  constexpr int CE = (ACT == kF32) ? 4 : 8;  // elements per 16-byte chunk
  const int nchunks = d / CE;
  const char* xrow = reinterpret_cast<const char*>(xv) + (size_t)t * d * (ACT == kF32 ? 4 : 2);
  for (int e = wave; e < E; e += 4) {
    const char* wrow = reinterpret_cast<const char*>(wv) + (size_t)e * d * (ACT == kF32 ? 4 : 2);
    float acc = 0.f;
    for (int c = lane; c < nchunks; c += kWave) {
      u32x4 a = ld16(xrow + (size_t)c * 16);
      u32x4 b = ld16(wrow + (size_t)c * 16);
      if (ACT == kF32) {
        acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
        acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
        acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
        acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
      } else {
        const uint32_t aa[4] = {a.x, a.y, a.z, a.w}, bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = fmaf(bf16_lo(aa[i]), bf16_lo(bb[i]), acc);
          acc = fmaf(bf16_hi(aa[i]), bf16_hi(bb[i]), acc);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[(size_t)t * E + e] = acc;
  }
}

// One wave per token, four tokens per block.
template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int sel_i;
  float sel_w;
  route_token<VPL>(logits + (size_t)t * E, E, k, sel_i, sel_w);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = sel_i;
    topk_w[(size_t)t * k + lane] = sel_w;
  }
}

}  // namespace

hipError_t launch_router_logits(const void* x, const void* w_r, float* logits, int T, int d,
                                int E, int act, hipStream_t s) {
  LaunchTimer tm("router_logits", s);
  if (act == kF32)
    router_logits_kernel<kF32><<<T, 256, 0, s>>>(x, w_r, logits, T, d, E);
  else
    router_logits_kernel<kBF16><<<T, 256, 0, s>>>(x, w_r, logits, T, d, E);
  return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int* topk_idx,
                             float* topk_w, hipStream_t s) {
  LaunchTimer tm("route_topk", s);
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    route_topk_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, topk_idx, topk_w);
  else if (E <= 128)
    route_topk_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, topk_idx, topk_w);
  else if (E <= 256)
    route_topk_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, topk_idx, topk_w);
  else if (E <= 512)
    route_topk_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, topk_idx, topk_w);
  else
    route_topk_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, topk_idx, topk_w);
  return hipGetLastError();
}

MOE_DBG_TAKE_DEFINE(dbg_take_route)

}  // namespace moe
