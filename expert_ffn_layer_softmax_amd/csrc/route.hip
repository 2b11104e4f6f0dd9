// Router: logits GEMV (optional in-path stage) and top-k with renormalised
// softmax weights.
//
// The layer sends each token to k of its E experts (SGLang-TorchTPU on TPU v7
// page, "Introduction": 8 of 256 per layer).  The combine uses normalised
// weights (TensorSharp Muse Spark report, "Performance" section); the reading
// taken is a softmax over all E logits renormalised over the selected k, which
// equals a softmax over the k selected logits.
#include <float.h>
#include <limits.h>

#include "device.h"
#include "internal.h"

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

// (value, index) order used for selection: larger value first, equal values
// by smaller index.  No NaN in the domain, so this is a total order.
__device__ __forceinline__ bool beats(float v, int i, float bv, int bi) {
  return bi == INT_MAX ? (i != INT_MAX) : (i != INT_MAX && (v > bv || (v == bv && i < bi)));
}

// One wave per token; lane l holds logits l, l+64, ... (VPL of them).  k
// rounds of wave argmax; the winner is marked taken.  Lane j keeps slot j.
template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[VPL];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    if (e < E) {
      v[i] = row[e];
    } else {
      v[i] = -FLT_MAX;
      taken |= 1u << i;
    }
  }
  float sel_v = 0.f;
  int sel_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      // indices grow with i, so a strict '>' keeps the lower index on ties
      if (!((taken >> i) & 1u) && (bi == INT_MAX || v[i] > bv)) {
        bv = v[i];
        bi = lane + kWave * i;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (beats(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      sel_v = bv;
      sel_i = bi;
    }
  }
  // Renormalised softmax over the k winners (slot 0 holds the maximum).
  const float l0 = __shfl(sel_v, 0, kWave);
  float ex = 0.f;
  if (lane < k) ex = (sel_v == l0) ? 1.0f : expf(sel_v - l0);
  const float sum = wave_sum(ex);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = sel_i;
    topk_w[(size_t)t * k + lane] = ex / sum;
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

}  // namespace moe
