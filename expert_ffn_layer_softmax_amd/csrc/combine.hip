// Weighted combine: out[t] = sum_j topk_w[t][j] * y_sorted[dest_row[t*k+j]].
//
// The selected experts' outputs are scaled by their normalised routing
// weights and summed (TensorSharp Muse Spark report, "Performance" section).
// The sum runs in fp32 in slot order and is rounded once to the activation
// dtype, since bf16 partial sums were tied to accuracy drift (same report,
// "Answer quality").  HBM-bound: each y_sorted row is read once.
#include "device.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kMaxK = 64;

// Grid (T, row chunks of 1024 values); each thread one float4 of the row.
template <int ACT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_sorted,
                                                      const int* __restrict__ dest_row,
                                                      const float* __restrict__ topk_w,
                                                      void* __restrict__ out, int d, int k) {
  __shared__ int rows[kMaxK];
  __shared__ float wts[kMaxK];
  const int t = blockIdx.y;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = dest_row[(size_t)t * k + threadIdx.x];
    wts[threadIdx.x] = topk_w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const int n4 = d >> 2;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float4 y = reinterpret_cast<const float4*>(y_sorted + (size_t)rows[j] * d)[i];
      const float w = wts[j];
      acc.x = fmaf(w, y.x, acc.x);
      acc.y = fmaf(w, y.y, acc.y);
      acc.z = fmaf(w, y.z, acc.z);
      acc.w = fmaf(w, y.w, acc.w);
    }
    if constexpr (ACT == kF32) {
      reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (size_t)t * d)[i] = acc;
    } else {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
      pk.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
      reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * d)[i] = pk;
    }
  }
}

}  // namespace

hipError_t launch_combine(const Dims& dm, const float* y_sorted, const int* dest_row,
                          const float* topk_w, void* out, hipStream_t s) {
  LaunchTimer tm("combine", s);
  const dim3 grid((unsigned)((dm.d / 4 + 255) / 256), (unsigned)dm.T), block(256);
  if (dm.act == kF32)
    combine_kernel<kF32><<<grid, block, 0, s>>>(y_sorted, dest_row, topk_w, out, dm.d, dm.k);
  else
    combine_kernel<kBF16><<<grid, block, 0, s>>>(y_sorted, dest_row, topk_w, out, dm.d, dm.k);
  return hipGetLastError();
}

}  // namespace moe
