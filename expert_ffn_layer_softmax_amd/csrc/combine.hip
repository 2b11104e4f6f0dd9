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
    rows[threadIdx.x] = dbg_idx(dest_row[(size_t)t * k + threadIdx.x], (int)gridDim.y * k, kDbgDestRow);
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

// With per-expert normalisation: each selected expert's output row is divided
// by its root mean square over d (plus kNormEps inside the root) before the
// weighted sum: the second reading of the report's normalise-then-combine
// step (same report, "Performance").  One block of NT threads per token.
// Pass 1: the block's waves share the k rows' sums of squares; with
// P = max(1, waves / k) waves per row, wave w takes row w % k and every P-th
// float4 column from (w / k) * 64 + lane on, a lane sums its columns in
// order, the wave sums its lanes (fixed xor tree), and the P partials are
// added in part order.  Pass 2 combines each float4 column with weights
// w_j / rms_j in slot order, four rows' loads in flight at a time; the rows
// are fresh in L2 from pass 1.
constexpr float kNormEps = 1e-6f;

__device__ __forceinline__ float sumsq4(float4 v, float acc) {
  return fmaf(v.w, v.w, fmaf(v.z, v.z, fmaf(v.y, v.y, fmaf(v.x, v.x, acc))));
}

template <int ACT, int NT>
__global__ __launch_bounds__(NT) void combine_norm_kernel(const float* __restrict__ y_sorted,
                                                          const int* __restrict__ dest_row,
                                                          const float* __restrict__ topk_w,
                                                          void* __restrict__ out, int d, int k) {
  constexpr int kWaves = NT / kWave;
  __shared__ int rows[kMaxK];
  __shared__ float wts[kMaxK];
  __shared__ float part[kWaves > kMaxK ? kWaves : kMaxK];
  const int t = blockIdx.x;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x < k)
    rows[threadIdx.x] = dbg_idx(dest_row[(size_t)t * k + threadIdx.x], (int)gridDim.x * k, kDbgDestRow);
  __syncthreads();
  const int n4 = d >> 2;
  const int P = kWaves > k ? kWaves / k : 1;  // waves per row
  const int stride = P * kWave;
  for (int w = wave; w < k * P; w += kWaves) {
    const int j = w % k;
    const float4* y = reinterpret_cast<const float4*>(y_sorted + (size_t)rows[j] * d);
    float ss = 0.f;
    int i = (w / k) * kWave + lane;
    for (; i + 3 * stride < n4; i += 4 * stride) {
      const float4 v0 = y[i], v1 = y[i + stride], v2 = y[i + 2 * stride], v3 = y[i + 3 * stride];
      ss = sumsq4(v3, sumsq4(v2, sumsq4(v1, sumsq4(v0, ss))));
    }
    for (; i < n4; i += stride) ss = sumsq4(y[i], ss);
    ss = wave_sum(ss);
    if (lane == 0) part[w] = ss;  // w < k * P <= max(kWaves, k)
  }
  __syncthreads();
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    float ss = 0.f;
    for (int q = 0; q < P; ++q) ss += part[q * k + j];
    wts[j] = topk_w[(size_t)t * k + j] / sqrtf(ss / (float)d + kNormEps);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n4; i += NT) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int j = 0;
    for (; j + 4 <= k; j += 4) {
      float4 y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = reinterpret_cast<const float4*>(y_sorted + (size_t)rows[j + q] * d)[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float w = wts[j + q];
        acc.x = fmaf(w, y[q].x, acc.x);
        acc.y = fmaf(w, y[q].y, acc.y);
        acc.z = fmaf(w, y[q].z, acc.z);
        acc.w = fmaf(w, y[q].w, acc.w);
      }
    }
    for (; j < k; ++j) {
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

// Register-resident variant for k <= KMAX and d <= 4 * C * NT: each thread
// loads its C float4 columns of all k rows once, keeps them in registers for
// both passes, so each row is read from HBM exactly once.  Row sums of
// squares: a lane sums its columns in order, the wave tree, then the NT / 64
// wave partials in wave order.
template <int ACT, int NT, int KMAX, int C>
__global__ __launch_bounds__(NT) void combine_norm_reg_kernel(const float* __restrict__ y_sorted,
                                                              const int* __restrict__ dest_row,
                                                              const float* __restrict__ topk_w,
                                                              void* __restrict__ out, int d, int k) {
  constexpr int kWaves = NT / kWave;
  __shared__ float part[KMAX][kWaves];
  __shared__ float wts[KMAX];
  const int t = blockIdx.x;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int n4 = d >> 2;
  float4 v[KMAX][C];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int row = j < k ? dbg_idx(dest_row[(size_t)t * k + j], (int)gridDim.x * k, kDbgDestRow) : 0;
    const float4* y = reinterpret_cast<const float4*>(y_sorted + (size_t)row * d);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int i = threadIdx.x + c * NT;
      v[j][c] = (j < k && i < n4) ? y[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) ss = sumsq4(v[j][c], ss);
      ss = wave_sum(ss);
      if (lane == 0) part[j][wave] = ss;
    }
  }
  __syncthreads();
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    float ss = 0.f;
    for (int q = 0; q < kWaves; ++q) ss += part[j][q];
    wts[j] = topk_w[(size_t)t * k + j] / sqrtf(ss / (float)d + kNormEps);
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int i = threadIdx.x + c * NT;
    if (i >= n4) break;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const float w = wts[j];
        acc.x = fmaf(w, v[j][c].x, acc.x);
        acc.y = fmaf(w, v[j][c].y, acc.y);
        acc.z = fmaf(w, v[j][c].z, acc.z);
        acc.w = fmaf(w, v[j][c].w, acc.w);
      }
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

template <int ACT>
void launch_combine_norm(const Dims& dm, const float* y_sorted, const int* dest_row,
                         const float* topk_w, void* out, hipStream_t s) {
  // Many tokens, k <= 8 and d <= 8192: rows read once, held in registers.
  const int n4 = dm.d / 4;
  const bool reg = dm.T >= 256 && dm.k <= 8;
  if (reg && n4 <= 2 * 256) {
    combine_norm_reg_kernel<ACT, 256, 8, 2><<<dim3((unsigned)dm.T), dim3(256), 0, s>>>(
        y_sorted, dest_row, topk_w, out, dm.d, dm.k);
    return;
  }
  if (reg && n4 <= 2 * 1024) {
    combine_norm_reg_kernel<ACT, 1024, 8, 2><<<dim3((unsigned)dm.T), dim3(1024), 0, s>>>(
        y_sorted, dest_row, topk_w, out, dm.d, dm.k);
    return;
  }
  // Otherwise two passes over the rows (the second from L2).  Few tokens: one
  // wide block per token (the chip is mostly idle, latency rules; measured
  // faster than the register-resident kernel at T = 1 and 16); many: 256
  // threads, several blocks per CU.
  if (dm.T < 256)
    combine_norm_kernel<ACT, 1024><<<dim3((unsigned)dm.T), dim3(1024), 0, s>>>(
        y_sorted, dest_row, topk_w, out, dm.d, dm.k);
  else
    combine_norm_kernel<ACT, 256><<<dim3((unsigned)dm.T), dim3(256), 0, s>>>(
        y_sorted, dest_row, topk_w, out, dm.d, dm.k);
}

}  // namespace

hipError_t launch_combine(const Dims& dm, const float* y_sorted, const int* dest_row,
                          const float* topk_w, void* out, hipStream_t s) {
  LaunchTimer tm("combine", s);
  if (dm.expert_norm) {
    if (dm.act == kF32)
      launch_combine_norm<kF32>(dm, y_sorted, dest_row, topk_w, out, s);
    else
      launch_combine_norm<kBF16>(dm, y_sorted, dest_row, topk_w, out, s);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((dm.d / 4 + 255) / 256), (unsigned)dm.T), block(256);
  if (dm.act == kF32)
    combine_kernel<kF32><<<grid, block, 0, s>>>(y_sorted, dest_row, topk_w, out, dm.d, dm.k);
  else
    combine_kernel<kBF16><<<grid, block, 0, s>>>(y_sorted, dest_row, topk_w, out, dm.d, dm.k);
  return hipGetLastError();
}

MOE_DBG_TAKE_DEFINE(dbg_take_combine)

}  // namespace moe
