// Grouping of (token, slot) pairs by expert: a stable counting sort in one
// workgroup.  Integer-only and atomic-order independent, so bit-exact.
//
// Beyond the four public outputs it can also write the execution plan the
// expert kernels read: the ascending list of experts that received at least
// one pair, and the list of m-tiles (expert, first row) of kGemmBM rows for
// the grouped MFMA GEMMs.  Nothing here is read back by the host.
#include "device.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;  // 16 waves
constexpr int kMaxE = 1024;

// Active-expert list and m-tile list from per-expert counts (thread e holds
// counts[e]; threads >= E hold 0).  Barriers inside: all threads call.
__device__ void write_lists(int c, int E, const Plan& p, int* tmp) {
  const int e = threadIdx.x;
  int total = 0;
  const int nz = (e < E && c > 0) ? 1 : 0;
  const int pos = block_exclusive_scan(nz, tmp, &total);
  if (nz) p.active[pos] = e;
  if (threadIdx.x == 0) *p.num_active = total;
  const int nt = (e < E) ? (c + kGemmBM - 1) / kGemmBM : 0;
  const int tpos = block_exclusive_scan(nt, tmp, &total);
  for (int i = 0; i < nt; ++i) {
    p.mtiles[2 * (tpos + i)] = e;
    p.mtiles[2 * (tpos + i) + 1] = i * kGemmBM;
  }
  if (threadIdx.x == 0) *p.num_mtiles = total;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int* __restrict__ topk_idx,
                                                               int N, int E, Plan p,
                                                               int with_lists) {
  __shared__ int hist[kMaxE];
  __shared__ int cursor[kMaxE];
  __shared__ int wave_cnt[kPermThreads / kWave][kMaxE];
  __shared__ int tmp[32];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;

  for (int i = tid; i < E; i += kPermThreads) {
    hist[i] = 0;
#pragma unroll
    for (int w = 0; w < kPermThreads / kWave; ++w) wave_cnt[w][i] = 0;
  }
  __syncthreads();
  for (int q = tid; q < N; q += kPermThreads) {
    const int e = min(max(topk_idx[q], 0), E - 1);
    atomicAdd(&hist[e], 1);  // integer: order independent
  }
  __syncthreads();

  const int c = tid < E ? hist[tid] : 0;
  int total = 0;
  const int excl = block_exclusive_scan(c, tmp, &total);
  if (tid < E) {
    p.counts[tid] = c;
    p.offsets[tid] = excl;
    cursor[tid] = excl;
  }
  if (tid == 0) p.offsets[E] = total;
  if (with_lists) write_lists(c, E, p, tmp);
  __syncthreads();

  // Stable scatter, 1024 pairs per round in flat-id order.  Inside a wave,
  // lanes with the same expert are found by a ballot per key bit; across
  // waves, by per-wave counts in LDS.
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = 0; base < N; base += kPermThreads) {
    const int q = base + tid;
    const bool valid = q < N;
    const int e = valid ? min(max(topk_idx[q], 0), E - 1) : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(valid && bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt_mask);
    const int cnt = __popcll(peers);
    const bool leader = valid && rank == 0;
    if (leader) wave_cnt[wave][e] = cnt;
    __syncthreads();
    if (valid) {
      int prefix = 0;
      for (int w = 0; w < wave; ++w) prefix += wave_cnt[w][e];
      const int pos = cursor[e] + prefix + rank;
      p.sorted_src[pos] = q;
      p.dest_row[q] = pos;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&cursor[e], cnt);
      wave_cnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kPermThreads) void plan_kernel(const int* __restrict__ offsets, int E,
                                                            Plan p) {
  __shared__ int tmp[32];
  const int e = threadIdx.x;
  const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
  write_lists(c, E, p, tmp);
}

}  // namespace

hipError_t launch_permute(const int* topk_idx, int T, int E, int k, const Plan& p,
                          bool with_lists, hipStream_t s) {
  LaunchTimer tm("permute", s);
  permute_kernel<<<1, kPermThreads, 0, s>>>(topk_idx, T * k, E, p, with_lists ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_plan_from_offsets(const int* offsets, int E, const Plan& p, hipStream_t s) {
  LaunchTimer tm("plan", s);
  plan_kernel<<<1, kPermThreads, 0, s>>>(offsets, E, p);
  return hipGetLastError();
}

}  // namespace moe
