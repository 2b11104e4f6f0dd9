// Grouping of (token, slot) pairs by expert: a stable counting sort in one
// workgroup.  Integer-only and independent of atomic order, so bit-exact.
//
// Besides the four public outputs it can write the execution plan the expert
// kernels read: the ascending list of experts with at least one pair, a
// per-slot (expert, first row, rows) table, and the list of m-tiles of up to
// kGemmBM rows for the grouped MFMA GEMMs (entry layout: internal.h).  Nothing here is read
// back by the host.
#include "device.h"
#include "internal.h"
#include "route_dev.h"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;  // 16 waves
constexpr int kMaxE = 1024;

struct PermShared {
  int wave_cnt[kPermThreads / kWave][kMaxE];  // per wave: counts, then cursors
  int tmp[32];
};

// Active-expert list, slot table and m-tile list from per-expert counts
// (thread e holds counts[e] and its exclusive prefix `first`; threads >= E
// hold 0).  Contains barriers: every thread calls.
__device__ void write_lists(int c, int first, int E, const Plan& p, int* tmp) {
  const int e = threadIdx.x;
  int total = 0;
  const int nz = (e < E && c > 0) ? 1 : 0;
  const int pos = block_exclusive_scan(nz, tmp, &total);
  if (nz) {
    p.active[pos] = e;
    p.slot_info[4 * pos + 0] = e;
    p.slot_info[4 * pos + 1] = first;
    p.slot_info[4 * pos + 2] = c;
    p.slot_info[4 * pos + 3] = 0;
  }
  if (threadIdx.x == 0) *p.num_active = total;
  const int nt = (e < E) ? (c + kGemmBM - 1) / kGemmBM : 0;
  const int tpos = block_exclusive_scan(nt, tmp, &total);
  for (int i = 0; i < nt; ++i) {
    int* m = p.mtiles + kMtileInts * (tpos + i);
    m[0] = e;
    m[1] = first + i * kGemmBM;
    m[2] = min(kGemmBM, c - i * kGemmBM);
    m[3] = tpos;
    m[4] = nt;
  }
  if (threadIdx.x == 0) *p.num_mtiles = total;
}

// Counting sort of N >= 1 keys (key(q) in [0, E) after clamping) by one
// block of kPermThreads threads.  Wave w owns the contiguous chunk of keys
// [w C, (w + 1) C) (C a multiple of 64): it counts its chunk per expert into
// its own LDS row, the block turns the rows into each wave's first position
// per expert (expert offset plus the counts of the waves before), and each
// wave then walks its chunk 64 keys at a time, in order, with no block
// barrier: lanes with the same key are found by one ballot per key bit, and
// one lane per key advances the wave's cursor.  Positions therefore ascend
// with the flat id within every expert (stable).
template <typename KeyFn>
__device__ void permute_block(KeyFn key, int N, int E, const Plan& p, bool with_lists,
                              PermShared& sh) {
  constexpr int W = kPermThreads / kWave;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  // positions in uint32_t: N < 2^31, so chunk ends and batch steps past
  // them stay representable
  const uint32_t n = (uint32_t)N;
  const uint32_t C = ((n + W - 1) / W + kWave - 1) / kWave * kWave;
  const uint32_t q0 = min((uint32_t)wave * C, n);
  const uint32_t q1 = q0 + min(C, n - q0);
  auto kat = [&](uint32_t q) { return key((int)min(q, n - 1)); };  // clamped key load

  for (int i = tid; i < E; i += kPermThreads) {
#pragma unroll
    for (int w = 0; w < W; ++w) sh.wave_cnt[w][i] = 0;
  }
  __syncthreads();
  // per-wave counts; keys in groups of kKeyBatch per lane, all loads before
  // the adds (a load-then-add loop waits out each load's latency in turn)
  constexpr int kKeyBatch = 32;
  for (uint32_t b = q0; b < q1; b += kWave * kKeyBatch) {
    int ks[kKeyBatch];
#pragma unroll
    for (int u = 0; u < kKeyBatch; ++u) ks[u] = kat(b + u * kWave + lane);
#pragma unroll
    for (int u = 0; u < kKeyBatch; ++u) {
      if (b + u * kWave >= q1) break;  // wave-uniform
      if (b + u * kWave + lane < q1) atomicAdd(&sh.wave_cnt[wave][min(max(ks[u], 0), E - 1)], 1);
    }
  }
  __syncthreads();

  int c = 0;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < W; ++w) c += sh.wave_cnt[w][tid];
  }
  int total = 0;
  const int excl = block_exclusive_scan(c, sh.tmp, &total);
  if (tid < E) {
    p.counts[tid] = c;
    p.offsets[tid] = excl;
    int run = excl;  // wave w's first position for expert tid
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const int cw = sh.wave_cnt[w][tid];
      sh.wave_cnt[w][tid] = run;
      run += cw;
    }
  }
  if (tid == 0) p.offsets[E] = total;
  if (with_lists) write_lists(c, excl, E, p, sh.tmp);
  __syncthreads();

  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  volatile int* const cursor = sh.wave_cnt[wave];  // read and moved in program order
  // the keys of kKeyBatch batches are loaded together, then sorted in order
  for (uint32_t g = q0; g < q1; g += kWave * kKeyBatch) {
    int ks[kKeyBatch];
#pragma unroll
    for (int u = 0; u < kKeyBatch; ++u) ks[u] = kat(g + u * kWave + lane);
#pragma unroll
    for (int u = 0; u < kKeyBatch; ++u) {
      if (g + u * kWave >= q1) break;  // wave-uniform: the chunk's last batch is done
      const uint32_t q = g + u * kWave + lane;
      const bool valid = q < q1;
      dbg_flag(valid && (unsigned)ks[u] >= (unsigned)E, kDbgTopk);
      const int e = valid ? min(max(ks[u], 0), E - 1) : 0;
      uint64_t peers = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bal = __ballot(valid && bit);
        peers &= bit ? bal : ~bal;
      }
      const int rank = __popcll(peers & lt_mask);
      // every lane reads its key's cursor before the leaders move them (one
      // wave: its LDS accesses happen in program order)
      const int start = cursor[e];
      if (valid) {
        const int pos = start + rank;
        p.sorted_src[pos] = (int)q;
        p.dest_row[q] = pos;
      }
      if (valid && rank == 0) cursor[e] = start + __popcll(peers);
    }
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int* __restrict__ topk_idx,
                                                               int N, int E, Plan p,
                                                               int with_lists) {
  __shared__ PermShared sh;
  permute_block([&](int q) { return topk_idx[q]; }, N, E, p, with_lists != 0, sh);
}

__global__ __launch_bounds__(kPermThreads) void plan_kernel(const int* __restrict__ offsets, int E,
                                                            int Tk, Plan p) {
  __shared__ int tmp[32];
  const int e = threadIdx.x;
  int first = e < E ? offsets[e] : 0;
  int next = e < E ? offsets[e + 1] : 0;
#ifdef MOE_DEBUG_CHECKS
  // caller's offsets: ascending from 0 to T*k; otherwise clamped so that the
  // plan stays inside [0, T*k]
  if (e < E) {
    dbg_flag(next < first || first < 0 || next > Tk || (e == 0 && first != 0) || (e == E - 1 && next != Tk),
             kDbgOffsets);
    first = min(max(first, 0), Tk);
    next = min(max(next, first), Tk);
  }
#endif
  write_lists(next - first, first, E, p, tmp);
}

// Decode-sized layers (T <= 16, T*k <= 1024): wave t routes token t, then the
// whole block sorts the T*k pairs from LDS.  One launch instead of two.
template <int VPL>
__global__ __launch_bounds__(kPermThreads) void route_permute_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int* __restrict__ topk_idx,
    float* __restrict__ topk_w, Plan p) {
  __shared__ PermShared sh;
  __shared__ int keys[kPermThreads];
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  if (wave < T) {
    int sel_i;
    float sel_w;
    route_token<VPL>(logits + (size_t)wave * E, E, k, sel_i, sel_w);
    if (lane < k) {
      topk_idx[wave * k + lane] = sel_i;
      topk_w[wave * k + lane] = sel_w;
      keys[wave * k + lane] = sel_i;
    }
  }
  __syncthreads();
  permute_block([&](int q) { return keys[q]; }, T * k, E, p, true, sh);
}

// Single-token layers: one wave routes the token and writes the whole plan.
template <int VPL>
__global__ __launch_bounds__(64) void route_plan_t1_kernel(const float* __restrict__ logits, int E,
                                                           int k, int* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w, Plan p) {
  int sel_i;
  float sel_w;
  route_token<VPL>(logits, E, k, sel_i, sel_w);
  write_plan_t1(sel_i, sel_w, selected_rank(sel_i, k), E, k, topk_idx, topk_w, p);
}

}  // namespace

hipError_t launch_route_plan_t1(const float* logits, int E, int k, int* topk_idx, float* topk_w,
                                const Plan& p, hipStream_t s) {
  LaunchTimer tm("route_plan_t1", s);
  const dim3 g(1), b(kWave);
  if (E <= 64)
    route_plan_t1_kernel<1><<<g, b, 0, s>>>(logits, E, k, topk_idx, topk_w, p);
  else if (E <= 128)
    route_plan_t1_kernel<2><<<g, b, 0, s>>>(logits, E, k, topk_idx, topk_w, p);
  else if (E <= 256)
    route_plan_t1_kernel<4><<<g, b, 0, s>>>(logits, E, k, topk_idx, topk_w, p);
  else if (E <= 512)
    route_plan_t1_kernel<8><<<g, b, 0, s>>>(logits, E, k, topk_idx, topk_w, p);
  else
    route_plan_t1_kernel<16><<<g, b, 0, s>>>(logits, E, k, topk_idx, topk_w, p);
  return hipGetLastError();
}

hipError_t launch_permute(const int* topk_idx, int T, int E, int k, const Plan& p,
                          bool with_lists, hipStream_t s) {
  LaunchTimer tm("permute", s);
  permute_kernel<<<1, kPermThreads, 0, s>>>(topk_idx, T * k, E, p, with_lists ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_plan_from_offsets(const int* offsets, int E, int Tk, const Plan& p, hipStream_t s) {
  LaunchTimer tm("plan", s);
  plan_kernel<<<1, kPermThreads, 0, s>>>(offsets, E, Tk, p);
  return hipGetLastError();
}

hipError_t launch_route_permute_small(const float* logits, int T, int E, int k, int* topk_idx,
                                      float* topk_w, const Plan& p, hipStream_t s) {
  LaunchTimer tm("route_permute", s);
  const dim3 g(1), b(kPermThreads);
  if (E <= 64)
    route_permute_small_kernel<1><<<g, b, 0, s>>>(logits, T, E, k, topk_idx, topk_w, p);
  else if (E <= 128)
    route_permute_small_kernel<2><<<g, b, 0, s>>>(logits, T, E, k, topk_idx, topk_w, p);
  else if (E <= 256)
    route_permute_small_kernel<4><<<g, b, 0, s>>>(logits, T, E, k, topk_idx, topk_w, p);
  else if (E <= 512)
    route_permute_small_kernel<8><<<g, b, 0, s>>>(logits, T, E, k, topk_idx, topk_w, p);
  else
    route_permute_small_kernel<16><<<g, b, 0, s>>>(logits, T, E, k, topk_idx, topk_w, p);
  return hipGetLastError();
}

MOE_DBG_TAKE_DEFINE(dbg_take_permute)

}  // namespace moe
