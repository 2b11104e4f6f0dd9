// Per-token top-k selection with renormalised softmax weights, for one wave64.
//
// The layer picks k of its E experts per token (SGLang-TorchTPU on TPU v7
// page, "Introduction": 8 of 256) and combines their outputs with normalised
// weights (TensorSharp Muse Spark report, "Performance" section).  The
// weights taken are a softmax over all E logits renormalised over the k
// selected ones, which equals a softmax over the k selected logits.
//
// Lane l holds the VPL consecutive logits [l*VPL, (l+1)*VPL), so ascending
// (lane, position) is ascending expert index.  Each of the k rounds takes the
// wave maximum of an order-preserving integer key (DPP within 16-lane rows,
// then the four row maxima by readlane), finds the lowest lane holding it with
// a ballot, and reads that lane's lowest-index candidate: larger logit first,
// ties to the lower expert index, with no chain of cross-lane shuffles.
#pragma once

#include <float.h>
#include <limits.h>

#include "device.h"

namespace moe {

// Order-preserving map fp32 -> uint32 (larger float, larger key); -0.0 is
// folded onto +0.0 so the two compare equal.  Key 0 is below every real
// value (-inf maps to 0x007fffff) and marks taken or padding entries.
__device__ __forceinline__ uint32_t route_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xf, 0xf, true);
}

// Maximum of a uint32 over the wave, returned uniformly.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]: lanes xor 1
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]: lanes xor 2
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror: 8-lane groups
  v = max(v, dpp_u32<0x140>(v));  // row_mirror: 16-lane rows
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0);
  const uint32_t r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32);
  const uint32_t r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// On return lane j < k holds slot j: its expert index and its weight.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k,
                                            int& sel_i, float& sel_w) {
  const int lane = lane_id();
  float v[VPL];
  uint32_t key[VPL];
  // all loads first, from clamped (in-row) positions: a load under a
  // condition would be waited for before the next one is issued
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = row[min(lane * VPL + i, E - 1)];
#pragma unroll
  for (int i = 0; i < VPL; ++i) key[i] = (lane * VPL + i < E) ? route_key(v[i]) : 0u;
  float sel_v = 0.f;
  sel_i = 0;
  for (int j = 0; j < k; ++j) {
    // lane-local best: largest key, lowest position on ties
    uint32_t bk = key[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < VPL; ++i) {
      if (key[i] > bk) {
        bk = key[i];
        bi = i;
      }
    }
    const uint32_t m = wave_max_u32(bk);
    const uint64_t holders = __ballot(bk == m);
    const int wl = __ffsll((unsigned long long)holders) - 1;  // lowest lane: lowest index
    const int wpos = __builtin_amdgcn_readlane(bi, wl);
    const int widx = wl * VPL + wpos;
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (i == wpos) key[i] = 0u;
    }
    if (lane == j) sel_i = widx;
    // the winner's logit, from its key (exact inverse of route_key)
    const uint32_t b = (m & 0x80000000u) ? (m & 0x7fffffffu) : ~m;
    if (lane == j) sel_v = __uint_as_float(b);
  }
  // Slot 0 holds the maximum; equal logits (also all -inf) contribute 1.
  const float l0 = __shfl(sel_v, 0, kWave);
  float ex = 0.f;
  if (lane < k) ex = (sel_v == l0) ? 1.0f : expf(sel_v - l0);
  const float sum = wave_sum(ex);
  sel_w = ex / sum;
}

// Lane j < k holding selected expert sel_i (the k are distinct): the number
// of selected experts below it, i.e. slot j's position in expert order.
__device__ __forceinline__ int selected_rank(int sel_i, int k) {
  int rank = 0;
  for (int j = 0; j < k; ++j) rank += (__builtin_amdgcn_readlane(sel_i, j) < sel_i) ? 1 : 0;
  return rank;
}

// The whole permutation plan of a single-token layer from one wave's routing
// (lane j < k: slot j's expert, weight and rank): every active expert has one
// row, at the position of its rank.  Every lane of the wave must call.
__device__ __forceinline__ void write_plan_t1(int sel_i, float sel_w, int rank, int E, int k,
                                              int* __restrict__ topk_idx, float* __restrict__ topk_w,
                                              const Plan& p) {
  const int lane = lane_id();
  if (lane < k) {
    topk_idx[lane] = sel_i;
    topk_w[lane] = sel_w;
    p.sorted_src[rank] = lane;
    p.dest_row[lane] = rank;
    p.active[rank] = sel_i;
    p.slot_info[4 * rank + 0] = sel_i;
    p.slot_info[4 * rank + 1] = rank;
    p.slot_info[4 * rank + 2] = 1;
    p.slot_info[4 * rank + 3] = 0;
    int* m = p.mtiles + kMtileInts * rank;
    m[0] = sel_i;
    m[1] = rank;
    m[2] = 1;
    m[3] = rank;
    m[4] = 1;
  }
  for (int e = lane; e < E; e += kWave) {
    int c = 0, below = 0;
    for (int j = 0; j < k; ++j) {
      const int o = __builtin_amdgcn_readlane(sel_i, j);
      c += (o == e) ? 1 : 0;
      below += (o < e) ? 1 : 0;
    }
    p.counts[e] = c;
    p.offsets[e] = below;
  }
  if (lane == 0) {
    p.offsets[E] = k;
    *p.num_active = k;
    *p.num_mtiles = k;
  }
}

}  // namespace moe
