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
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane * VPL + i;
    v[i] = (e < E) ? row[e] : 0.f;
    key[i] = (e < E) ? route_key(v[i]) : 0u;
  }
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

}  // namespace moe
