// Expert FFN for few tokens per expert (decode, speculative verify): weight
// streaming GEMVs.
//
// Small-batch decode waits on expert weights arriving from HBM, not on
// arithmetic (SGLang-TorchTPU on TPU v7 page, "Introduction"), so these
// kernels are built around the weight stream: every weight row of an active
// expert is read exactly once with 16-byte non-temporal loads (all of a row's
// loads in flight at once), applied in registers to every token routed to
// that expert, and reduced in fp32 (TensorSharp Muse Spark report, "Answer
// quality": bf16 partial sums cost accuracy).
//
// Work unit: one wave64 per weight row.  A 16-byte "chunk" of a row holds 4
// fp32, 8 bf16 or 32 MX-FP4 codes (exactly one 32-element scale block); lane
// l takes chunks l, l+64, ... so every load instruction reads 1 KiB of
// contiguous row.  Rows longer than MAXC*64 chunks are streamed in segments.
#include "device.h"
#include "internal.h"

namespace moe {
namespace {

template <int WF>
struct WT;
template <>
struct WT<kF32> {
  static constexpr int CE = 4;  // elements per 16-byte weight chunk
  static constexpr int XB = 16; // activation bytes for one chunk
  __host__ __device__ static size_t row_bytes(int K) { return (size_t)K * 4; }
};
template <>
struct WT<kBF16> {
  static constexpr int CE = 8;
  static constexpr int XB = 16;
  __host__ __device__ static size_t row_bytes(int K) { return (size_t)K * 2; }
};
template <>
struct WT<kMXFP4> {
  static constexpr int CE = 32;
  static constexpr int XB = 64;
  __host__ __device__ static size_t row_bytes(int K) { return (size_t)K / 2; }
};

// Activations are fp32 with fp32 weights and bf16 otherwise.
template <int WF>
constexpr int act_bytes() { return WF == kF32 ? 4 : 2; }

template <int WF>
struct XChunk {
  u32x4 v[WT<WF>::XB / 16];
};

template <int WF>
__device__ __forceinline__ XChunk<WF> load_x(const char* row, int c) {
  XChunk<WF> x;
#pragma unroll
  for (int i = 0; i < WT<WF>::XB / 16; ++i) x.v[i] = ld16(row + (size_t)c * WT<WF>::XB + 16 * i);
  return x;
}

// acc + <w, x> over one chunk.  For MX-FP4 the block scale is left out: the
// caller multiplies the block's partial sum by it (one scale per chunk).
template <int WF>
__device__ __forceinline__ float dot_chunk(const u32x4& w, const XChunk<WF>& x, float acc) {
  if constexpr (WF == kF32) {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.v[0].x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.v[0].y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.v[0].z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.v[0].w), acc);
  } else if constexpr (WF == kBF16) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    const uint32_t xx[4] = {x.v[0].x, x.v[0].y, x.v[0].z, x.v[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo(ww[i]), bf16_lo(xx[i]), acc);
      acc = fmaf(bf16_hi(ww[i]), bf16_hi(xx[i]), acc);
    }
  } else {
    // code word j holds elements 8j..8j+7 (byte b: elements 8j+2b, 8j+2b+1);
    // activation vector j holds the same 8 elements as 4 bf16 pairs.
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t xx[4] = {x.v[j].x, x.v[j].y, x.v[j].z, x.v[j].w};
      float2 p0 = fp4x2_to_f32<0>(ww[j]);
      float2 p1 = fp4x2_to_f32<1>(ww[j]);
      float2 p2 = fp4x2_to_f32<2>(ww[j]);
      float2 p3 = fp4x2_to_f32<3>(ww[j]);
      acc = fmaf(p0.x, bf16_lo(xx[0]), acc);
      acc = fmaf(p0.y, bf16_hi(xx[0]), acc);
      acc = fmaf(p1.x, bf16_lo(xx[1]), acc);
      acc = fmaf(p1.y, bf16_hi(xx[1]), acc);
      acc = fmaf(p2.x, bf16_lo(xx[2]), acc);
      acc = fmaf(p2.y, bf16_hi(xx[2]), acc);
      acc = fmaf(p3.x, bf16_lo(xx[3]), acc);
      acc = fmaf(p3.y, bf16_hi(xx[3]), acc);
    }
  }
  return acc;
}

template <int WF>
__device__ __forceinline__ void store_act(void* base, size_t i, float v) {
  if constexpr (WF == kF32)
    reinterpret_cast<float*>(base)[i] = v;
  else
    reinterpret_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

struct GateUpArgs {
  const void* x;
  const void* wg;
  const void* wu;
  const uint8_t* sg;
  const uint8_t* su;
  const int* offsets;
  const int* sorted_src;
  const int* active;
  const int* num_active;
  void* h;
  int d, f, k;
};

// h[r][n] = silu(<w_gate[e][n], x[t]>) * <w_up[e][n], x[t]> for every row r
// of expert e (t = sorted_src[r] / k).  Block = 4 waves = 4 consecutive n of
// one active expert.
template <int WF, int MAXC, int MAXT>
__global__ __launch_bounds__(256) void gemv_gate_up_kernel(GateUpArgs a) {
  constexpr int CE = WT<WF>::CE;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int tiles = (a.f + 3) >> 2;
  const int slot = blockIdx.x / tiles;
  if (slot >= *a.num_active) return;
  const int n = (blockIdx.x - slot * tiles) * 4 + wave;
  if (n >= a.f) return;
  const int e = a.active[slot];
  const int r0 = a.offsets[e];
  const int ntok = a.offsets[e + 1] - r0;
  const int nchunks = a.d / CE;
  const int nseg = (nchunks + MAXC * kWave - 1) / (MAXC * kWave);
  const size_t rb = WT<WF>::row_bytes(a.d);
  const char* gp = reinterpret_cast<const char*>(a.wg) + ((size_t)e * a.f + n) * rb;
  const char* up = reinterpret_cast<const char*>(a.wu) + ((size_t)e * a.f + n) * rb;
  const uint8_t* sgp = (WF == kMXFP4) ? a.sg + ((size_t)e * a.f + n) * (a.d / 32) : nullptr;
  const uint8_t* sup = (WF == kMXFP4) ? a.su + ((size_t)e * a.f + n) * (a.d / 32) : nullptr;
  const size_t xrb = (size_t)a.d * act_bytes<WF>();
  const char* xb = reinterpret_cast<const char*>(a.x);

  u32x4 wg[MAXC], wu[MAXC];
  float sgv[MAXC], suv[MAXC];
  for (int g0 = 0; g0 < ntok; g0 += MAXT) {
    const int ng = min(MAXT, ntok - g0);
    const char* xr[MAXT];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt)
      xr[tt] = xb + (size_t)(a.sorted_src[r0 + g0 + min(tt, ng - 1)] / a.k) * xrb;
    float ag[MAXT], au[MAXT];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) ag[tt] = au[tt] = 0.f;
    for (int seg = 0; seg < nseg; ++seg) {
      const int cb = seg * MAXC * kWave + lane;
      if (nseg > 1 || g0 == 0) {
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
          const int c = cb + i * kWave;
          if (c < nchunks) {
            wg[i] = ld_stream16(gp + (size_t)c * 16);
            wu[i] = ld_stream16(up + (size_t)c * 16);
            if constexpr (WF == kMXFP4) {
              sgv[i] = e8m0_to_f32(sgp[c]);
              suv[i] = e8m0_to_f32(sup[c]);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = cb + i * kWave;
        if (c < nchunks) {
#pragma unroll
          for (int tt = 0; tt < MAXT; ++tt) {
            if (tt < ng) {
              const XChunk<WF> xc = load_x<WF>(xr[tt], c);
              if constexpr (WF == kMXFP4) {
                ag[tt] = fmaf(dot_chunk<WF>(wg[i], xc, 0.f), sgv[i], ag[tt]);
                au[tt] = fmaf(dot_chunk<WF>(wu[i], xc, 0.f), suv[i], au[tt]);
              } else {
                ag[tt] = dot_chunk<WF>(wg[i], xc, ag[tt]);
                au[tt] = dot_chunk<WF>(wu[i], xc, au[tt]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) {
      if (tt < ng) {
        const float G = wave_sum(ag[tt]);
        const float U = wave_sum(au[tt]);
        if (lane == 0) store_act<WF>(a.h, (size_t)(r0 + g0 + tt) * a.f + n, silu(G) * U);
      }
    }
  }
}

struct DownArgs {
  const void* h;
  const void* wd;
  const uint8_t* sd;
  const int* offsets;
  const int* sorted_src;
  const int* active;
  const int* num_active;
  const float* topk_w;
  float* y_sorted;
  void* out;
  int T, d, f, k;
};

// y_sorted[r][n] = <w_down[e][n], h[r]> for every row r of expert e.
template <int WF, int MAXC, int MAXT>
__global__ __launch_bounds__(256) void gemv_down_kernel(DownArgs a) {
  constexpr int CE = WT<WF>::CE;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int tiles = (a.d + 3) >> 2;
  const int slot = blockIdx.x / tiles;
  if (slot >= *a.num_active) return;
  const int n = (blockIdx.x - slot * tiles) * 4 + wave;
  if (n >= a.d) return;
  const int e = a.active[slot];
  const int r0 = a.offsets[e];
  const int ntok = a.offsets[e + 1] - r0;
  const int nchunks = a.f / CE;
  const int nseg = (nchunks + MAXC * kWave - 1) / (MAXC * kWave);
  const size_t rb = WT<WF>::row_bytes(a.f);
  const char* wp = reinterpret_cast<const char*>(a.wd) + ((size_t)e * a.d + n) * rb;
  const uint8_t* sp = (WF == kMXFP4) ? a.sd + ((size_t)e * a.d + n) * (a.f / 32) : nullptr;
  const size_t hrb = (size_t)a.f * act_bytes<WF>();
  const char* hb = reinterpret_cast<const char*>(a.h);

  u32x4 wv[MAXC];
  float sv[MAXC];
  for (int g0 = 0; g0 < ntok; g0 += MAXT) {
    const int ng = min(MAXT, ntok - g0);
    float acc[MAXT];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) acc[tt] = 0.f;
    for (int seg = 0; seg < nseg; ++seg) {
      const int cb = seg * MAXC * kWave + lane;
      if (nseg > 1 || g0 == 0) {
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
          const int c = cb + i * kWave;
          if (c < nchunks) {
            wv[i] = ld_stream16(wp + (size_t)c * 16);
            if constexpr (WF == kMXFP4) sv[i] = e8m0_to_f32(sp[c]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = cb + i * kWave;
        if (c < nchunks) {
#pragma unroll
          for (int tt = 0; tt < MAXT; ++tt) {
            if (tt < ng) {
              const XChunk<WF> hc = load_x<WF>(hb + (size_t)(r0 + g0 + tt) * hrb, c);
              if constexpr (WF == kMXFP4)
                acc[tt] = fmaf(dot_chunk<WF>(wv[i], hc, 0.f), sv[i], acc[tt]);
              else
                acc[tt] = dot_chunk<WF>(wv[i], hc, acc[tt]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) {
      if (tt < ng) {
        const float y = wave_sum(acc[tt]);
        if (lane == 0) a.y_sorted[(size_t)(r0 + g0 + tt) * a.d + n] = y;
      }
    }
  }
}

// Down projection fused with the weighted combine, for T <= TT tokens:
// out[t][n] = sum over active experts e (ascending), over e's rows r with
// token t, of topk_w[q] * <w_down[e][n], h[r]>.  One wave per output column
// n; per-lane partial sums per token, one wave reduction per token at the end.
template <int WF, int MAXC, int TT>
__global__ __launch_bounds__(256) void gemv_down_combine_kernel(DownArgs a) {
  constexpr int CE = WT<WF>::CE;
  const int lane = lane_id();
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= a.d) return;
  const int na = *a.num_active;
  const int nchunks = a.f / CE;
  const int nseg = (nchunks + MAXC * kWave - 1) / (MAXC * kWave);
  const size_t rb = WT<WF>::row_bytes(a.f);
  const size_t hrb = (size_t)a.f * act_bytes<WF>();
  const char* hb = reinterpret_cast<const char*>(a.h);

  float acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.f;
  u32x4 wv[MAXC];
  float sv[MAXC];
  for (int s = 0; s < na; ++s) {
    const int e = a.active[s];
    const int r0 = a.offsets[e];
    const int ntok = a.offsets[e + 1] - r0;
    const char* wp = reinterpret_cast<const char*>(a.wd) + ((size_t)e * a.d + n) * rb;
    const uint8_t* sp = (WF == kMXFP4) ? a.sd + ((size_t)e * a.d + n) * (a.f / 32) : nullptr;
    for (int seg = 0; seg < nseg; ++seg) {
      const int cb = seg * MAXC * kWave + lane;
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = cb + i * kWave;
        if (c < nchunks) {
          wv[i] = ld_stream16(wp + (size_t)c * 16);
          if constexpr (WF == kMXFP4) sv[i] = e8m0_to_f32(sp[c]);
        }
      }
      for (int rr = 0; rr < ntok; ++rr) {
        const int q = a.sorted_src[r0 + rr];
        const char* hr = hb + (size_t)(r0 + rr) * hrb;
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
          const int c = cb + i * kWave;
          if (c < nchunks) {
            const XChunk<WF> hc = load_x<WF>(hr, c);
            if constexpr (WF == kMXFP4)
              p = fmaf(dot_chunk<WF>(wv[i], hc, 0.f), sv[i], p);
            else
              p = dot_chunk<WF>(wv[i], hc, p);
          }
        }
        const float wt = a.topk_w[q];
        if constexpr (TT == 1) {
          acc[0] = fmaf(wt, p, acc[0]);
        } else {
          const int t = q / a.k;
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
            if (tt == t) acc[tt] = fmaf(wt, p, acc[tt]);
        }
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    if (tt < a.T) {
      const float v = wave_sum(acc[tt]);
      if (lane == 0) store_act<WF>(a.out, (size_t)tt * a.d + n, v);
    }
  }
}

// Registers per lane for one row: the smallest supported MAXC covering the
// row, capped at 16 (longer rows are streamed in segments).
int pick_maxc(int nchunks) {
  const int need = (nchunks + kWave - 1) / kWave;
  static const int opts[] = {1, 2, 4, 6, 8, 12, 16};
  for (int o : opts)
    if (need <= o) return o;
  return 16;
}

#define MOE_MAXC_SWITCH(MAXC, CALL)      \
  switch (MAXC) {                        \
    case 1: { constexpr int MC = 1; CALL; } break;   \
    case 2: { constexpr int MC = 2; CALL; } break;   \
    case 4: { constexpr int MC = 4; CALL; } break;   \
    case 6: { constexpr int MC = 6; CALL; } break;   \
    case 8: { constexpr int MC = 8; CALL; } break;   \
    case 12: { constexpr int MC = 12; CALL; } break; \
    default: { constexpr int MC = 16; CALL; } break; \
  }

#define MOE_WF_SWITCH(WFV, CALL)                            \
  switch (WFV) {                                            \
    case kF32: { constexpr int WF = kF32; CALL; } break;     \
    case kBF16: { constexpr int WF = kBF16; CALL; } break;   \
    default: { constexpr int WF = kMXFP4; CALL; } break;     \
  }

int chunk_elems(int wf) { return wf == kF32 ? 4 : (wf == kBF16 ? 8 : 32); }

constexpr int kGemvMaxT = 4;

}  // namespace

hipError_t launch_gemv_gate_up(const Dims& dm, const void* x, const Plan& p, const int* sorted_src,
                               const Weights& w, void* h, hipStream_t s) {
  LaunchTimer tm("gemv_gate_up", s);
  GateUpArgs a{x, w.wg, w.wu, w.sg, w.su, p.offsets, sorted_src, p.active, p.num_active, h,
               dm.d, dm.f, dm.k};
  const long long max_active = dm.Tk() < dm.E ? dm.Tk() : dm.E;
  const dim3 grid((unsigned)(max_active * ((dm.f + 3) / 4))), block(256);
  const int maxc = pick_maxc(dm.d / chunk_elems(dm.wfmt));
  MOE_WF_SWITCH(dm.wfmt, MOE_MAXC_SWITCH(maxc, (gemv_gate_up_kernel<WF, MC, kGemvMaxT><<<grid, block, 0, s>>>(a))));
  return hipGetLastError();
}

hipError_t launch_gemv_down(const Dims& dm, const void* h, const Plan& p, const Weights& w,
                            float* y_sorted, hipStream_t s) {
  LaunchTimer tm("gemv_down", s);
  DownArgs a{h, w.wd, w.sd, p.offsets, p.sorted_src, p.active, p.num_active, nullptr,
             y_sorted, nullptr, dm.T, dm.d, dm.f, dm.k};
  const long long max_active = dm.Tk() < dm.E ? dm.Tk() : dm.E;
  const dim3 grid((unsigned)(max_active * ((dm.d + 3) / 4))), block(256);
  const int maxc = pick_maxc(dm.f / chunk_elems(dm.wfmt));
  MOE_WF_SWITCH(dm.wfmt, MOE_MAXC_SWITCH(maxc, (gemv_down_kernel<WF, MC, kGemvMaxT><<<grid, block, 0, s>>>(a))));
  return hipGetLastError();
}

hipError_t launch_gemv_down_combine(const Dims& dm, const void* h, const Plan& p,
                                    const int* sorted_src, const float* topk_w,
                                    const Weights& w, void* out, hipStream_t s) {
  LaunchTimer tm("gemv_down_combine", s);
  DownArgs a{h, w.wd, w.sd, p.offsets, sorted_src, p.active, p.num_active, topk_w,
             nullptr, out, dm.T, dm.d, dm.f, dm.k};
  const dim3 grid((unsigned)((dm.d + 3) / 4)), block(256);
  const int maxc = pick_maxc(dm.f / chunk_elems(dm.wfmt));
  if (dm.T == 1) {
    MOE_WF_SWITCH(dm.wfmt, MOE_MAXC_SWITCH(maxc, (gemv_down_combine_kernel<WF, MC, 1><<<grid, block, 0, s>>>(a))));
  } else {
    MOE_WF_SWITCH(dm.wfmt, MOE_MAXC_SWITCH(maxc, (gemv_down_combine_kernel<WF, MC, kDecodeMaxT><<<grid, block, 0, s>>>(a))));
  }
  return hipGetLastError();
}

}  // namespace moe
