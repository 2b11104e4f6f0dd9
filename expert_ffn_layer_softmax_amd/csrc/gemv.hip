// Expert FFN for few tokens per expert (decode, speculative verify): weight
// streaming GEMVs.
//
// Small-batch decode waits on expert weights arriving from HBM, not on
// arithmetic (SGLang-TorchTPU on TPU v7 page, "Introduction"), so these
// kernels are built around the weight stream: every weight row of an active
// expert is read exactly once with 16-byte non-temporal loads, all of a
// wave's loads in flight together, and applied in registers to every token
// routed to that expert with fp32 accumulation (TensorSharp Muse Spark report,
// "Answer quality": bf16 partial sums cost accuracy).
//
// Work unit: one wave64 per RPW weight rows of one active expert.  A 16-byte
// "chunk" of a row holds 4 fp32, 8 bf16 or 32 4-bit codes (one MX-FP4 scale
// block, two NVFP4 ones; the NVFP4 matrix scale multiplies each finished row
// sum, as in the pages' own 4-bit format: SGLang-TorchTPU on TPU v7 page,
// "Results"); lane l takes chunks l, l+64, ... so each load
// instruction reads 1 KiB of contiguous row.  The weight loads are issued
// right after one scalar lookup of the slot's (expert, rows) entry, before the
// token indices are resolved, so the index chain overlaps the weight stream.
// Tokens are then processed one at a time against the weights held in
// registers.  Rows longer than MAXC*64 chunks (MULTISEG) are streamed in
// segments, re-reading the weights per token.
#include <algorithm>
#include <map>
#include <type_traits>
#include <mutex>
#include <tuple>

#include "device.h"
#include "internal.h"
#include "route_dev.h"

namespace moe {
namespace {

template <int WF>
struct WT;
template <>
struct WT<kF32> {
  static constexpr int CE = 4;   // elements per 16-byte weight chunk
  static constexpr int XB = 16;  // activation bytes matching one chunk
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
template <>
struct WT<kNVFP4> {
  static constexpr int CE = 32;
  static constexpr int XB = 64;
  __host__ __device__ static size_t row_bytes(int K) { return (size_t)K / 2; }
};

// Block-scale bytes per weight row: one E8M0 per 32 elements (MX-FP4), one
// E4M3 per 16 (NVFP4, two per 16-byte chunk).
template <int WF>
constexpr size_t scale_row_bytes(int K) {
  return WF == kMXFP4 ? (size_t)K / 32 : (WF == kNVFP4 ? (size_t)K / 16 : 0);
}

// Activations are fp32 with fp32 weights and bf16 otherwise.
template <int WF>
constexpr int act_bytes() { return WF == kF32 ? 4 : 2; }

template <int WF>
struct XChunk {
  u32x4 v[WT<WF>::XB / 16];
};

// acc + <codes * scale, x> for code word j of a 4-bit chunk (elements
// 8j..8j+7; byte b holds elements 8j+2b, 8j+2b+1) and the matching activation
// vector j.  `sc` is the convert's scale operand (only its exponent is read).
// OPQ hides the word from the optimiser, so that kernels which apply the same
// weights to several tokens convert them again per token instead of holding
// four times the registers.
template <bool OPQ>
__device__ __forceinline__ float fp4_word_dot(uint32_t cw_in, const u32x4& xv, float sc, float acc) {
  const uint32_t cw = OPQ ? opaque(cw_in) : cw_in;
  acc = dot2_bf16(fp4x2_to_bf16x2<0>(cw, sc), xv.x, acc);
  acc = dot2_bf16(fp4x2_to_bf16x2<1>(cw, sc), xv.y, acc);
  acc = dot2_bf16(fp4x2_to_bf16x2<2>(cw, sc), xv.z, acc);
  acc = dot2_bf16(fp4x2_to_bf16x2<3>(cw, sc), xv.w, acc);
  return acc;
}

// acc + <w, x> over one chunk.  4-bit codes are converted with scale `sc`.
template <int WF, bool OPQ = true>
__device__ __forceinline__ float dot_chunk(const u32x4& w, const XChunk<WF>& x, float acc,
                                           float sc = 1.0f) {
  if constexpr (WF == kF32) {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.v[0].x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.v[0].y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.v[0].z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.v[0].w), acc);
  } else if constexpr (WF == kBF16) {
    acc = dot2_bf16(w.x, x.v[0].x, acc);
    acc = dot2_bf16(w.y, x.v[0].y, acc);
    acc = dot2_bf16(w.z, x.v[0].z, acc);
    acc = dot2_bf16(w.w, x.v[0].w, acc);
  } else {
    // activation vector j holds the 8 elements of code word j as 4 bf16 pairs
    acc = fp4_word_dot<OPQ>(w.x, x.v[0], sc, acc);
    acc = fp4_word_dot<OPQ>(w.y, x.v[1], sc, acc);
    acc = fp4_word_dot<OPQ>(w.z, x.v[2], sc, acc);
    acc = fp4_word_dot<OPQ>(w.w, x.v[3], sc, acc);
  }
  return acc;
}

// acc + the chunk's contribution with its block scales.  MX-FP4: the E8M0
// scale (a power of two) goes into the convert, so each weight reaches the
// dot product as code * 2^(s-127) in bf16 -- exact while it is finite in bf16
// (block scales up to 2^125), as in the grouped GEMMs.  NVFP4 (E4M3 scales,
// not powers of two): elements 0..15 (words 0, 1) sum to a partial that is
// scaled by s in fp32, elements 16..31 (words 2, 3) by s2.  Other formats have
// no block scale.
template <int WF, bool OPQ = true>
__device__ __forceinline__ float scaled_chunk(const u32x4& w, const XChunk<WF>& x, float s, float s2,
                                              float acc) {
  if constexpr (WF == kMXFP4) {
    return dot_chunk<WF, OPQ>(w, x, acc, s);
  } else if constexpr (WF == kNVFP4) {
    const float lo = fp4_word_dot<OPQ>(w.y, x.v[1], 1.0f, fp4_word_dot<OPQ>(w.x, x.v[0], 1.0f, 0.f));
    const float hi = fp4_word_dot<OPQ>(w.w, x.v[3], 1.0f, fp4_word_dot<OPQ>(w.z, x.v[2], 1.0f, 0.f));
    return fmaf(hi, s2, fmaf(lo, s, acc));
  } else {
    return dot_chunk<WF>(w, x, acc);
  }
}

template <int WF>
__device__ __forceinline__ void store_act(void* base, size_t i, float v) {
  if constexpr (WF == kF32)
    reinterpret_cast<float*>(base)[i] = v;
  else
    reinterpret_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// A row's finished sum times its matrix's fp32 scale (NVFP4 only).
template <int WF>
__device__ __forceinline__ float matrix_scaled(float v, const float* t, int e) {
  if constexpr (WF == kNVFP4)
    return v * t[e];
  else
    return v;
}

// Weight rows of RPW consecutive outputs, one segment, in registers.
template <int WF, int MAXC, int RPW>
struct RowRegs {
  u32x4 w[RPW][MAXC];
  float s[RPW][MAXC];   // MX-FP4: convert scale operand; NVFP4: scale of elements 0..15
  float s2[RPW][MAXC];  // NVFP4: block scale of elements 16..31
  uint32_t sw[RPW];     // this lane's scale word(s), until unpack()
  uint32_t sw2[RPW];    // NVFP4: second word
  bool words;

  // Issue the loads of chunks c = c0 + i*64 + lane (c < cend).  Block scales
  // (MX-FP4: one byte per chunk; NVFP4: two) are fetched with 4- or 8-byte
  // loads covering four chunks per lane, issued before the weight loads;
  // unpack() hands them to the lanes that use them with a lane shuffle (byte
  // loads per chunk would double the load instructions of the stream).
  __device__ __forceinline__ void load(const char* row0, size_t rb, const uint8_t* s0, size_t sb,
                                       int nrows, int c0, int cend, int lane) {
    constexpr size_t SPC = WF == kNVFP4 ? 2 : 1;  // scale bytes per chunk
    words = is_fp4(WF) && ((sb & (4 * SPC - 1)) == 0) && ((c0 & 3) == 0);
    if constexpr (is_fp4(WF)) {
      if (words) {
        const int q = (c0 >> 2) + lane;  // scale word(s) of chunks 4q .. 4q+3
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          sw[r] = sw2[r] = 0;
          if (r < nrows && 4 * q < cend && lane < MAXC * 16) {
            const uint8_t* sp = s0 + r * sb + 4 * SPC * (size_t)q;
            if constexpr (WF == kNVFP4) {
              const uint2 v = *reinterpret_cast<const uint2*>(sp);
              sw[r] = v.x;
              sw2[r] = v.y;
            } else {
              sw[r] = *reinterpret_cast<const uint32_t*>(sp);
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = c0 + i * kWave + lane;
        if (r < nrows && c < cend) {
          w[r][i] = ld_stream16(row0 + r * rb + (size_t)c * 16);
          if constexpr (WF == kMXFP4) {
            if (!words) s[r][i] = e8m0_cvt_scale(s0[r * sb + c]);
          } else if constexpr (WF == kNVFP4) {
            if (!words) {
              s[r][i] = e4m3_to_f32(s0[r * sb + 2 * (size_t)c]);
              s2[r][i] = e4m3_to_f32(s0[r * sb + 2 * (size_t)c + 1]);
            }
          }
        }
      }
    }
  }
  // Scales into s[][] / s2[][] (word path).  Every lane of the wave must call.
  __device__ __forceinline__ void unpack(int lane) {
    if constexpr (is_fp4(WF)) {
      if (words) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
#pragma unroll
          for (int i = 0; i < MAXC; ++i) {
            const int cl = i * kWave + lane;  // chunk relative to c0
            const int src = (cl >> 2) & (kWave - 1);
            const uint32_t v = __shfl(sw[r], src, kWave);
            if constexpr (WF == kMXFP4) {
              s[r][i] = e8m0_cvt_scale((v >> (8 * (cl & 3))) & 0xffu);
            } else {
              const uint32_t v2 = __shfl(sw2[r], src, kWave);
              const uint32_t word = (cl & 2) ? v2 : v;
              const uint32_t sh = 16 * (cl & 1);
              s[r][i] = e4m3_to_f32((word >> sh) & 0xffu);
              s2[r][i] = e4m3_to_f32((word >> (sh + 8)) & 0xffu);
            }
          }
        }
      }
    }
  }
  __device__ __forceinline__ void load_all(const char* row0, size_t rb, const uint8_t* s0, size_t sb,
                                           int nrows, int c0, int cend, int lane) {
    load(row0, rb, s0, sb, nrows, c0, cend, lane);
    unpack(lane);
  }
  // acc + chunk i of row r with its block scales (OPQ: see fp4_word_dot)
  template <bool OPQ = true>
  __device__ __forceinline__ float fma_chunk(int r, int i, const XChunk<WF>& x, float acc) const {
    if constexpr (WF == kNVFP4)
      return scaled_chunk<WF, OPQ>(w[r][i], x, s[r][i], s2[r][i], acc);
    else if constexpr (WF == kMXFP4)
      return scaled_chunk<WF, OPQ>(w[r][i], x, s[r][i], 0.f, acc);
    else
      return scaled_chunk<WF>(w[r][i], x, 0.f, 0.f, acc);
  }
};

template <int WF>
__device__ __forceinline__ XChunk<WF> load_x(const char* row, int c) {
  XChunk<WF> x;
#pragma unroll
  for (int j = 0; j < WT<WF>::XB / 16; ++j) x.v[j] = ld16(row + (size_t)c * WT<WF>::XB + 16 * j);
  return x;
}

struct GateUpArgs {
  const void* x;
  const void* wg;
  const void* wu;
  const uint8_t* sg;
  const uint8_t* su;
  const float* tg;  // NVFP4 matrix scales [E]
  const float* tu;
  const int* sorted_src;
  const int* slot_info;
  const int* num_active;
  void* h;
  int d, f, k;
  int T;  // tokens: sorted_src values lie in [0, T*k)
};

// h[r][n] = silu(<w_gate[e][n], x[t]>) * <w_up[e][n], x[t]> for every row r
// of the slot's expert e (t = sorted_src[r] / k).  Block = 4 waves; KS waves
// share one group of RPW rows, each taking 1/KS of the reduction dimension
// (more, lighter waves in flight), and their partial sums meet in LDS in a
// fixed order.  A block covers 4/KS*RPW consecutive n of one active expert.
template <int WF, int MAXC, int RPW, int KS, bool MULTISEG>
__global__ __launch_bounds__(256) void gemv_gate_up_kernel(GateUpArgs a) {
  static_assert(KS == 1 || !MULTISEG, "split reduction needs whole rows");
  __shared__ float red[4][RPW][2];
  constexpr int CE = WT<WF>::CE;
  constexpr int SEG = MAXC * kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int grp = wave / KS;
  const int part = wave - grp * KS;
  const int RB = (4 / KS) * RPW;
  const int tiles = (a.f + RB - 1) / RB;
  const int slot = blockIdx.x / tiles;
  if (slot >= *a.num_active) return;  // uniform over the block
  const int n0 = (blockIdx.x - slot * tiles) * RB + grp * RPW;
  if (KS == 1 && n0 >= a.f) return;
  const int e = a.slot_info[4 * slot + 0];
  const int nrows = max(0, min(RPW, a.f - n0));
  const int nchunks = a.d / CE;
  const int cpp = (nchunks + KS - 1) / KS;  // chunks per part
  const int cbeg = part * cpp;
  const int cend = min(nchunks, cbeg + cpp);
  const size_t rb = WT<WF>::row_bytes(a.d);
  const size_t sb = scale_row_bytes<WF>(a.d);
  const size_t woff = (size_t)e * a.f + min(n0, a.f - 1);
  const char* gp = reinterpret_cast<const char*>(a.wg) + woff * rb;
  const char* up = reinterpret_cast<const char*>(a.wu) + woff * rb;
  const uint8_t* sgp = is_fp4(WF) ? a.sg + woff * sb : nullptr;
  const uint8_t* sup = is_fp4(WF) ? a.su + woff * sb : nullptr;

  RowRegs<WF, MAXC, RPW> G, U;
  if (!MULTISEG) {  // whole (part of the) rows, loaded once, before the token chain
    G.load_all(gp, rb, sgp, sb, nrows, cbeg, cend, lane);
    U.load_all(up, rb, sup, sb, nrows, cbeg, cend, lane);
  }
  const int r0 = a.slot_info[4 * slot + 1];
  const int ntok = a.slot_info[4 * slot + 2];
  const size_t xrb = (size_t)a.d * act_bytes<WF>();
  const int nseg = MULTISEG ? (nchunks + SEG - 1) / SEG : 1;
  for (int tt = 0; tt < ntok; ++tt) {
    const char* xr = reinterpret_cast<const char*>(a.x) +
                     (size_t)(dbg_idx(a.sorted_src[r0 + tt], a.T * a.k, kDbgSortedSrc) / a.k) * xrb;
    float ag[RPW], au[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) ag[r] = au[r] = 0.f;
    for (int seg = 0; seg < nseg; ++seg) {
      const int c0 = cbeg + seg * SEG;
      if (MULTISEG) {
        G.load_all(gp, rb, sgp, sb, nrows, c0, cend, lane);
        U.load_all(up, rb, sup, sb, nrows, c0, cend, lane);
      }
      XChunk<WF> xc[MAXC];
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = c0 + i * kWave + lane;
        if (c < cend) xc[i] = load_x<WF>(xr, c);
      }
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = c0 + i * kWave + lane;
        if (c < cend) {
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            ag[r] = G.fma_chunk(r, i, xc[i], ag[r]);
            au[r] = U.fma_chunk(r, i, xc[i], au[r]);
          }
        }
      }
    }
    if constexpr (KS == 1) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if (r < nrows) {
          const float gs = matrix_scaled<WF>(wave_sum(ag[r]), a.tg, e);
          const float us = matrix_scaled<WF>(wave_sum(au[r]), a.tu, e);
          if (lane == 0) store_act<WF>(a.h, (size_t)(r0 + tt) * a.f + n0 + r, silu(gs) * us);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float gs = wave_sum(ag[r]);
        const float us = wave_sum(au[r]);
        if (lane == 0) {
          red[wave][r][0] = gs;
          red[wave][r][1] = us;
        }
      }
      __syncthreads();
      if (part == 0 && lane < nrows) {
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int q = 0; q < KS; ++q) {
          gs += red[grp * KS + q][lane][0];
          us += red[grp * KS + q][lane][1];
        }
        store_act<WF>(a.h, (size_t)(r0 + tt) * a.f + n0 + lane, silu(gs) * us);
      }
      __syncthreads();
    }
  }
}

// Single token, balanced over the CUs: the grid is exactly the blocks the GPU
// holds at once, and wave g of W takes rows g, g + W, g + 2W, ... of all the
// active slots' rows laid end to end, so every CU streams the same number of
// rows and every wave starts at once (with a few blocks per CU, whole blocks
// per CU differ by up to half).  The activation row sits in LDS, chunk c at
// byte 80c (64 bytes plus padding, spreading neighbouring lanes over the
// banks), instead of in registers, leaving room for more waves.  A wave keeps
// the next row's loads in flight while it computes the current one.  Every
// global load and store is issued unconditionally (addresses clamped into the
// row; past the wave's last row the prefetch is a buffer load over an empty
// range, which returns zeros without touching memory), so the wait before a
// row's arithmetic covers that row's loads only, not the prefetch behind them.
// Requires d % 128 == 0 (whole 4-byte scale words per row).  Each row is
// computed as in gemv_gate_up_kernel: same chunks per lane, same order.
constexpr int kXStride = 80;
// Raw buffer descriptors: word 3 of the resource (32-bit data format, as for
// untyped loads) and the non-temporal cache-policy bit of a buffer load.
constexpr int kBufWord3 = 0x00020000;
constexpr int kBufNT = 2;

// One 4-bit weight row held by a wave: chunk c = i*64 + lane in w[i], the
// block scales of chunks 4*lane .. 4*lane+3 in sw (NVFP4: sw, sw2) until
// unpack().  Loads are buffer loads with in-row (clamped) offsets; live ==
// false gives empty ranges.  Needs whole scale words: chunks % 4 == 0.
template <int WF, int MAXC>
struct BufRow {
  u32x4 w[MAXC];
  uint32_t sw, sw2;
  float s[MAXC], s2[MAXC];

  __device__ __forceinline__ void load(const char* row, const uint8_t* srow, bool live, int rb,
                                       int sb, int nchunks, int lane) {
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)row, 0, live ? rb : 0, kBufWord3);
    const __amdgpu_buffer_rsrc_t sr =
        __builtin_amdgcn_make_buffer_rsrc((void*)srow, 0, live ? sb : 0, kBufWord3);
    const int qw = min(lane, (nchunks >> 2) - 1);
    if constexpr (WF == kNVFP4) {
      sw = __builtin_amdgcn_raw_buffer_load_b32(sr, 8 * qw, 0, 0);
      sw2 = __builtin_amdgcn_raw_buffer_load_b32(sr, 8 * qw + 4, 0, 0);
    } else {
      sw = __builtin_amdgcn_raw_buffer_load_b32(sr, 4 * qw, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < MAXC; ++i)
      w[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, min(i * kWave + lane, nchunks - 1) * 16, 0, kBufNT);
  }
  // Every lane of the wave must call.
  __device__ __forceinline__ void unpack(int lane) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = i * kWave + lane;
      const int src = (c >> 2) & (kWave - 1);
      const uint32_t v = __shfl(sw, src, kWave);
      if constexpr (WF == kMXFP4) {
        s[i] = e8m0_cvt_scale((v >> (8 * (c & 3))) & 0xffu);
      } else {
        const uint32_t v2 = __shfl(sw2, src, kWave);
        const uint32_t word = (c & 2) ? v2 : v;
        const uint32_t sh = 16 * (c & 1);
        s[i] = e4m3_to_f32((word >> sh) & 0xffu);
        s2[i] = e4m3_to_f32((word >> (sh + 8)) & 0xffu);
      }
    }
  }
  // acc + chunk i against x; a chunk past the row (the clamped duplicate) is
  // left out by a select, not a branch (a branch would hide waits)
  __device__ __forceinline__ float fma_chunk(int i, const XChunk<WF>& x, float acc, int nchunks,
                                             int lane) const {
    const float t = scaled_chunk<WF, false>(w[i], x, s[i], s2[i], acc);
    return i * kWave + lane < nchunks ? t : acc;
  }
};

// A gate/up row: gate and up weights of row n of an active slot's expert.
template <int WF, int MAXC>
struct T1Row {
  BufRow<WF, MAXC> g, u;
  int e;
  size_t hidx;  // element of h the row's result goes to

  // Row q (wave-uniform) of the active slots' rows.  Lane l of slot_e / slot_r
  // holds slot l's expert and first row (preloaded: a table lookup here would
  // be a vector load queued behind the prefetch, and waiting for it would wait
  // for everything).
  __device__ __forceinline__ void load(const GateUpArgs& a, int q, bool live, int slot_e,
                                       int slot_r, int nchunks, int lane) {
    const int slot = q / a.f;
    const int n = q - slot * a.f;
    e = __builtin_amdgcn_readlane(slot_e, slot);
    hidx = (size_t)__builtin_amdgcn_readlane(slot_r, slot) * a.f + n;
    const size_t woff = (size_t)e * a.f + n;
    const int rb = (int)WT<WF>::row_bytes(a.d);
    const int sb = (int)scale_row_bytes<WF>(a.d);
    g.load(reinterpret_cast<const char*>(a.wg) + woff * rb, a.sg + woff * sb, live, rb, sb, nchunks, lane);
    u.load(reinterpret_cast<const char*>(a.wu) + woff * rb, a.su + woff * sb, live, rb, sb, nchunks, lane);
  }
};

template <int WF, int MAXC>
__device__ __forceinline__ void t1_row_compute(const GateUpArgs& a, T1Row<WF, MAXC>& R,
                                               const char* xs, int nchunks, int lane) {
  R.g.unpack(lane);
  R.u.unpack(lane);
  float ag = 0.f, au = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    // re-read per row (the offset is hidden from the optimiser), so the
    // activations are not hoisted back into registers
    const char* xp = xs + opaque((uint32_t)(min(i * kWave + lane, nchunks - 1) * kXStride));
    XChunk<WF> xc;
#pragma unroll
    for (int j = 0; j < 4; ++j) xc.v[j] = *reinterpret_cast<const u32x4*>(xp + 16 * j);
    ag = R.g.fma_chunk(i, xc, ag, nchunks, lane);
    au = R.u.fma_chunk(i, xc, au, nchunks, lane);
  }
  const float gs = matrix_scaled<WF>(wave_sum(ag), a.tg, R.e);
  const float us = matrix_scaled<WF>(wave_sum(au), a.tu, R.e);
  store_act<WF>(a.h, R.hidx, silu(gs) * us);  // every lane stores the same value
}

// The token's activations (T = 1: row 0 of x) into LDS, 16 bytes per thread
// a step.  Every thread of the block calls; the loads go out first.
template <int MAXC>
__device__ __forceinline__ void t1_x_to_lds(const void* x, char* xs, int nchunks) {
  u32x4 xv[MAXC];
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int p = min(k * 256 + (int)threadIdx.x, nchunks * 4 - 1);
    xv[k] = ld16(reinterpret_cast<const char*>(x) + (size_t)p * 16);
  }
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int p = min(k * 256 + (int)threadIdx.x, nchunks * 4 - 1);
    *reinterpret_cast<u32x4*>(xs + (p >> 2) * kXStride + 16 * (p & 3)) = xv[k];
  }
}

// The row loop of the balanced single-token kernels, after x is in LDS (and a
// barrier): wave g of W takes rows g, g + W, ... of the nact * f rows.
template <int WF, int MAXC>
__device__ __forceinline__ void t1_bal_rows(const GateUpArgs& a, const char* xs, int nact, int slot_e,
                                            int slot_r, int nchunks, int lane, int wave) {
  const int W = gridDim.x * 4;
  const int N = nact * a.f;
  int q = blockIdx.x * 4 + wave;
  if (q >= N) q = N - 1;  // surplus waves (grid larger than the rows) redo the last row
  T1Row<WF, MAXC> A, B;
  A.load(a, q, true, slot_e, slot_r, nchunks, lane);
  for (;;) {
    const bool lb = q + W < N;
    const int qb = lb ? q + W : q;
    B.load(a, qb, lb, slot_e, slot_r, nchunks, lane);
    // memory instructions keep this order (the prefetch goes out before this
    // row's scale shuffles); arithmetic may cross
    __builtin_amdgcn_sched_barrier(1);
    t1_row_compute<WF, MAXC>(a, A, xs, nchunks, lane);
    if (!lb) break;
    const bool la = qb + W < N;
    const int qa = la ? qb + W : qb;
    A.load(a, qa, la, slot_e, slot_r, nchunks, lane);
    __builtin_amdgcn_sched_barrier(1);
    t1_row_compute<WF, MAXC>(a, B, xs, nchunks, lane);
    if (!la) break;
    q = qa;
  }
}

template <int WF, int MAXC>
__global__ __launch_bounds__(256) void gemv_gate_up_t1_bal_kernel(GateUpArgs a) {
  static_assert(is_fp4(WF), "4-bit weights only");
  extern __shared__ __align__(16) char xs[];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunks = a.d / WT<WF>::CE;
  const int nact = *a.num_active;  // at most k <= 64 slots for one token
  if (nact * a.f <= 0) return;     // uniform over the grid
  const int sl = min(lane, nact - 1);
  const int slot_e = a.slot_info[4 * sl + 0];
  const int slot_r = a.slot_info[4 * sl + 1];
  t1_x_to_lds<MAXC>(a.x, xs, nchunks);
  __syncthreads();
  t1_bal_rows<WF, MAXC>(a, xs, nact, slot_e, slot_r, nchunks, lane, wave);
}

// Routing for the routed variant: the token's logits and the outputs of the
// route and permute steps.
struct T1RouteArgs {
  const float* logits;
  int E;
  int* topk_idx;
  float* topk_w;
  Plan plan;
};

// gemv_gate_up_t1_bal_kernel with the routing step folded in, for one token:
// wave 0 of every block routes the token (the same selection and weights as
// the routing kernels) while the other waves stage x, and block 0 also writes
// the routing outputs and the whole plan for the kernels after it.  This
// saves a kernel launch, which costs more than the routing itself.
template <int WF, int MAXC, int VPL>
__global__ __launch_bounds__(256) void gemv_gate_up_t1_routed_kernel(GateUpArgs a, T1RouteArgs r) {
  static_assert(is_fp4(WF), "4-bit weights only");
  extern __shared__ __align__(16) char xs[];
  __shared__ int slot_expert[kWave];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunks = a.d / WT<WF>::CE;
  const int k = a.k;
  if (wave == 0) {
    int sel_i;
    float sel_w;
    route_token<VPL>(r.logits, r.E, k, sel_i, sel_w);
    const int rank = selected_rank(sel_i, k);
    if (lane < k) slot_expert[rank] = sel_i;
    if (blockIdx.x == 0) write_plan_t1(sel_i, sel_w, rank, r.E, k, r.topk_idx, r.topk_w, r.plan);
  }
  t1_x_to_lds<MAXC>(a.x, xs, nchunks);
  __syncthreads();
  // slot s (rank s) holds the s-th smallest selected expert and row s
  const int sl = min(lane, k - 1);
  t1_bal_rows<WF, MAXC>(a, xs, k, slot_expert[sl], sl, nchunks, lane, wave);
}

struct DownArgs {
  const void* h;
  const void* wd;
  const uint8_t* sd;
  const float* td;  // NVFP4 matrix scales [E]
  const int* slot_info;
  const int* num_active;
  float* y_sorted;
  int d, f;
};

// y_sorted[r][n] = <w_down[e][n], h[r]> for every row r of the slot's expert.
template <int WF, int MAXC, int RPW, bool MULTISEG>
__global__ __launch_bounds__(256) void gemv_down_kernel(DownArgs a) {
  constexpr int CE = WT<WF>::CE;
  constexpr int SEG = MAXC * kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int RB = 4 * RPW;
  const int tiles = (a.d + RB - 1) / RB;
  const int slot = blockIdx.x / tiles;
  if (slot >= *a.num_active) return;
  const int n0 = (blockIdx.x - slot * tiles) * RB + wave * RPW;
  if (n0 >= a.d) return;
  const int e = a.slot_info[4 * slot + 0];
  const int nrows = min(RPW, a.d - n0);
  const int nchunks = a.f / CE;
  const size_t rb = WT<WF>::row_bytes(a.f);
  const size_t sb = scale_row_bytes<WF>(a.f);
  const size_t woff = (size_t)e * a.d + n0;
  const char* wp = reinterpret_cast<const char*>(a.wd) + woff * rb;
  const uint8_t* sp = is_fp4(WF) ? a.sd + woff * sb : nullptr;

  RowRegs<WF, MAXC, RPW> W;
  if (!MULTISEG) W.load_all(wp, rb, sp, sb, nrows, 0, nchunks, lane);
  const int r0 = a.slot_info[4 * slot + 1];
  const int ntok = a.slot_info[4 * slot + 2];
  const size_t hrb = (size_t)a.f * act_bytes<WF>();
  const int nseg = MULTISEG ? (nchunks + SEG - 1) / SEG : 1;
  for (int tt = 0; tt < ntok; ++tt) {
    const char* hr = reinterpret_cast<const char*>(a.h) + (size_t)(r0 + tt) * hrb;
    float acc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[r] = 0.f;
    for (int seg = 0; seg < nseg; ++seg) {
      const int c0 = seg * SEG;
      if (MULTISEG) W.load_all(wp, rb, sp, sb, nrows, c0, nchunks, lane);
      XChunk<WF> hc[MAXC];
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = c0 + i * kWave + lane;
        if (c < nchunks) hc[i] = load_x<WF>(hr, c);
      }
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        const int c = c0 + i * kWave + lane;
        if (c < nchunks) {
#pragma unroll
          for (int r = 0; r < RPW; ++r) acc[r] = W.fma_chunk(r, i, hc[i], acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if (r < nrows) {
        const float y = matrix_scaled<WF>(wave_sum(acc[r]), a.td, e);
        if (lane == 0) a.y_sorted[(size_t)(r0 + tt) * a.d + n0 + r] = y;
      }
    }
  }
}

struct DownCombineArgs {
  const void* h;
  const void* wd;
  const uint8_t* sd;
  const float* td;
  const int* topk_idx;
  const float* topk_w;
  const int* dest_row;
  void* out;
  int d, f, k;
  int E;
};

// Single token: down projection fused with the weighted combine.  Block =
// k waves over the same RPW output rows, wave j on slot j's expert; the k
// results meet in LDS and are summed in slot order (the combine kernel's
// arithmetic), so no cross-block synchronisation is needed.
template <int WF, int MAXC, int RPW, int NTH>
__global__ __launch_bounds__(NTH) void gemv_down_combine_t1_kernel(DownCombineArgs a) {
  __shared__ float ys[16][RPW];
  constexpr int CE = WT<WF>::CE;
  const int lane = lane_id();
  const int j = threadIdx.x >> 6;
  const int n0 = blockIdx.x * RPW;
  const int nrows = min(RPW, a.d - n0);
  const int e = dbg_idx(a.topk_idx[j], a.E, kDbgExpert);
  const int nchunks = a.f / CE;
  const size_t rb = WT<WF>::row_bytes(a.f);
  const size_t sb = scale_row_bytes<WF>(a.f);
  const size_t woff = (size_t)e * a.d + n0;
  RowRegs<WF, MAXC, RPW> W;
  W.load_all(reinterpret_cast<const char*>(a.wd) + woff * rb, rb,
             is_fp4(WF) ? a.sd + woff * sb : nullptr, sb, nrows, 0, nchunks, lane);
  const char* hr =
      reinterpret_cast<const char*>(a.h) + (size_t)dbg_idx(a.dest_row[j], a.k, kDbgDestRow) * a.f * act_bytes<WF>();
  XChunk<WF> hc[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = i * kWave + lane;
    if (c < nchunks) hc[i] = load_x<WF>(hr, c);
  }
  float acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = i * kWave + lane;
    if (c < nchunks) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) acc[r] = W.template fma_chunk<false>(r, i, hc[i], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float y = matrix_scaled<WF>(wave_sum(acc[r]), a.td, e);
    if (lane == 0) ys[j][r] = y;
  }
  __syncthreads();
  if ((int)threadIdx.x < nrows) {
    const int r = threadIdx.x;
    float v = 0.f;
    for (int q = 0; q < a.k; ++q) v = fmaf(a.topk_w[q], ys[q][r], v);
    store_act<WF>(a.out, (size_t)n0 + r, v);
  }
}

// Single token, 4-bit weights: down projection fused with the weighted
// combine as in gemv_down_combine_t1_kernel (block = k waves over the same RPW
// output rows, wave j on slot j, results meeting in LDS and summed in slot
// order), but a wave streams its rows through a ring of D + 1 row buffers
// instead of holding all of them at once.  Fewer registers let the blocks the
// grid needs be resident together (holding all rows took two rounds).  The
// ring turns in a loop the compiler does not unroll, so it cannot hoist later
// rows' loads and undo the ring.  Loads are issued unconditionally -- past the
// block's rows as buffer loads over an empty range -- so the wait before a
// row's arithmetic covers that row only.  Each row is computed as in the
// other kernel: same chunks per lane, same order, a chunk past the row left
// out.  Requires f % 128 == 0 and RPW % (D + 1) == 0.
template <int WF, int MAXC, int RPW, int D, int NTH>
__global__ __launch_bounds__(NTH) void gemv_down_combine_t1_ring_kernel(DownCombineArgs a) {
  static_assert(is_fp4(WF), "4-bit weights only");
  static_assert(RPW % (D + 1) == 0, "whole turns of the ring");
  __shared__ float ys[16][RPW];
  const int lane = lane_id();
  const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * RPW;
  const int nrows = min(RPW, a.d - n0);
  const int e = dbg_idx(a.topk_idx[j], a.E, kDbgExpert);
  const int nchunks = a.f / WT<WF>::CE;
  const int rb = (int)WT<WF>::row_bytes(a.f);
  const int sb = (int)scale_row_bytes<WF>(a.f);
  // slot j's activations (its row of h), loaded first so that waiting for
  // them does not wait for the weights
  const char* hr = reinterpret_cast<const char*>(a.h) + (size_t)dbg_idx(a.dest_row[j], a.k, kDbgDestRow) * a.f * act_bytes<WF>();
  XChunk<WF> hc[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) hc[i] = load_x<WF>(hr, min(i * kWave + lane, nchunks - 1));
  const size_t woff = (size_t)e * a.d + n0;
  const char* w0 = reinterpret_cast<const char*>(a.wd) + woff * rb;
  const uint8_t* s0 = a.sd + woff * sb;
  auto load_row = [&](BufRow<WF, MAXC>& buf, int r) {
    const int rr = min(r, nrows - 1);
    buf.load(w0 + (size_t)rr * rb, s0 + (size_t)rr * sb, r < nrows, rb, sb, nchunks, lane);
  };
  BufRow<WF, MAXC> ring[D + 1];
#pragma unroll
  for (int r = 0; r < D; ++r) load_row(ring[r], r);
#pragma unroll 1
  for (int r0 = 0; r0 < RPW; r0 += D + 1) {
#pragma unroll
    for (int t = 0; t <= D; ++t) {
      load_row(ring[(t + D) % (D + 1)], r0 + t + D);
      // memory instructions keep this order; arithmetic may cross
      __builtin_amdgcn_sched_barrier(1);
      ring[t].unpack(lane);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < MAXC; ++i) acc = ring[t].fma_chunk(i, hc[i], acc, nchunks, lane);
      const float y = matrix_scaled<WF>(wave_sum(acc), a.td, e);
      ys[j][r0 + t] = y;  // every lane writes the same value
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < nrows) {
    const int r = threadIdx.x;
    float v = 0.f;
    for (int q = 0; q < a.k; ++q) v = fmaf(a.topk_w[q], ys[q][r], v);
    store_act<WF>(a.out, (size_t)n0 + r, v);
  }
}

// ---------------------------------------------------------------- launch --
int chunk_elems(int wf) { return wf == kF32 ? 4 : (wf == kBF16 ? 8 : 32); }  // 4-bit: 32

// Registers per lane for one row: the smallest supported MAXC covering the
// row (4-bit formats capped at 4: each chunk needs 64 B of activations).
int pick_maxc(int nchunks, int wf) {
  const int need = (nchunks + kWave - 1) / kWave;
  static const int opts[] = {1, 2, 3, 4, 6, 8, 12, 16};
  const int cap = is_fp4(wf) ? 4 : 16;
  for (int o : opts)
    if (need <= o && o <= cap) return o;
  return cap;
}

// Rows per wave: about 12 chunks per matrix in flight, and for short rows
// enough rows that each token's activations (read per wave from L2) stay
// below the weight bytes they are applied to (MX-FP4 gate/up rows of 96
// chunks at T = 16: 420 us with one row per wave, 383 us with two).
constexpr int rpw_for(int maxc) { return maxc >= 12 ? 1 : (maxc >= 6 ? 2 : (maxc >= 3 ? 2 : 4)); }
constexpr int rpw_t1_small(int maxc) { return maxc <= 2 ? 8 : rpw_for(maxc); }

#define MOE_MAXC_SWITCH(WFV, MAXC, CALL)                                              \
  switch (MAXC) {                                                                     \
    case 1: { constexpr int MC = 1; CALL; } break;                                    \
    case 2: { constexpr int MC = 2; CALL; } break;                                    \
    case 3: { constexpr int MC = 3; CALL; } break;                                    \
    case 4: { constexpr int MC = 4; CALL; } break;                                    \
    case 6: { if constexpr (!is_fp4(WFV)) { constexpr int MC = 6; CALL; } } break;   \
    case 8: { if constexpr (!is_fp4(WFV)) { constexpr int MC = 8; CALL; } } break;   \
    case 12: { if constexpr (!is_fp4(WFV)) { constexpr int MC = 12; CALL; } } break; \
    default: { if constexpr (!is_fp4(WFV)) { constexpr int MC = 16; CALL; } } break; \
  }

#define MOE_MAXC12_SWITCH(WFV, MAXC, CALL)                                            \
  switch (MAXC) {                                                                     \
    case 1: { constexpr int MC = 1; CALL; } break;                                    \
    case 2: { constexpr int MC = 2; CALL; } break;                                    \
    case 3: { constexpr int MC = 3; CALL; } break;                                    \
    case 4: { if constexpr (!is_fp4(WFV)) { constexpr int MC = 4; CALL; } } break;   \
    case 6: { if constexpr (!is_fp4(WFV)) { constexpr int MC = 6; CALL; } } break;   \
    case 8: { if constexpr (!is_fp4(WFV)) { constexpr int MC = 8; CALL; } } break;   \
    default: { if constexpr (!is_fp4(WFV)) { constexpr int MC = 12; CALL; } } break; \
  }

#define MOE_WF_SWITCH(WFV, CALL)                             \
  switch (WFV) {                                             \
    case kF32: { constexpr int WF = kF32; CALL; } break;      \
    case kBF16: { constexpr int WF = kBF16; CALL; } break;    \
    case kMXFP4: { constexpr int WF = kMXFP4; CALL; } break;  \
    default: { constexpr int WF = kNVFP4; CALL; } break;      \
  }

#define MOE_SEG_SWITCH(MULTI, CALL)                 \
  if (MULTI) { constexpr bool MS = true; CALL; }     \
  else { constexpr bool MS = false; CALL; }

// Blocks of `threads` threads that the current device holds at once for kernel
// `fn` with `lds` bytes of dynamic LDS: CUs times blocks per CU (cached per
// device, kernel and LDS size).
long long resident_blocks(const void* fn, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, long long> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  const auto key = std::make_tuple(dev, fn, lds);
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess)
    return 1;
  const long long n = std::max(1LL, (long long)cus * per_cu);
  cache[key] = n;
  return n;
}

}  // namespace

hipError_t launch_gemv_gate_up(const Dims& dm, const void* x, const Plan& p, const Weights& w,
                               void* h, hipStream_t s) {
  LaunchTimer tm("gemv_gate_up", s);
  GateUpArgs a{x, w.wg, w.wu, w.sg, w.su, w.tg, w.tu, p.sorted_src, p.slot_info, p.num_active,
               h, dm.d, dm.f, dm.k, dm.T};
  const long long max_active = dm.Tk() < dm.E ? dm.Tk() : dm.E;
  const int nchunks = dm.d / chunk_elems(dm.wfmt);
  const int maxc = pick_maxc(nchunks, dm.wfmt);
  const bool multi = nchunks > maxc * kWave;
  if (!multi && !is_fp4(dm.wfmt) && maxc >= 8) {
    // long rows: four waves per row, each streaming a quarter of it (more,
    // lighter waves in flight: measured 79.5 us against 90.2 us with halves
    // for the single-token bf16 layer at d = 6144)
    const int maxc4 = pick_maxc((nchunks + 3) / 4, dm.wfmt);
    const dim3 grid((unsigned)(max_active * dm.f)), block(256);
    if (dm.wfmt == kBF16) {
      if (maxc4 <= 2) gemv_gate_up_kernel<kBF16, 2, 1, 4, false><<<grid, block, 0, s>>>(a);
      else if (maxc4 <= 3) gemv_gate_up_kernel<kBF16, 3, 1, 4, false><<<grid, block, 0, s>>>(a);
      else gemv_gate_up_kernel<kBF16, 4, 1, 4, false><<<grid, block, 0, s>>>(a);
    } else {
      if (maxc4 <= 2) gemv_gate_up_kernel<kF32, 2, 1, 4, false><<<grid, block, 0, s>>>(a);
      else if (maxc4 <= 3) gemv_gate_up_kernel<kF32, 3, 1, 4, false><<<grid, block, 0, s>>>(a);
      else gemv_gate_up_kernel<kF32, 4, 1, 4, false><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
  }
  if (dm.T == 1 && is_fp4(dm.wfmt) && !multi && dm.d % 128 == 0 && dm.k <= kWave) {
    // short rows, one token: rows dealt evenly over a grid the GPU holds at once
    const size_t lds = (size_t)nchunks * kXStride;
    const long long rows = max_active * dm.f;
    auto go = [&](const void* fn, auto kern) {
      const long long g = std::min<long long>(resident_blocks(fn, 256, lds), (rows + 3) / 4);
      kern<<<dim3((unsigned)std::max<long long>(g, 1)), dim3(256), lds, s>>>(a);
    };
#define MOE_T1BAL(WFV)                                                                                       \
  switch (maxc) {                                                                                            \
    case 1: go((const void*)gemv_gate_up_t1_bal_kernel<WFV, 1>, gemv_gate_up_t1_bal_kernel<WFV, 1>); break;  \
    case 2: go((const void*)gemv_gate_up_t1_bal_kernel<WFV, 2>, gemv_gate_up_t1_bal_kernel<WFV, 2>); break;  \
    case 3: go((const void*)gemv_gate_up_t1_bal_kernel<WFV, 3>, gemv_gate_up_t1_bal_kernel<WFV, 3>); break;  \
    default: go((const void*)gemv_gate_up_t1_bal_kernel<WFV, 4>, gemv_gate_up_t1_bal_kernel<WFV, 4>); break; \
  }
    if (dm.wfmt == kMXFP4) {
      MOE_T1BAL(kMXFP4)
    } else {
      MOE_T1BAL(kNVFP4)
    }
#undef MOE_T1BAL
    return hipGetLastError();
  }
  const int rpw = rpw_for(maxc);
  const dim3 grid((unsigned)(max_active * ((dm.f + 4 * rpw - 1) / (4 * rpw)))), block(256);
  MOE_WF_SWITCH(dm.wfmt, MOE_MAXC_SWITCH(WF, maxc, MOE_SEG_SWITCH(multi, (
      gemv_gate_up_kernel<WF, MC, rpw_for(MC), 1, MS><<<grid, block, 0, s>>>(a)))));
  return hipGetLastError();
}

bool gemv_gate_up_t1_routed_ok(const Dims& dm) {
  const int nchunks = dm.d / chunk_elems(dm.wfmt);
  return dm.T == 1 && is_fp4(dm.wfmt) && nchunks <= 4 * kWave && dm.d % 128 == 0 && dm.k <= kWave &&
         dm.E <= 16 * kWave;
}

hipError_t launch_gemv_gate_up_t1_routed(const Dims& dm, const float* logits, const void* x,
                                         const Plan& p, const Weights& w, void* h, int* topk_idx,
                                         float* topk_w, hipStream_t s) {
  LaunchTimer tm("gemv_gate_up", s);
  GateUpArgs a{x, w.wg, w.wu, w.sg, w.su, w.tg, w.tu, p.sorted_src, p.slot_info, p.num_active,
               h, dm.d, dm.f, dm.k, dm.T};
  const T1RouteArgs r{logits, dm.E, topk_idx, topk_w, p};
  const int nchunks = dm.d / chunk_elems(dm.wfmt);
  const int maxc = pick_maxc(nchunks, dm.wfmt);
  const size_t lds = (size_t)nchunks * kXStride;
  const long long rows = (long long)dm.k * dm.f;
  auto go = [&](auto kern) {
    const long long g = std::min<long long>(resident_blocks((const void*)kern, 256, lds), (rows + 3) / 4);
    kern<<<dim3((unsigned)std::max<long long>(g, 1)), dim3(256), lds, s>>>(a, r);
  };
  // logits per lane: E <= 64 * VPL
  auto by_vpl = [&](auto wf, auto mc) {
    constexpr int WF = decltype(wf)::value, MC = decltype(mc)::value;
    if (dm.E <= 64) go(gemv_gate_up_t1_routed_kernel<WF, MC, 1>);
    else if (dm.E <= 128) go(gemv_gate_up_t1_routed_kernel<WF, MC, 2>);
    else if (dm.E <= 256) go(gemv_gate_up_t1_routed_kernel<WF, MC, 4>);
    else if (dm.E <= 512) go(gemv_gate_up_t1_routed_kernel<WF, MC, 8>);
    else go(gemv_gate_up_t1_routed_kernel<WF, MC, 16>);
  };
  auto by_maxc = [&](auto wf) {
    switch (maxc) {
      case 1: by_vpl(wf, std::integral_constant<int, 1>{}); break;
      case 2: by_vpl(wf, std::integral_constant<int, 2>{}); break;
      case 3: by_vpl(wf, std::integral_constant<int, 3>{}); break;
      default: by_vpl(wf, std::integral_constant<int, 4>{}); break;
    }
  };
  if (dm.wfmt == kMXFP4)
    by_maxc(std::integral_constant<int, kMXFP4>{});
  else
    by_maxc(std::integral_constant<int, kNVFP4>{});
  return hipGetLastError();
}

hipError_t launch_gemv_down(const Dims& dm, const void* h, const Plan& p, const Weights& w,
                            float* y_sorted, hipStream_t s) {
  LaunchTimer tm("gemv_down", s);
  DownArgs a{h, w.wd, w.sd, w.td, p.slot_info, p.num_active, y_sorted, dm.d, dm.f};
  const long long max_active = dm.Tk() < dm.E ? dm.Tk() : dm.E;
  const int nchunks = dm.f / chunk_elems(dm.wfmt);
  const int maxc = pick_maxc(nchunks, dm.wfmt);
  const bool multi = nchunks > maxc * kWave;
  const int rpw = rpw_for(maxc);
  const dim3 grid((unsigned)(max_active * ((dm.d + 4 * rpw - 1) / (4 * rpw)))), block(256);
  MOE_WF_SWITCH(dm.wfmt, MOE_MAXC_SWITCH(WF, maxc, MOE_SEG_SWITCH(multi, (
      gemv_down_kernel<WF, MC, rpw_for(MC), MS><<<grid, block, 0, s>>>(a)))));
  return hipGetLastError();
}

bool gemv_down_combine_t1_ok(const Dims& dm) {
  // up to 1024 threads per block leave 128 VGPRs per lane: keep rows short
  // enough that the weight registers fit without spilling
  const int nchunks = dm.f / chunk_elems(dm.wfmt);
  const int maxc = pick_maxc(nchunks, dm.wfmt);
  const int limit = is_fp4(dm.wfmt) ? 3 : 12;
  return dm.T == 1 && dm.k <= 16 && nchunks <= maxc * kWave && maxc <= limit;
}

hipError_t launch_gemv_down_combine_t1(const Dims& dm, const void* h, const Plan& p,
                                       const int* topk_idx, const float* topk_w,
                                       const Weights& w, void* out, hipStream_t s) {
  LaunchTimer tm("gemv_down_combine_t1", s);
  DownCombineArgs a{h, w.wd, w.sd, w.td, topk_idx, topk_w, p.dest_row, out, dm.d, dm.f, dm.k, dm.E};
  const int maxc = pick_maxc(dm.f / chunk_elems(dm.wfmt), dm.wfmt);
  const dim3 block(64 * dm.k);
  if (is_fp4(dm.wfmt) && dm.k <= 8 && maxc <= 2 && dm.f % 128 == 0) {
    // 4-bit rows of up to 128 chunks: 12 output rows per block streamed
    // through a four-row ring (d = 6144 gives 512 blocks, two per CU)
    const dim3 grid((unsigned)((dm.d + 11) / 12));
    if (dm.wfmt == kMXFP4) {
      if (maxc == 1) gemv_down_combine_t1_ring_kernel<kMXFP4, 1, 12, 3, 512><<<grid, block, 0, s>>>(a);
      else gemv_down_combine_t1_ring_kernel<kMXFP4, 2, 12, 3, 512><<<grid, block, 0, s>>>(a);
    } else {
      if (maxc == 1) gemv_down_combine_t1_ring_kernel<kNVFP4, 1, 12, 3, 512><<<grid, block, 0, s>>>(a);
      else gemv_down_combine_t1_ring_kernel<kNVFP4, 2, 12, 3, 512><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
  }
  if (dm.k <= 8) {  // 512-thread blocks: up to 256 registers, twice the short rows per wave
    const int rpw = rpw_t1_small(maxc);
    const dim3 grid((unsigned)((dm.d + rpw - 1) / rpw));
    MOE_WF_SWITCH(dm.wfmt, MOE_MAXC12_SWITCH(WF, maxc, (
        gemv_down_combine_t1_kernel<WF, MC, rpw_t1_small(MC), 512><<<grid, block, 0, s>>>(a))));
  } else {
    const int rpw = rpw_for(maxc);
    const dim3 grid((unsigned)((dm.d + rpw - 1) / rpw));
    MOE_WF_SWITCH(dm.wfmt, MOE_MAXC12_SWITCH(WF, maxc, (
        gemv_down_combine_t1_kernel<WF, MC, rpw_for(MC), 1024><<<grid, block, 0, s>>>(a))));
  }
  return hipGetLastError();
}

MOE_DBG_TAKE_DEFINE(dbg_take_gemv)

}  // namespace moe
