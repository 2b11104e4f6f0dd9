// Device-side helpers shared by the gfx950 kernels: number formats, wave64
// reductions and streaming loads.  Written for CDNA4 only (wave64, MFMA).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace moe {

constexpr int kWave = 64;

// 16 bytes as a native clang vector (HIP's uint4 is a struct, which the
// non-temporal builtins do not accept).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Storage formats (Fmt values: internal.h)
// ---------------------------------------------------------------------------
// bf16 is kept as raw uint16 bits: the upper half of an fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.  One gfx950
// convert (v_cvt_pk_bf16_f32), with no branch: a data-dependent branch inside
// a streaming loop makes the compiler's wait counting conservative.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// An E8M0 byte as the scale operand of the gfx950 scaled FP4 converts: they
// read only the exponent field, with E8M0 meaning (checked on the device:
// exponent 0 scales by 2^-127, exponent 255 gives NaN), so the byte goes
// straight into the exponent.  Not a value for fp32 arithmetic.
__device__ __forceinline__ float e8m0_cvt_scale(uint32_t s) { return __uint_as_float(s << 23); }

// OCP FP8 E4M3 byte (the low byte of b) -> fp32, exactly, by the gfx950
// convert, which reads the OCP format: 1 sign, 4 exponent bits (bias 7), 3
// mantissa bits, subnormals m * 2^-9 at exponent 0, NaN for 0x7F and 0xFF
// (outside the supported inputs).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two E2M1 codes in byte `sel` of `w` -> packed bf16 pair (low nibble in the
// low half), each times the power of two in `sc`'s exponent field.  E2M1
// values are exact in bf16; scaled ones are while finite.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w, float sc = 1.0f) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, SEL));
}

// acc + a.lo*b.lo + a.hi*b.hi for packed bf16 pairs (v_dot2c_f32_bf16; the
// bf16 products are exact in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Hide a value from loop-invariant code motion (an empty asm that "modifies"
// it), so per-use conversions are not hoisted into extra live registers.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// ---------------------------------------------------------------------------
// Wave64 reductions (xor butterfly: every lane ends with the same value)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Block-wide exclusive prefix sum of one int per thread (blockDim.x a
// multiple of 64, at most 1024).  `tmp` needs 17 ints of LDS.  Also returns
// the block total.  Contains barriers: every thread of the block must call.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) tmp[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nwaves; ++w) {
      int c = tmp[w];
      tmp[w] = run;
      run += c;
    }
    tmp[16] = run;
  }
  __syncthreads();
  int res = tmp[wave] + incl - v;
  *total = tmp[16];
  __syncthreads();
  return res;
}

// ---------------------------------------------------------------------------
// Debug builds (MOE_DEBUG_CHECKS): bounds checks on index arrays
// ---------------------------------------------------------------------------
// An index read from memory (dest_row, sorted_src, an expert id, a row range
// of the plan) is checked before it addresses anything: out of [0, n) it sets
// bit `code` of this file's flag word and is clamped into range, so the
// access stays in bounds and the kernel runs to its end (wrong results, no
// fault).  moe_debug_check() reads and clears the flag words of every file.
// Release builds compile the checks away.
enum : unsigned {
  kDbgDestRow = 1u,     // dest_row outside [0, T*k)
  kDbgSortedSrc = 2u,   // sorted_src outside [0, T*k)
  kDbgExpert = 4u,      // expert id outside [0, E)
  kDbgRows = 8u,        // a segment's rows outside [0, T*k]
  kDbgOffsets = 16u,    // offsets not ascending from 0 to T*k
  kDbgTopk = 32u        // topk_idx outside [0, E)
};
#ifdef MOE_DEBUG_CHECKS
static __device__ unsigned g_dbg_flags;
__device__ __forceinline__ int dbg_idx(int v, int n, unsigned code) {
  if ((unsigned)v >= (unsigned)n) {
    atomicOr(&g_dbg_flags, code);
    v = v < 0 ? 0 : n - 1;
  }
  return v;
}
__device__ __forceinline__ void dbg_flag(bool bad, unsigned code) {
  if (bad) atomicOr(&g_dbg_flags, code);
}
// Host side, one per file: OR this file's flag word into *flags, then clear it.
#define MOE_DBG_TAKE_DEFINE(NAME)                                                 \
  hipError_t NAME(unsigned* flags) {                                              \
    unsigned v = 0, z = 0;                                                        \
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_dbg_flags), sizeof v);     \
    if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(g_dbg_flags), &z, sizeof z); \
    *flags |= v;                                                                  \
    return e;                                                                     \
  }
#else
__device__ __forceinline__ int dbg_idx(int v, int, unsigned) { return v; }
__device__ __forceinline__ void dbg_flag(bool, unsigned) {}
#define MOE_DBG_TAKE_DEFINE(NAME) \
  hipError_t NAME(unsigned*) { return hipSuccess; }
#endif

// ---------------------------------------------------------------------------
// Loads
// ---------------------------------------------------------------------------
// Streaming (non-temporal) 16-byte load: weights are read once per call, so
// they should not evict reusable lines from L2.
__device__ __forceinline__ u32x4 ld_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

}  // namespace moe
