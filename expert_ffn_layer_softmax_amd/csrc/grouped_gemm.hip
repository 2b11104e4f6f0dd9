// Expert FFN for many tokens per expert (prefill): grouped GEMMs on MFMA.
//
// Prefill's bottleneck differs from token-by-token decode (SGLang-TorchTPU
// on TPU v7 page, "Key optimizations": the prefill path uses a fused MoE
// kernel of its own).  Here every expert's rows form a dense contraction:
//   gate/up: H_e = silu(X_e W_gate[e]^T) * (X_e W_up[e]^T), X_e gathered from x
//   down:    Y_e = H_e W_down[e]^T
// computed with v_mfma_f32_32x32x16_bf16 and fp32 accumulation (TensorSharp
// Muse Spark report, "Answer quality": bf16 partial sums cost accuracy).
// MX-FP4 weights are dequantised to bf16 in registers by the gfx950 scaled
// convert (the block scale is applied by the instruction), then fed to the
// same MFMA.
//
// Every kernel works on tiles of 128 rows (one m-tile of an expert) with 8
// waves (two per SIMD), K advancing 64 per step, and skips the 32-row
// sub-tiles of an m-tile that hold no rows of the expert (skewed routing
// leaves most m-tiles partly filled).
//
// gg_dma_kernel (bf16 weights): 256 weight rows per tile (gate/up: 128
// columns of W_gate and the same 128 of W_up, so the SwiGLU epilogue is
// wave-local; down: 256 columns of W_down).  Both operands are fetched with
// global_load_lds straight into three XOR-swizzled LDS stages, two steps
// ahead of the MFMAs; waves form a 2 (rows) x 4 (columns) grid of 64 x 64.
//
// gg_mx_group_kernel (MX-FP4 weights, K % 256 == 0): the same tile and wave
// grid; activation rows as above, weight codes fetched in whole cache lines
// (four K-steps of a row per line) into group buffers two groups ahead, and
// converted to bf16 in registers by the gfx950 scaled convert (block scale
// applied by the instruction) just before their MFMAs.
//
// gg_mx_row_kernel (NVFP4 weights, K % 256 == 0): the same loads, with the
// eight waves side by side, each owning all 128 rows and 32 weight rows.
//
// gg_direct_b_kernel (MX-FP4 weights, other K): each wave owns all 128 rows
// and two 32-column weight operands that stream from memory into a register
// ring; the activation rows go through a register ring into double-buffered
// LDS.  K % 64 == 32 adds one tail step after the loop (both GEMM kernels
// for bf16 and MX-FP4 take it).
//
// Tile order: logical tiles run expert by expert, n-tile by n-tile, m-tile
// by m-tile, and each XCD (blockIdx % 8 under round-robin dispatch) takes a
// contiguous range.  The m-tiles of one (expert, n-tile) panel therefore run
// together on one XCD and share the weight panel through its L2; the n-tiles
// of one expert follow each other there and reuse its activation rows.  The
// MX-FP4 group kernel and the FP8-by-FP4 kernel swap the inner two levels
// (m-tile by m-tile, then n-tile): their weight panels are a quarter or half
// the bytes of bf16 ones, and keeping one m-tile's activation rows hot was
// measured faster there, while for bf16 weights it raised the fetched bytes.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace moe {
namespace {

// silu(g) * u = g * u / (1 + e^-g) for the gate/up epilogues, with the
// hardware exponential and reciprocal (each about one ulp of fp32) instead of
// the library expf and an IEEE division: h is rounded to bf16 or MXFP8 right
// after, far more coarsely, and with one block per CU nothing hides the
// epilogue's instructions.  Large negative g gives 0 (the exponential
// overflows to inf, its reciprocal to 0), as the exact form does; silu(g) is
// formed before the product with u, so a large u cannot turn that 0 into
// inf * 0 = NaN.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896f * g)) * u;
}


// OCP FP8 E4M3 byte of v (already divided by its block scale): round to
// nearest even, saturating at +-448 (the convert itself would give NaN).  A
// NaN stays NaN: the clamp would turn it into -448, so it is selected around.
__device__ __forceinline__ uint32_t e4m3_byte(float v) {
  const float c = fminf(fmaxf(v, -448.0f), 448.0f);
  v = v != v ? v : c;
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xffu;
}

// E8M0 byte of a block whose largest magnitude is amax: 2^(floor(log2 amax)
// - 8), the MX rule for E4M3 elements, kept in [1, 254].  amax is taken with
// fmaxf, which skips NaN: a block's scale comes from its non-NaN elements.
__device__ __forceinline__ uint32_t mxfp8_scale_byte(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return (uint32_t)min(max(ef - 8, 1), 254);
}

// v rounded to the MXFP8 grid of a 32-element block whose largest magnitude
// is amax, as fp32: E4M3(code) * 2^(s - 127), which bf16 holds exactly for
// block scales s >= 3 (smaller ones only below 2^-124).
__device__ __forceinline__ float mxfp8_round(float v, float amax) {
  const uint32_t sbyte = mxfp8_scale_byte(amax);
  const float inv = __uint_as_float((254u - sbyte) << 23);  // 2^(127 - s)
  return e4m3_to_f32(e4m3_byte(v * inv)) * __uint_as_float(sbyte << 23);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = kGemmBM;  // 128
constexpr int BK = 64;
constexpr int kThreads = 512;
constexpr int kXcds = 8;

struct GGArgs {
  const void* a_src;      // gate/up: x [T][K]; down: h [T*k][K] (bf16)
  const int* sorted_src;  // gate/up: row r reads x[sorted_src[r] / k]
  const void* w0;         // gate/up: W_gate; down: W_down   ([E][N][K] or codes)
  const void* w1;         // gate/up: W_up
  const uint8_t* s0;      // 4-bit block scales of w0 / w1
  const uint8_t* s1;
  const float* t0;        // NVFP4 matrix scales [E] of w0 / w1
  const float* t1;
  const uint8_t* a_scale; // FP8 activations: E8M0 scales [rows][K/32] of a_src
  void* out_scale;        // FP8 gate/up: E8M0 scales [T*k][N/32] of the fp8 h in out
  const int* mtiles;
  const int* num_mtiles;
  void* out;              // gate/up: h bf16 [T*k][N]; down: y_sorted fp32 [T*k][N]
  int K, N, k, ntiles;
  int T;                  // tokens: sorted_src values lie in [0, T*k)
};

// LDS tiles hold rows of 128 B (64 bf16 of K).  16-byte unit u of row r
// lives at unit u ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1): a fragment read
// (16 consecutive rows, one unit) then touches 16 distinct 16-byte bank
// groups, and so do 8 consecutive rows, and the row-wise stores of the
// global fetch (8 units of one row per 8 lanes) stay conflict-free too.
__device__ __forceinline__ int t_off(int row, int unit) {
  const int f = (row & 7) ^ ((row >> 3) & 1);
  return row * (BK * 2) + ((unit ^ f) << 4);
}

constexpr int kAPieces = BM * 8 / kThreads;  // 16-B pieces of A per thread per step

template <int WF>
struct BRegs;
template <>
struct BRegs<kBF16> {  // 4 x 16 B per matrix per step: the lane's 32 K-values
  u32x4 v[2][4];
};
template <>
struct BRegs<kMXFP4> {  // 16 B of codes (one 32-element block) and its scale per matrix
  u32x4 v[2];
  uint32_t s[2];
};

template <int WF>
__device__ __forceinline__ void load_b(BRegs<WF>& b, const char* p0, const char* p1,
                                       const uint8_t* q0, const uint8_t* q1, int kk) {
  if constexpr (WF == kBF16) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      b.v[0][s] = ld16(p0 + (size_t)kk * (BK * 2) + 16 * s);
      b.v[1][s] = ld16(p1 + (size_t)kk * (BK * 2) + 16 * s);
    }
  } else {
    b.v[0] = ld16(p0 + (size_t)kk * (BK / 2));
    b.v[1] = ld16(p1 + (size_t)kk * (BK / 2));
    b.s[0] = q0[2 * kk];
    b.s[1] = q1[2 * kk];
  }
}

// B fragment s (K offsets 8s..8s+7 of the lane's 32) of matrix m.
template <int WF>
__device__ __forceinline__ bf16x8_t b_frag(const BRegs<WF>& b, int m, int s) {
  if constexpr (WF == kBF16) {
    return __builtin_bit_cast(bf16x8_t, b.v[m][s]);
  } else {
    const uint32_t w = b.v[m][s];
    const float sc = e8m0_cvt_scale(b.s[m]);
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
    return __builtin_bit_cast(bf16x8_t, r);
  }
}

constexpr int BN = 256;  // weight rows per tile of gg_dma_kernel and gg_mx_group_kernel

template <int WF, bool GATEUP, int D>
__global__ __launch_bounds__(kThreads) void gg_direct_b_kernel(GGArgs a) {
  __shared__ __align__(16) char lds_a[2][BM * BK * 2];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int cl = lane & 31;

  // ---- tile
  const int num_tiles = *a.num_mtiles * a.ntiles;
  const int per_xcd = (num_tiles + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int L = (blockIdx.x % kXcds) * per_xcd + slot;
  if (L >= num_tiles) return;
  const int* eq = a.mtiles + kMtileInts * (L / a.ntiles);
  const int e = eq[0];
  const int first_mt = eq[3];
  const int nmt = eq[4];
  const int local = L - first_mt * a.ntiles;
  const int ntile = local / nmt;
  const int* em = a.mtiles + kMtileInts * (first_mt + (local - ntile * nmt));
  const int row0 = em[1];
  const int nrows = em[2];

  // ---- B columns of this lane
  int col0, col1;
  if (GATEUP) {
    col0 = ntile * 256 + wave * 32 + cl;
    col1 = col0;
  } else {
    col0 = ntile * 512 + wave * 64 + cl;
    col1 = col0 + 32;
  }
  const int c0c = min(col0, a.N - 1);
  const int c1c = min(col1, a.N - 1);
  const char* wb0 = reinterpret_cast<const char*>(a.w0);
  const char* wb1 = reinterpret_cast<const char*>(GATEUP ? a.w1 : a.w0);
  const char *p0, *p1;
  const uint8_t *q0 = nullptr, *q1 = nullptr;
  if constexpr (WF == kBF16) {
    p0 = wb0 + ((size_t)e * a.N + c0c) * a.K * 2 + half * 64;
    p1 = wb1 + ((size_t)e * a.N + c1c) * a.K * 2 + half * 64;
  } else {
    p0 = wb0 + ((size_t)e * a.N + c0c) * (a.K / 2) + half * 16;
    p1 = wb1 + ((size_t)e * a.N + c1c) * (a.K / 2) + half * 16;
    q0 = a.s0 + ((size_t)e * a.N + c0c) * (a.K / 32) + half;
    q1 = (GATEUP ? a.s1 : a.s0) + ((size_t)e * a.N + c1c) * (a.K / 32) + half;
  }

  // ---- A pieces of this thread: rows tid/8 + 64 i, unit tid%8
  const int unit = tid & 7;
  const size_t a_rb = (size_t)a.K * 2;
  const char* ap[kAPieces];
#pragma unroll
  for (int i = 0; i < kAPieces; ++i) {
    const int r = (tid >> 3) + i * (kThreads / 8);
    const int src = row0 + min(r, nrows - 1);
    ap[i] = reinterpret_cast<const char*>(a.a_src) +
            (GATEUP ? (size_t)(dbg_idx(a.sorted_src[src], a.T * a.k, kDbgSortedSrc) / a.k) : (size_t)src) * a_rb + unit * 16;
  }

  // K % 64 == 32: step nk is a tail of 32 K.  Its A units 4..7 and the
  // half-1 lanes' weight block lie past the row: they re-read the step's
  // first half (in bounds), and the half-1 lanes feed zeros to its MFMAs.
  const int nk = a.K / BK;
  const int ns = (a.K + BK - 1) / BK;  // steps, the tail included
  const int aback = unit >= 4 ? 64 : 0;
  u32x4 aring[D][kAPieces];
  BRegs<WF> bring[D];
  auto load_a = [&](u32x4* r, int kk) {
    const size_t off = (size_t)kk * (BK * 2) - (kk == nk ? aback : 0);
#pragma unroll
    for (int i = 0; i < kAPieces; ++i) r[i] = ld16(ap[i] + off);
  };
  auto load_b_step = [&](BRegs<WF>& b, int kk) {
    if (kk < nk) {
      load_b<WF>(b, p0, p1, q0, q1, kk);
    } else if constexpr (WF == kBF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        b.v[0][q] = ld16(p0 + (size_t)nk * (BK * 2) - half * 64 + 16 * q);
        b.v[1][q] = ld16(p1 + (size_t)nk * (BK * 2) - half * 64 + 16 * q);
      }
    } else {
      b.v[0] = ld16(p0 + (size_t)nk * (BK / 2) - half * 16);
      b.v[1] = ld16(p1 + (size_t)nk * (BK / 2) - half * 16);
      b.s[0] = q0[2 * nk - half];
      b.s[1] = q1[2 * nk - half];
    }
  };
  auto store_a = [&](const u32x4* r, int buf) {
#pragma unroll
    for (int i = 0; i < kAPieces; ++i)
      *reinterpret_cast<u32x4*>(&lds_a[buf][t_off((tid >> 3) + i * (kThreads / 8), unit)]) = r[i];
  };

  f32x16_t acc[2][4];  // [B operand][row subtile]
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) acc[m][mi] = f32x16_t{};

  auto mfma_step = [&](const char* abuf, const BRegs<WF>& b, bool zero_lane) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t af[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8_t*>(abuf + t_off(32 * mi + cl, half * 4 + s));
      bf16x8_t b0 = b_frag<WF>(b, 0, s);
      bf16x8_t b1 = b_frag<WF>(b, 1, s);
      if (zero_lane) {
        b0 = bf16x8_t{};
        b1 = bf16x8_t{};
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) af[mi] = bf16x8_t{};
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        acc[0][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], b0, acc[0][mi], 0, 0, 0);
        acc[1][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], b1, acc[1][mi], 0, 0, 0);
      }
    }
  };

  // ---- prologue: steps 0..D-1 in flight, step 0 into LDS
  const int klast = ns - 1;
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_a(aring[j], min(j, klast));
    load_b_step(bring[j], min(j, klast));
  }
  store_a(aring[0], 0);
  load_a(aring[0], min(D, klast));
  __syncthreads();

  // ---- main loop, unrolled by D so ring slots are static.  A last partial
  // group (ns % D != 0) only skips the MFMAs.
  for (int kk0 = 0; kk0 < ns; kk0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int kk = kk0 + j;
      if (kk < ns) mfma_step(lds_a[kk & 1], bring[j], kk == nk && half);
      load_b_step(bring[j], min(kk + D, klast));
      const int jn = (j + 1) % D;
      store_a(aring[jn], (kk + 1) & 1);
      load_a(aring[jn], min(kk + 1 + D, klast));
      __syncthreads();
    }
  }

  // ---- epilogue.  C layout of a 32x32 MFMA: lane holds column lane%32 and
  // rows 8*(i/4) + 4*(lane/32) + i%4 for i in 0..15.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * mi + 8 * (i >> 2) + 4 * half + (i & 3);
      if (row < nrows) {
        const size_t orow = (size_t)(row0 + row) * a.N;
        if (GATEUP) {
          if (col0 < a.N) {
            const float g = acc[0][mi][i];
            const float u = acc[1][mi][i];
            reinterpret_cast<uint16_t*>(a.out)[orow + col0] = f32_to_bf16(silu_mul(g, u));
          }
        } else {
          if (col0 < a.N) reinterpret_cast<float*>(a.out)[orow + col0] = acc[0][mi][i];
          if (col1 < a.N) reinterpret_cast<float*>(a.out)[orow + col1] = acc[1][mi][i];
        }
      }
    }
  }
}

// ---- bf16 weights, streamed straight into LDS.
//
// Tile of 128 rows x 256 weight rows, 8 waves in a 2 x 4 grid of 64 x 64.
// The global loads write LDS directly
// (global_load_lds_dwordx4: lane i of a wave lands 16 bytes at M0 + 16 i), so
// no register ring and no LDS store instructions are needed, and three
// 48 KB stages fit in LDS: loads run two K-steps ahead of the MFMAs.  Each
// DMA instruction fills 8 LDS rows of 128 B; lane i takes row i/8 and stores
// into slot i%8 the global 16-byte unit (i%8) ^ f(row), so the stage ends up in
// the XOR-swizzled layout of t_off.
//
// A wave waits only for its own DMAs of the stage it is about to read (the
// loads of one wave complete in issue order), then the block barrier makes
// every wave's part visible.  The compiler's workgroup fence would wait for
// all outstanding loads, including the ones two steps ahead, so the barrier is
// the bare instruction, fenced against compiler reordering only.
//
// Row sub-tiles of 32 past the m-tile's rows are skipped: a wave runs its
// MFMAs only on the sub-tiles that hold rows of the expert.
constexpr int kStages = 3;
constexpr int kStageA = BM * BK * 2;          // 16 KB
constexpr int kStageB = BN * BK * 2;          // 32 KB
constexpr int kStageBytes = kStageA + kStageB;
constexpr int kWaves = kThreads / kWave;      // 8
constexpr int kDmaA = kStageA / (kWave * 16) / kWaves;  // DMA instructions per wave per stage
constexpr int kDmaB = kStageB / (kWave * 16) / kWaves;
constexpr int kDmaPerStage = kDmaA + kDmaB;   // 6

typedef __attribute__((address_space(3))) void lds_void_t;

// AUX: cache policy of the load (0: default, 2: non-temporal).
template <int AUX>
__device__ __forceinline__ void dma16(const char* g, char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, AUX);
}
constexpr int kAuxA = 0;  // activation rows: reused by every n-tile of the m-tile
constexpr int kAuxB = 0;  // weight panel
constexpr int kAuxNT = 2; // non-temporal: a weight panel no other block reads

// Wait until at most N of this wave's vector-memory operations are
// outstanding and its LDS reads have returned, then join the block.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("" ::: "memory");
  // vmcnt(N) (bits 3:0 and 15:14), expcnt(7), lgkmcnt(0)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// MFMAs of one K-step on LDS stage `st` for the VM valid row sub-tiles
// (of two) of this wave; fragments are read one substep ahead.  A lane of
// half h feeds K units 4h + s of the step (s = substep); in a TAIL step only
// the first 32 K exist, so the half-1 lanes feed zeros.
template <int VM, bool TAIL = false>
__device__ __forceinline__ void dma_step(const char* st, const int* aoff, const int* boff,
                                         f32x16_t (&acc)[2][2], int half = 0) {
  if constexpr (VM > 0) {
    const char* abuf = st;
    const char* bbuf = st + kStageA;
    bf16x8_t af[2][2], bf[2][2];
    auto rd = [&](int s, bf16x8_t* a2, bf16x8_t* b2) {
#pragma unroll
      for (int mi = 0; mi < VM; ++mi)
        a2[mi] = *reinterpret_cast<const bf16x8_t*>(abuf + aoff[4 * mi + s]);
#pragma unroll
      for (int m = 0; m < 2; ++m) b2[m] = *reinterpret_cast<const bf16x8_t*>(bbuf + boff[4 * m + s]);
      if constexpr (TAIL) {
        if (half) {
#pragma unroll
          for (int mi = 0; mi < VM; ++mi) a2[mi] = bf16x8_t{};
#pragma unroll
          for (int m = 0; m < 2; ++m) b2[m] = bf16x8_t{};
        }
      }
    };
    rd(0, af[0], bf[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) rd(s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int mi = 0; mi < VM; ++mi)
          acc[m][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][mi], bf[s & 1][m],
                                                             acc[m][mi], 0, 0, 0);
    }
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(kThreads) void gg_dma_kernel(GGArgs a) {
  __shared__ __align__(1024) char lds[kStages * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2;  // 0..1: rows 64*wm ..
  const int wn = wave & 3;   // 0..3: columns
  const int half = lane >> 5;
  const int cl = lane & 31;

  // ---- tile (same logical order and XCD mapping as the other kernels)
  const int num_tiles = *a.num_mtiles * a.ntiles;
  const int per_xcd = (num_tiles + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int L = (blockIdx.x % kXcds) * per_xcd + slot;
  if (L >= num_tiles) return;
  const int* eq = a.mtiles + kMtileInts * (L / a.ntiles);
  const int e = eq[0];
  const int first_mt = eq[3];
  const int nmt = eq[4];
  const int local = L - first_mt * a.ntiles;
  const int ntile = local / nmt;
  const int* em = a.mtiles + kMtileInts * (first_mt + (local - ntile * nmt));
  const int row0 = em[1];
  const int nrows = em[2];
  const int nbase = ntile * (GATEUP ? BN / 2 : BN);

  // ---- DMA sources: instruction j of this wave fills LDS rows 8j.. of its
  // share; lane -> (row, slot), global unit slot ^ f(row).
  const size_t rb = (size_t)a.K * 2;
  const int slot16 = lane & 7;
  // K % 64 == 32: after the nk full steps a tail step holds 32 K; a lane
  // whose 16-byte unit lies in the missing half re-reads unit - 4 of its row
  // (in bounds; fed to the MFMAs as zeros).  The tail is loaded after the
  // main loop, which stays that of the K % 64 == 0 case.
  const int nk = a.K / BK;
  const bool ktail = (a.K % BK) != 0;
  const char* asrc[kDmaA];
  int ahi = 0, bhi = 0;  // bit j: the lane's unit of DMA j is in the upper half of the step
#pragma unroll
  for (int j = 0; j < kDmaA; ++j) {
    const int r = (kDmaA * 8) * wave + 8 * j + (lane >> 3);
    const int f = (r & 7) ^ ((r >> 3) & 1);
    const int src = row0 + min(r, nrows - 1);
    asrc[j] = reinterpret_cast<const char*>(a.a_src) +
              (GATEUP ? (size_t)(dbg_idx(a.sorted_src[src], a.T * a.k, kDbgSortedSrc) / a.k) : (size_t)src) * rb + ((slot16 ^ f) << 4);
    ahi |= ((slot16 ^ f) >= 4 ? 1 : 0) << j;
  }
  const char* bsrc[kDmaB];
#pragma unroll
  for (int j = 0; j < kDmaB; ++j) {
    const int r = (kDmaB * 8) * wave + 8 * j + (lane >> 3);
    const int f = (r & 7) ^ ((r >> 3) & 1);
    const void* w = a.w0;
    int col;
    if (GATEUP) {
      const bool up = r >= BN / 2;
      w = up ? a.w1 : a.w0;
      col = nbase + (up ? r - BN / 2 : r);
    } else {
      col = nbase + r;
    }
    col = min(col, a.N - 1);
    bsrc[j] = reinterpret_cast<const char*>(w) + ((size_t)e * a.N + col) * rb + ((slot16 ^ f) << 4);
    bhi |= ((slot16 ^ f) >= 4 ? 1 : 0) << j;
  }
  char* const adst = lds + (kDmaA * 8) * wave * (BK * 2);
  char* const bdst = lds + kStageA + (kDmaB * 8) * wave * (BK * 2);
  // Weight panels of an expert with one m-tile are read by this block alone:
  // they are fetched non-temporally (measured on this chip: the LDS DMA
  // streams at 6.8 TB/s non-temporal against 6.0 TB/s with the default
  // policy).  Panels shared by several m-tiles keep the default policy, so
  // the m-tiles find them in L2 (non-temporal there re-fetches them).
  auto issue = [&](int kk, int stage, auto nt_c) {
    constexpr int AUXB = decltype(nt_c)::value ? kAuxNT : kAuxB;
    const size_t go = (size_t)kk * (BK * 2);
    const int so = stage * kStageBytes;
#pragma unroll
    for (int j = 0; j < kDmaA; ++j) dma16<kAuxA>(asrc[j] + go, adst + so + j * 8 * (BK * 2));
#pragma unroll
    for (int j = 0; j < kDmaB; ++j) dma16<AUXB>(bsrc[j] + go, bdst + so + j * 8 * (BK * 2));
  };
  auto issue_tail = [&](int stage, auto nt_c) {
    constexpr int AUXB = decltype(nt_c)::value ? kAuxNT : kAuxB;
    const size_t go = (size_t)nk * (BK * 2);
    const int so = stage * kStageBytes;
#pragma unroll
    for (int j = 0; j < kDmaA; ++j)
      dma16<kAuxA>(asrc[j] + go - ((ahi >> j) & 1) * BK, adst + so + j * 8 * (BK * 2));
#pragma unroll
    for (int j = 0; j < kDmaB; ++j)
      dma16<AUXB>(bsrc[j] + go - ((bhi >> j) & 1) * BK, bdst + so + j * 8 * (BK * 2));
  };

  // ---- fragment offsets inside a stage: [sub-tile or matrix][substep]
  int aoff[8], boff[8];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int s = 0; s < 4; ++s) aoff[4 * mi + s] = t_off(64 * wm + 32 * mi + cl, half * 4 + s);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int br = GATEUP ? (m * (BN / 2) + 32 * wn + cl) : (64 * wn + 32 * m + cl);
#pragma unroll
    for (int s = 0; s < 4; ++s) boff[4 * m + s] = t_off(br, half * 4 + s);
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) acc[m][mi] = f32x16_t{};

  // valid 32-row sub-tiles of this wave's 64 rows (block-uniform per wave)
  const int vm = min(max((nrows + 31) / 32 - 2 * wm, 0), 2);

  // The loop is instantiated per sub-tile count (so the accumulators keep
  // fixed registers) and per weight cache policy.
  auto main_loop = [&](auto vm_c, auto nt_c) {
    constexpr int VM = decltype(vm_c)::value;
    if (nk > 0) issue(0, 0, nt_c);
    if (nk > 1) issue(1, 1, nt_c);
    int stage = 0;
    for (int kk = 0; kk < nk; ++kk) {
      if (kk + 1 < nk)
        wait_and_barrier<kDmaPerStage>();
      else
        wait_and_barrier<0>();
      if (kk + 2 < nk) issue(kk + 2, stage == 0 ? 2 : stage - 1, nt_c);
      dma_step<VM>(lds + stage * kStageBytes, aoff, boff, acc);
      stage = stage == kStages - 1 ? 0 : stage + 1;
    }
    if (ktail) {
      // stage `stage` was last read at step nk - 3, before every wave passed
      // the barrier of step nk - 2
      issue_tail(stage, nt_c);
      wait_and_barrier<0>();
      dma_step<VM, true>(lds + stage * kStageBytes, aoff, boff, acc, half);
    }
  };
  auto by_vm = [&](auto nt_c) {
    if (vm == 2)
      main_loop(std::integral_constant<int, 2>{}, nt_c);
    else if (vm == 1)
      main_loop(std::integral_constant<int, 1>{}, nt_c);
    else
      main_loop(std::integral_constant<int, 0>{}, nt_c);
  };
  if (nmt == 1)
    by_vm(std::true_type{});
  else
    by_vm(std::false_type{});

  // ---- epilogue (C layout of a 32x32 MFMA: lane holds column lane%32 and
  // rows 8*(i/4) + 4*(lane/32) + i%4 for i in 0..15)
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    if (mi < vm) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * half + (i & 3);
        if (row < nrows) {
          const size_t orow = (size_t)(row0 + row) * a.N;
          if (GATEUP) {
            const int col = nbase + 32 * wn + cl;
            if (col < a.N) {
              const float g = acc[0][mi][i];
              const float u = acc[1][mi][i];
              reinterpret_cast<uint16_t*>(a.out)[orow + col] = f32_to_bf16(silu_mul(g, u));
            }
          } else {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const int col = nbase + 64 * wn + 32 * m + cl;
              if (col < a.N) reinterpret_cast<float*>(a.out)[orow + col] = acc[m][mi][i];
            }
          }
        }
      }
    }
  }
}

// ---- 4-bit weights (MX-FP4 or NVFP4), cache-line groups of codes in LDS.
//
// A weight row's codes for one K-step are 32 bytes, a quarter of a 128-byte
// line; fetched step by step, a line is needed again three steps later, by
// which time the streaming traffic of the XCD has pushed it out of L2 and it
// is read from HBM again (counters showed about 2.5x the code bytes).  Here
// the codes travel in groups of four K-steps: each DMA instruction fills 8
// weight rows x 128 bytes (whole lines, 8 lanes per line), a group of 256
// weight rows x 4 steps is 32 KB, and three group buffers let a group be
// issued two groups ahead of its use, one instruction per wave per step.  The
// block scales of a group (MX-FP4: 8 E8M0 bytes per weight row; NVFP4: 16
// E4M3 bytes) arrive with one or two 4-byte DMAs per lane at the group's first
// step, and the NVFP4 matrix scale multiplies the accumulators in the
// epilogue (E2M1 x E4M3 is exact in bf16, and is formed in fp32: the scaled
// convert only takes powers of two).  The activation tile and the
// 2 x 4 wave grid are those of gg_dma_kernel (64 rows x two 32-column
// operands per wave, wave-local SwiGLU); codes are converted to bf16 (scale
// applied by the instruction) just before their MFMAs.
//
// Per step the loads are issued activations, then codes[, scales].  A wave's
// vector loads complete in issue order, so waiting for the activation stage
// issued two steps earlier also waits for everything issued before it; with
// the codes issued after the activations, that never includes the code group
// issued at the same step for use eight steps later (issued first, it would
// have had two steps to arrive from HBM instead of eight).  Requires
// K % 256 == 0.
constexpr int kGroupSteps = 4;
constexpr int kGroupBufs = 3;
constexpr int kCodesGroup = BN * 128;                 // 32 KB: 256 weight rows x one line
constexpr int kMx4A = 3;                              // activation stages
constexpr int kCodeDmaPerStep = kCodesGroup / (kWave * 16) / kWaves / kGroupSteps;  // 1
static_assert(kCodeDmaPerStep == 1, "one code DMA per wave per step");

// 16-byte unit u of 128-byte code row r (four K-steps of one weight row)
// lives at unit u ^ c(r), c(r) = (r >> 1) & 7: a fragment read of 8 or 16
// consecutive rows at one unit then touches distinct 16-byte bank groups (an
// even and an odd row share a 256-byte bank line).
__device__ __forceinline__ int code_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int code_off(int r, int unit) { return r * 128 + ((unit ^ code_swz(r)) << 4); }

// Scale bytes per weight row per group, and the group's scale DMAs per wave.
template <int WF>
struct GroupScales {
  static constexpr int kBytesPerRow = WF == kNVFP4 ? 16 : 8;
  static constexpr int kBytes = BN * kBytesPerRow;
  static constexpr int kDmas = kBytes / (kWaves * kWave * 4);
  static constexpr int kLds = kMx4A * kStageA + kGroupBufs * (kCodesGroup + kBytes);
  static_assert(kDmas * kWaves * kWave * 4 == kBytes, "whole scale DMAs");
};

// A lane's 4-bit operand for one K-step: its 32-element block of codes per
// matrix and the scales of the block's halves (equal for MX-FP4).
struct Fp4Regs {
  u32x4 v[2];
  float lo[2], hi[2];
};

// Two E2M1 codes (byte SEL of w) times an NVFP4 block scale, as a packed bf16
// pair.  The gfx950 scaled convert applies only the exponent of its fp32
// scale (checked on the device: scale 1.5 multiplies by 1), which suits the
// E8M0 scales of MX-FP4 but not E4M3, so the product is formed in fp32.  It
// has at most 6 significant bits (E2M1: 2, E4M3: 4), so the upper half of its
// fp32 bits is the exact bf16 value.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_times(uint32_t w, float sc) {
  auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  const uint32_t lo = __float_as_uint(f[0] * sc);
  const uint32_t hi = __float_as_uint(f[1] * sc);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // {hi[31:16], lo[31:16]}
}

// bf16 fragment for substep s of matrix m: code word s holds elements
// 8s..8s+7, so words 0 and 1 take the first half's scale.
template <int WF>
__device__ __forceinline__ bf16x8_t fp4_frag(const Fp4Regs& b, int m, int s) {
  const uint32_t w = b.v[m][s];
  const float sc = s < 2 ? b.lo[m] : b.hi[m];
  u32x4 r;
  if constexpr (WF == kNVFP4) {
    r.x = fp4x2_times<0>(w, sc);
    r.y = fp4x2_times<1>(w, sc);
    r.z = fp4x2_times<2>(w, sc);
    r.w = fp4x2_times<3>(w, sc);
  } else {  // E8M0: a power of two, applied by the instruction
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  }
  return __builtin_bit_cast(bf16x8_t, r);
}

// MFMAs of one K-step for the VM valid row sub-tiles of this wave.  `cb` and
// `sb` are the group's code and scale buffers, p the step's place in it.
template <int WF, int VM>
__device__ __forceinline__ void mx4_step(const char* st, const char* cb, const char* sb, int p,
                                         const int* aoff, const int* brow, int half,
                                         f32x16_t (&acc)[2][2]) {
  if constexpr (VM > 0) {
    Fp4Regs b;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int u = 2 * p + half;  // the lane's 32-element block inside the line
      b.v[m] = *reinterpret_cast<const u32x4*>(cb + code_off(brow[m], u));
      if constexpr (WF == kNVFP4) {
        const uint8_t* q = reinterpret_cast<const uint8_t*>(sb) + brow[m] * 16 + 2 * u;
        b.lo[m] = e4m3_to_f32(q[0]);
        b.hi[m] = e4m3_to_f32(q[1]);
      } else {
        b.lo[m] = b.hi[m] = e8m0_cvt_scale(static_cast<uint8_t>(sb[brow[m] * 8 + u]));
      }
    }
    bf16x8_t af[2][2];
#pragma unroll
    for (int mi = 0; mi < VM; ++mi) af[0][mi] = *reinterpret_cast<const bf16x8_t*>(st + aoff[4 * mi]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) {
#pragma unroll
        for (int mi = 0; mi < VM; ++mi)
          af[(s + 1) & 1][mi] = *reinterpret_cast<const bf16x8_t*>(st + aoff[4 * mi + s + 1]);
      }
      const bf16x8_t b0 = fp4_frag<WF>(b, 0, s);
      const bf16x8_t b1 = fp4_frag<WF>(b, 1, s);
#pragma unroll
      for (int mi = 0; mi < VM; ++mi) {
        acc[0][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][mi], b0, acc[0][mi], 0, 0, 0);
        acc[1][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][mi], b1, acc[1][mi], 0, 0, 0);
      }
    }
  }
}

template <int WF, bool GATEUP>
__global__ __launch_bounds__(kThreads) void gg_mx_group_kernel(GGArgs a) {
  using GS = GroupScales<WF>;
  __shared__ __align__(1024) char lds[GS::kLds];
  char* const lds_a = lds;
  char* const lds_c = lds + kMx4A * kStageA;
  char* const lds_s = lds_c + kGroupBufs * kCodesGroup;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2;
  const int wn = wave & 3;
  const int half = lane >> 5;
  const int cl = lane & 31;

  // ---- tile (as in the other kernels)
  const int num_tiles = *a.num_mtiles * a.ntiles;
  const int per_xcd = (num_tiles + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int L = (blockIdx.x % kXcds) * per_xcd + slot;
  if (L >= num_tiles) return;
  const int* eq = a.mtiles + kMtileInts * (L / a.ntiles);
  const int e = eq[0];
  const int first_mt = eq[3];
  const int local = L - first_mt * a.ntiles;
  // m-tile by m-tile within the expert: the n-tiles of one m-tile run
  // back to back, so its activation rows stay in L2 (the packed weights
  // are small enough that their re-reads cost less here)
  const int mloc = local / a.ntiles;
  const int ntile = local - mloc * a.ntiles;
  const int* em = a.mtiles + kMtileInts * (first_mt + mloc);
  const int row0 = em[1];
  const int nrows = em[2];
  const int nbase = ntile * (GATEUP ? BN / 2 : BN);

  // weight row r of the tile (0..255) -> its codes and scales
  auto wrow = [&](int r, const char*& code, const uint8_t*& scale) {
    const void* w = a.w0;
    const uint8_t* sc = a.s0;
    int col;
    if (GATEUP) {
      const bool up = r >= BN / 2;
      w = up ? a.w1 : a.w0;
      sc = up ? a.s1 : a.s0;
      col = nbase + (up ? r - BN / 2 : r);
    } else {
      col = nbase + r;
    }
    col = min(col, a.N - 1);
    code = reinterpret_cast<const char*>(w) + ((size_t)e * a.N + col) * (a.K / 2);
    scale = sc + ((size_t)e * a.N + col) * ((size_t)a.K / 256 * GS::kBytesPerRow);
  };

  // ---- activation DMA sources (see gg_dma_kernel)
  const size_t rb = (size_t)a.K * 2;
  const int slot16 = lane & 7;
  const char* asrc[kDmaA];
#pragma unroll
  for (int j = 0; j < kDmaA; ++j) {
    const int r = (kDmaA * 8) * wave + 8 * j + (lane >> 3);
    const int f = (r & 7) ^ ((r >> 3) & 1);
    const int src = row0 + min(r, nrows - 1);
    asrc[j] = reinterpret_cast<const char*>(a.a_src) +
              (GATEUP ? (size_t)(dbg_idx(a.sorted_src[src], a.T * a.k, kDbgSortedSrc) / a.k) : (size_t)src) * rb + ((slot16 ^ f) << 4);
  }
  char* const adst = lds_a + (kDmaA * 8) * wave * (BK * 2);

  // ---- code DMA sources: at group place p, wave w fills weight rows
  // 32 w + 8 p + lane/8, line slot lane%8 <- global unit (lane%8) ^ code_swz(row)
  const char* csrc[kGroupSteps];
#pragma unroll
  for (int p = 0; p < kGroupSteps; ++p) {
    const int r = 32 * wave + 8 * p + (lane >> 3);
    const char* code;
    const uint8_t* scale;
    wrow(r, code, scale);
    csrc[p] = code + ((slot16 ^ code_swz(r)) << 4);
  }
  // ---- scale DMA sources: dword d = 64 (kDmas w + i) + lane of the group
  // covers weight row d / W, bytes 4 (d % W) .. +3 of the row's group bytes
  // (W = words per row)
  constexpr int W = GS::kBytesPerRow / 4;
  const uint8_t* ssrc[GS::kDmas];
#pragma unroll
  for (int i = 0; i < GS::kDmas; ++i) {
    const int d = kWave * (GS::kDmas * wave + i) + lane;
    const char* code;
    wrow(d / W, code, ssrc[i]);
    ssrc[i] += 4 * (d % W);
  }
  const int nk = a.K / BK;
  const int ng = nk / kGroupSteps;

  // Loads for group g / step kk go to that group's / step's buffer; past the
  // end they re-read the last group or step, still into the buffer that is
  // free at that point.
  auto issue_codes = [&](int g, int p) {  // part p of group g
    char* d = lds_c + (g % kGroupBufs) * kCodesGroup + (32 * wave + 8 * p) * 128;
    dma16<0>(csrc[p] + (size_t)min(g, ng - 1) * 128, d);
  };
  auto issue_scales = [&](int g) {
    char* d = lds_s + (g % kGroupBufs) * GS::kBytes + GS::kDmas * wave * kWave * 4;
    const size_t go = (size_t)min(g, ng - 1) * GS::kBytesPerRow;
#pragma unroll
    for (int i = 0; i < GS::kDmas; ++i)
      __builtin_amdgcn_global_load_lds(ssrc[i] + go, (lds_void_t*)(d + i * kWave * 4), 4, 0, 0);
  };
  auto issue_a = [&](int kk) {
    char* d = adst + (kk % kMx4A) * kStageA;
    const size_t go = (size_t)min(kk, nk - 1) * (BK * 2);
#pragma unroll
    for (int j = 0; j < kDmaA; ++j) dma16<kAuxA>(asrc[j] + go, d + j * 8 * (BK * 2));
  };

  // ---- fragment offsets
  int aoff[8], brow[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int s = 0; s < 4; ++s) aoff[4 * mi + s] = t_off(64 * wm + 32 * mi + cl, half * 4 + s);
#pragma unroll
  for (int m = 0; m < 2; ++m) brow[m] = GATEUP ? (m * (BN / 2) + 32 * wn + cl) : (64 * wn + 32 * m + cl);

  f32x16_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) acc[m][mi] = f32x16_t{};

  const int vm = min(max((nrows + 31) / 32 - 2 * wm, 0), 2);

  // ---- prologue: groups 0 and 1, then activation steps 0 and 1 (youngest)
#pragma unroll
  for (int g = 0; g < 2; ++g) {
#pragma unroll
    for (int p = 0; p < kGroupSteps; ++p) issue_codes(g, p);
    issue_scales(g);
  }
  asm volatile("" ::: "memory");  // activation DMAs are the youngest loads
  issue_a(0);
  issue_a(1);

  // Groups run three to a loop turn, so group g's buffer (g % 3) and step
  // kk's activation stage (kk % 3 = (g + p) % 3, as 4 = 1 mod 3) are
  // compile-time: every LDS fragment address is then a loop-invariant register
  // plus an immediate offset, instead of two adds per fragment per step.
  auto main_loop = [&](auto vm_c) {
    constexpr int VM = decltype(vm_c)::value;
    auto group = [&](int g, auto j_c) {
      constexpr int J = decltype(j_c)::value;  // g % 3
      const char* cb = lds_c + J * kCodesGroup;
      const char* sb = lds_s + J * GS::kBytes;
      auto step = [&](auto p_c) {
        constexpr int p = decltype(p_c)::value;
        const int kk = kGroupSteps * g + p;
        // Younger than activation stage kk (issued first at step kk-2): the
        // code DMA (and at a group's first place the scale DMAs) issued after
        // it at step kk-2, then every load of step kk-1.  In group 0 the
        // prologue stands in for steps -2 and -1: only stage 1 (two DMAs),
        // then step 0's loads.
        constexpr int S = GS::kDmas;
        if constexpr (p == 0) {
          if (g == 0)
            wait_and_barrier<2>();
          else
            wait_and_barrier<4>();
        } else if constexpr (p == 1) {
          if (g == 0)
            wait_and_barrier<3 + S>();
          else
            wait_and_barrier<4 + S>();
        } else if constexpr (p == 2) {
          wait_and_barrier<4 + S>();
        } else {
          wait_and_barrier<4>();
        }
        issue_a(kk + 2);
        asm volatile("" ::: "memory");  // codes and scales after the step's activations
        issue_codes(g + 2, p);
        if constexpr (p == 0) issue_scales(g + 2);
        mx4_step<WF, VM>(lds_a + ((J + p) % kMx4A) * kStageA, cb, sb, p, aoff, brow, half, acc);
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
      step(std::integral_constant<int, 3>{});
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    int g = 0;
    for (; g + 3 <= ng; g += 3) {
      group(g, I0{});
      group(g + 1, I1{});
      group(g + 2, I2{});
    }
    if (g < ng) group(g, I0{});
    if (g + 1 < ng) group(g + 1, I1{});
  };
  if (vm == 2)
    main_loop(std::integral_constant<int, 2>{});
  else if (vm == 1)
    main_loop(std::integral_constant<int, 1>{});
  else
    main_loop(std::integral_constant<int, 0>{});
  // the clamped loads past the end must land before the block's LDS is released
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue (as gg_dma_kernel, after the NVFP4 matrix scales)
  if constexpr (WF == kNVFP4) {
    const float t0 = a.t0[e];
    const float t1 = GATEUP ? a.t1[e] : t0;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      acc[0][mi] *= t0;
      acc[1][mi] *= t1;
    }
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    if (mi < vm) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * half + (i & 3);
        if (row < nrows) {
          const size_t orow = (size_t)(row0 + row) * a.N;
          if (GATEUP) {
            const int col = nbase + 32 * wn + cl;
            if (col < a.N) {
              const float g = acc[0][mi][i];
              const float u = acc[1][mi][i];
              reinterpret_cast<uint16_t*>(a.out)[orow + col] = f32_to_bf16(silu_mul(g, u));
            }
          } else {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const int col = nbase + 64 * wn + 32 * m + cl;
              if (col < a.N) reinterpret_cast<float*>(a.out)[orow + col] = acc[m][mi][i];
            }
          }
        }
      }
    }
  }
}

// MFMAs of one K-step for a wave owning all VM valid row sub-tiles and one
// 32-column weight operand (gg_mx_row_kernel): the operand is converted once
// per substep and feeds VM MFMAs.
template <int WF, int VM>
__device__ __forceinline__ void mx4_row_step(const char* st, const char* cb, const char* sb, int p,
                                             const int* aoff, int brow, int half, f32x16_t (&acc)[4]) {
  Fp4Regs b;
  const int u = 2 * p + half;  // the lane's 32-element block inside the line
  b.v[0] = *reinterpret_cast<const u32x4*>(cb + code_off(brow, u));
  if constexpr (WF == kNVFP4) {
    const uint8_t* q = reinterpret_cast<const uint8_t*>(sb) + brow * 16 + 2 * u;
    b.lo[0] = e4m3_to_f32(q[0]);
    b.hi[0] = e4m3_to_f32(q[1]);
  } else {
    b.lo[0] = b.hi[0] = e8m0_cvt_scale(static_cast<uint8_t>(sb[brow * 8 + u]));
  }
  bf16x8_t af[2][VM];
#pragma unroll
  for (int mi = 0; mi < VM; ++mi) af[0][mi] = *reinterpret_cast<const bf16x8_t*>(st + aoff[4 * mi]);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s + 1 < 4) {
#pragma unroll
      for (int mi = 0; mi < VM; ++mi)
        af[(s + 1) & 1][mi] = *reinterpret_cast<const bf16x8_t*>(st + aoff[4 * mi + s + 1]);
    }
    const bf16x8_t bb = fp4_frag<WF>(b, 0, s);
#pragma unroll
    for (int mi = 0; mi < VM; ++mi)
      acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][mi], bb, acc[mi], 0, 0, 0);
  }
}

// gg_mx_group_kernel with the eight waves side by side (1 x 8): each wave
// owns all 128 rows of the tile and 32 of its 256 weight rows.  Every wave
// then works on every tile whatever its fill (with the 2 x 4 grid the lower
// half of the waves idles on tiles of up to 64 rows, leaving one working wave
// per SIMD), and each weight operand is converted once instead of by two
// waves; the activation fragments are read from LDS twice as often.  Loads,
// waits and LDS layout are gg_mx_group_kernel's.  Used for NVFP4, whose
// conversion (E2M1 x E4M3 formed in fp32) costs four instructions per code
// pair: prefill 5.88 -> 5.34 ms.  For MX-FP4 (one convert per pair) the extra
// activation reads cost more than the halved conversions save (gate/up 2.65
// -> 2.84 ms), so it keeps the 2 x 4 grid.
// QH (gate/up only): h is rounded to the MXFP8 grid before it is stored (as
// bf16), for FP8 activations with NVFP4 weights.  A wave holds 16 output
// columns, so each 32-column MX block spans waves 2j and 2j + 1: their
// per-row partial maxima meet in LDS after the main loop.
template <int WF, bool GATEUP, bool QH = false>
__global__ __launch_bounds__(kThreads) void gg_mx_row_kernel(GGArgs a) {
  using GS = GroupScales<WF>;
  __shared__ __align__(1024) char lds[GS::kLds];
  char* const lds_a = lds;
  char* const lds_c = lds + kMx4A * kStageA;
  char* const lds_s = lds_c + kGroupBufs * kCodesGroup;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int cl = lane & 31;

  // ---- tile (as in the other kernels)
  const int num_tiles = *a.num_mtiles * a.ntiles;
  const int per_xcd = (num_tiles + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int L = (blockIdx.x % kXcds) * per_xcd + slot;
  if (L >= num_tiles) return;
  const int* eq = a.mtiles + kMtileInts * (L / a.ntiles);
  const int e = eq[0];
  const int first_mt = eq[3];
  const int nmt = eq[4];
  const int local = L - first_mt * a.ntiles;
  const int ntile = local / nmt;
  const int* em = a.mtiles + kMtileInts * (first_mt + (local - ntile * nmt));
  const int row0 = em[1];
  const int nrows = em[2];
  const int nbase = ntile * (GATEUP ? BN / 2 : BN);

  // weight row r of the tile (0..255) -> its codes and scales
  auto wrow = [&](int r, const char*& code, const uint8_t*& scale) {
    const void* w = a.w0;
    const uint8_t* sc = a.s0;
    int col;
    if (GATEUP) {
      const bool up = r >= BN / 2;
      w = up ? a.w1 : a.w0;
      sc = up ? a.s1 : a.s0;
      col = nbase + (up ? r - BN / 2 : r);
    } else {
      col = nbase + r;
    }
    col = min(col, a.N - 1);
    code = reinterpret_cast<const char*>(w) + ((size_t)e * a.N + col) * (a.K / 2);
    scale = sc + ((size_t)e * a.N + col) * ((size_t)a.K / 256 * GS::kBytesPerRow);
  };

  // ---- activation DMA sources (see gg_dma_kernel)
  const size_t rb = (size_t)a.K * 2;
  const int slot16 = lane & 7;
  const char* asrc[kDmaA];
#pragma unroll
  for (int j = 0; j < kDmaA; ++j) {
    const int r = (kDmaA * 8) * wave + 8 * j + (lane >> 3);
    const int f = (r & 7) ^ ((r >> 3) & 1);
    const int src = row0 + min(r, nrows - 1);
    asrc[j] = reinterpret_cast<const char*>(a.a_src) +
              (GATEUP ? (size_t)(dbg_idx(a.sorted_src[src], a.T * a.k, kDbgSortedSrc) / a.k) : (size_t)src) * rb + ((slot16 ^ f) << 4);
  }
  char* const adst = lds_a + (kDmaA * 8) * wave * (BK * 2);

  // ---- code DMA sources: at group place p, wave w fills weight rows
  // 32 w + 8 p + lane/8, line slot lane%8 <- global unit (lane%8) ^ code_swz(row)
  const char* csrc[kGroupSteps];
#pragma unroll
  for (int p = 0; p < kGroupSteps; ++p) {
    const int r = 32 * wave + 8 * p + (lane >> 3);
    const char* code;
    const uint8_t* scale;
    wrow(r, code, scale);
    csrc[p] = code + ((slot16 ^ code_swz(r)) << 4);
  }
  // ---- scale DMA sources: dword d = 64 (kDmas w + i) + lane of the group
  // covers weight row d / W, bytes 4 (d % W) .. +3 of the row's group bytes
  // (W = words per row)
  constexpr int W = GS::kBytesPerRow / 4;
  const uint8_t* ssrc[GS::kDmas];
#pragma unroll
  for (int i = 0; i < GS::kDmas; ++i) {
    const int d = kWave * (GS::kDmas * wave + i) + lane;
    const char* code;
    wrow(d / W, code, ssrc[i]);
    ssrc[i] += 4 * (d % W);
  }
  const int nk = a.K / BK;
  const int ng = nk / kGroupSteps;

  // Loads for group g / step kk go to that group's / step's buffer; past the
  // end they re-read the last group or step, still into the buffer that is
  // free at that point.
  auto issue_codes = [&](int g, int p) {  // part p of group g
    char* d = lds_c + (g % kGroupBufs) * kCodesGroup + (32 * wave + 8 * p) * 128;
    dma16<0>(csrc[p] + (size_t)min(g, ng - 1) * 128, d);
  };
  auto issue_scales = [&](int g) {
    char* d = lds_s + (g % kGroupBufs) * GS::kBytes + GS::kDmas * wave * kWave * 4;
    const size_t go = (size_t)min(g, ng - 1) * GS::kBytesPerRow;
#pragma unroll
    for (int i = 0; i < GS::kDmas; ++i)
      __builtin_amdgcn_global_load_lds(ssrc[i] + go, (lds_void_t*)(d + i * kWave * 4), 4, 0, 0);
  };
  auto issue_a = [&](int kk) {
    char* d = adst + (kk % kMx4A) * kStageA;
    const size_t go = (size_t)min(kk, nk - 1) * (BK * 2);
#pragma unroll
    for (int j = 0; j < kDmaA; ++j) dma16<kAuxA>(asrc[j] + go, d + j * 8 * (BK * 2));
  };

  // ---- fragment offsets: all four 32-row sub-tiles, one 32-column weight
  // operand (gate/up: 16 columns of W_gate and the same 16 of W_up)
  int aoff[16];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int s = 0; s < 4; ++s) aoff[4 * mi + s] = t_off(32 * mi + cl, half * 4 + s);
  const int brow = GATEUP ? (cl < 16 ? 16 * wave + cl : BN / 2 + 16 * wave + (cl - 16)) : 32 * wave + cl;

  f32x16_t acc[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) acc[mi] = f32x16_t{};

  const int vm = min((nrows + 31) / 32, 4);

  // ---- prologue: groups 0 and 1, then activation steps 0 and 1 (youngest)
#pragma unroll
  for (int g = 0; g < 2; ++g) {
#pragma unroll
    for (int p = 0; p < kGroupSteps; ++p) issue_codes(g, p);
    issue_scales(g);
  }
  asm volatile("" ::: "memory");  // activation DMAs are the youngest loads
  issue_a(0);
  issue_a(1);

  // Groups run three to a loop turn, so group g's buffer (g % 3) and step
  // kk's activation stage (kk % 3 = (g + p) % 3, as 4 = 1 mod 3) are
  // compile-time: every LDS fragment address is then a loop-invariant register
  // plus an immediate offset, instead of two adds per fragment per step.
  auto main_loop = [&](auto vm_c) {
    constexpr int VM = decltype(vm_c)::value;
    auto group = [&](int g, auto j_c) {
      constexpr int J = decltype(j_c)::value;  // g % 3
      const char* cb = lds_c + J * kCodesGroup;
      const char* sb = lds_s + J * GS::kBytes;
      auto step = [&](auto p_c) {
        constexpr int p = decltype(p_c)::value;
        const int kk = kGroupSteps * g + p;
        // Younger than activation stage kk (issued first at step kk-2): the
        // code DMA (and at a group's first place the scale DMAs) issued after
        // it at step kk-2, then every load of step kk-1.  In group 0 the
        // prologue stands in for steps -2 and -1: only stage 1 (two DMAs),
        // then step 0's loads.
        constexpr int S = GS::kDmas;
        if constexpr (p == 0) {
          if (g == 0)
            wait_and_barrier<2>();
          else
            wait_and_barrier<4>();
        } else if constexpr (p == 1) {
          if (g == 0)
            wait_and_barrier<3 + S>();
          else
            wait_and_barrier<4 + S>();
        } else if constexpr (p == 2) {
          wait_and_barrier<4 + S>();
        } else {
          wait_and_barrier<4>();
        }
        issue_a(kk + 2);
        asm volatile("" ::: "memory");  // codes and scales after the step's activations
        issue_codes(g + 2, p);
        if constexpr (p == 0) issue_scales(g + 2);
        mx4_row_step<WF, VM>(lds_a + ((J + p) % kMx4A) * kStageA, cb, sb, p, aoff, brow, half, acc);
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
      step(std::integral_constant<int, 3>{});
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    int g = 0;
    for (; g + 3 <= ng; g += 3) {
      group(g, I0{});
      group(g + 1, I1{});
      group(g + 2, I2{});
    }
    if (g < ng) group(g, I0{});
    if (g + 1 < ng) group(g + 1, I1{});
  };
  if (vm == 4)
    main_loop(std::integral_constant<int, 4>{});
  else if (vm == 3)
    main_loop(std::integral_constant<int, 3>{});
  else if (vm == 2)
    main_loop(std::integral_constant<int, 2>{});
  else
    main_loop(std::integral_constant<int, 1>{});
  // the clamped loads past the end must land before the block's LDS is released
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue (C layout of a 32x32 MFMA: lane holds column lane%32 and
  // rows 8*(i/4) + 4*(lane/32) + i%4).  Gate/up: lanes with column < 16 hold
  // W_gate, the lane 16 above holds W_up of the same output column.
  if constexpr (WF == kNVFP4) {
    const float t = (GATEUP && cl >= 16) ? a.t1[e] : a.t0[e];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) acc[mi] *= t;
  }
  if constexpr (GATEUP && QH) {
    // h in place of the W_gate sums (lanes cl < 16; the others hold W_up's),
    // then each row's maximum over the wave's 16 columns: one value per row
    // per wave into LDS, which every wave has finished reading
    __syncthreads();
    float* part = reinterpret_cast<float*>(lds);  // [8 waves][128 rows]
    // sub-tiles past the tile's rows hold nothing to store (vm is the same
    // in both waves of a pair)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi >= vm) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float v = acc[mi][i];
        const float u = __shfl_xor(v, 16, kWave);  // every lane takes part
        const float h = silu_mul(v, u);
        acc[mi][i] = h;
        float am = cl < 16 ? fabsf(h) : 0.f;  // fmaxf below skips NaN
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, kWave));
        const int row = 32 * mi + 8 * (i >> 2) + 4 * half + (i & 3);
        if (cl == 0) part[wave * BM + row] = am;
      }
    }
    __syncthreads();
    const int col = nbase + 16 * wave + cl;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi >= vm) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * mi + 8 * (i >> 2) + 4 * half + (i & 3);
        const float amax = fmaxf(part[wave * BM + row], part[(wave ^ 1) * BM + row]);
        const float hq = mxfp8_round(acc[mi][i], amax);
        if (cl < 16 && row < nrows && col < a.N)
          reinterpret_cast<uint16_t*>(a.out)[(size_t)(row0 + row) * a.N + col] = f32_to_bf16(hq);
      }
    }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if (mi < vm) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 32 * mi + 8 * (i >> 2) + 4 * half + (i & 3);
        const float v = acc[mi][i];
        if (GATEUP) {
          const float u = __shfl_xor(v, 16, kWave);  // every lane takes part
          const int col = nbase + 16 * wave + cl;
          if (cl < 16 && row < nrows && col < a.N)
            reinterpret_cast<uint16_t*>(a.out)[(size_t)(row0 + row) * a.N + col] =
                f32_to_bf16(silu_mul(v, u));
        } else {
          const int col = nbase + 32 * wave + cl;
          if (row < nrows && col < a.N) reinterpret_cast<float*>(a.out)[(size_t)(row0 + row) * a.N + col] = v;
        }
      }
    }
  }
}

// ---- FP8 activations x MX-FP4 weights on the scaled MFMA.
//
// The pages run the experts with FP8 compute and 4-bit weights
// (SGLang-TorchTPU on TPU v7 page, "Results").  Here the activation operand
// (x for gate/up, h for down) is MXFP8, E4M3 values with one E8M0 scale per
// 32 elements, and the weights MX-FP4; v_mfma_scale_f32_32x32x64_f8f6f4 takes
// both with their block scales, so no code is converted in registers and one
// instruction covers K = 64.  Operand layout of that instruction, checked on
// the device: a weight lane (column c = lane % 32, half h = lane / 32) holds
// the 32 codes of K-block h, low nibble first, and supplies that block's scale;
// an activation lane (row lane % 32, half h) holds K [16h, 16h+16) and
// [32+16h, 32+16h+16) and supplies the scale of K-block h of its row.
//
// Tile, wave grid, code groups, weight scales and tile order are those of
// gg_mx_group_kernel.  The activation stage is 128 rows x 64 fp8 bytes (one
// DMA instruction per wave, 16 rows of 4 units), small enough for five
// stages: activations are issued four steps ahead of use (the bf16 ones of
// gg_mx_group_kernel two), which measured 8 % faster than two.  The
// activation scales of a group (8 bytes per row) come with one 32-lane
// 4-byte DMA per wave at the group's first step.  The gate/up epilogue writes h as MXFP8: each wave's 32
// columns are one block, whose maximum it takes across the 32 lanes of a half.
constexpr int kF8D = 4;                                   // activation steps in flight
constexpr int kF8A = kF8D + 1;                            // activation stages
constexpr int kStageA8 = BM * 64;                         // 8 KB
constexpr int kAScalesGroup = BM * 8;                     // 1 KB
constexpr int kF8Lds = kF8A * kStageA8 + kGroupBufs * (kCodesGroup + BN * 8 + kAScalesGroup);

// 16-byte unit u of 64-byte activation row r lives at unit u ^ g8(r): a
// fragment read (16 consecutive rows, one unit) then touches distinct bank
// groups in 8- and 16-lane groups (checked on the CPU).
__device__ __forceinline__ int a8_off(int row, int unit) {
  const int g = ((row >> 2) & 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 1);
  return row * 64 + ((unit ^ g) << 4);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int VM>
__device__ __forceinline__ void f8_step(const char* st, const char* cb, const char* sb, const char* ab,
                                        int p, const int* arow, const int* brow, int half,
                                        f32x16_t (&acc)[2][2]) {
  if constexpr (VM > 0) {
    i32x8_t bv[2];
    int bs[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int u = 2 * p + half;  // the lane's 32-element block inside the line
      const u32x4 c = *reinterpret_cast<const u32x4*>(cb + code_off(brow[m], u));
      bv[m] = i32x8_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
      bs[m] = static_cast<uint8_t>(sb[brow[m] * 8 + u]);
    }
#pragma unroll
    for (int mi = 0; mi < VM; ++mi) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(st + a8_off(arow[mi], half));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(st + a8_off(arow[mi], 2 + half));
      const i32x8_t av{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int as = static_cast<uint8_t>(ab[arow[mi] * 8 + 2 * p + half]);
#pragma unroll
      for (int m = 0; m < 2; ++m)
        acc[m][mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv[m], acc[m][mi], 0, 4, 0, as,
                                                                     0, bs[m]);
    }
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(kThreads) void gg_f8f4_kernel(GGArgs a) {
  __shared__ __align__(1024) char lds[kF8Lds];
  char* const lds_a = lds;
  char* const lds_c = lds + kF8A * kStageA8;
  char* const lds_s = lds_c + kGroupBufs * kCodesGroup;
  char* const lds_as = lds_s + kGroupBufs * BN * 8;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2;
  const int wn = wave & 3;
  const int half = lane >> 5;
  const int cl = lane & 31;

  // ---- tile (as in the other kernels)
  const int num_tiles = *a.num_mtiles * a.ntiles;
  const int per_xcd = (num_tiles + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  if (slot >= per_xcd) return;
  const int L = (blockIdx.x % kXcds) * per_xcd + slot;
  if (L >= num_tiles) return;
  const int* eq = a.mtiles + kMtileInts * (L / a.ntiles);
  const int e = eq[0];
  const int first_mt = eq[3];
  const int local = L - first_mt * a.ntiles;
  // m-tile by m-tile within the expert: the n-tiles of one m-tile run
  // back to back, so its activation rows stay in L2 (the packed weights
  // are small enough that their re-reads cost less here)
  const int mloc = local / a.ntiles;
  const int ntile = local - mloc * a.ntiles;
  const int* em = a.mtiles + kMtileInts * (first_mt + mloc);
  const int row0 = em[1];
  const int nrows = em[2];
  const int nbase = ntile * (GATEUP ? BN / 2 : BN);
  const int nk = a.K / BK;
  const int ng = nk / kGroupSteps;

  // weight row r of the tile (0..255) -> its codes and scales
  auto wrow = [&](int r, const char*& code, const uint8_t*& scale) {
    const void* w = a.w0;
    const uint8_t* sc = a.s0;
    int col;
    if (GATEUP) {
      const bool up = r >= BN / 2;
      w = up ? a.w1 : a.w0;
      sc = up ? a.s1 : a.s0;
      col = nbase + (up ? r - BN / 2 : r);
    } else {
      col = nbase + r;
    }
    col = min(col, a.N - 1);
    code = reinterpret_cast<const char*>(w) + ((size_t)e * a.N + col) * (a.K / 2);
    scale = sc + ((size_t)e * a.N + col) * (a.K / 32);
  };
  // activation row r of the tile (0..127) -> source row index
  auto arow_src = [&](int r) -> size_t {
    const int src = row0 + min(r, nrows - 1);
    return GATEUP ? (size_t)(dbg_idx(a.sorted_src[src], a.T * a.k, kDbgSortedSrc) / a.k) : (size_t)src;
  };

  // ---- activation DMA: wave w fills rows 16w .. 16w+15; lane -> row
  // 16w + lane/4, slot lane%4 <- global unit slot ^ g8(row)
  const char* asrc;
  {
    const int r = 16 * wave + (lane >> 2);
    const int g = ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
    asrc = reinterpret_cast<const char*>(a.a_src) + arow_src(r) * (size_t)a.K + (((lane & 3) ^ g) << 4);
  }
  char* const adst = lds_a + 16 * wave * 64;
  // ---- activation scale DMA: lanes 0..31 of wave w fill rows 16w + lane/2,
  // word lane%2 of the row's 8 group bytes
  const uint8_t* assrc = a.a_scale + arow_src(16 * wave + ((lane & 31) >> 1)) * (size_t)(a.K / 32) +
                         4 * (lane & 1);
  // ---- code and weight-scale DMA sources (as gg_mx_group_kernel)
  const int slot16 = lane & 7;
  const char* csrc[kGroupSteps];
#pragma unroll
  for (int p = 0; p < kGroupSteps; ++p) {
    const int r = 32 * wave + 8 * p + (lane >> 3);
    const char* code;
    const uint8_t* scale;
    wrow(r, code, scale);
    csrc[p] = code + ((slot16 ^ code_swz(r)) << 4);
  }
  const uint8_t* ssrc;
  {
    const int d = kWave * wave + lane;
    const char* code;
    wrow(d >> 1, code, ssrc);
    ssrc += 4 * (d & 1);
  }

  auto issue_codes = [&](int g, int p) {
    char* d = lds_c + (g % kGroupBufs) * kCodesGroup + (32 * wave + 8 * p) * 128;
    dma16<0>(csrc[p] + (size_t)min(g, ng - 1) * 128, d);
  };
  auto issue_scales = [&](int g) {  // weight and activation scales of group g
    const int gs = min(g, ng - 1);
    char* d = lds_s + (g % kGroupBufs) * (BN * 8) + wave * kWave * 4;
    __builtin_amdgcn_global_load_lds(ssrc + (size_t)gs * 8, (lds_void_t*)d, 4, 0, 0);
    char* da = lds_as + (g % kGroupBufs) * kAScalesGroup + 16 * wave * 8;
    if (lane < 32) __builtin_amdgcn_global_load_lds(assrc + (size_t)gs * 8, (lds_void_t*)da, 4, 0, 0);
  };
  auto issue_a = [&](int kk) {
    dma16<kAuxA>(asrc + (size_t)min(kk, nk - 1) * 64, adst + (kk % kF8A) * kStageA8);
  };

  int arow[2], brow[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) arow[mi] = 64 * wm + 32 * mi + cl;
#pragma unroll
  for (int m = 0; m < 2; ++m) brow[m] = GATEUP ? (m * (BN / 2) + 32 * wn + cl) : (64 * wn + 32 * m + cl);

  f32x16_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) acc[m][mi] = f32x16_t{};

  const int vm = min(max((nrows + 31) / 32 - 2 * wm, 0), 2);

  // ---- prologue: groups 0 and 1, then activation steps 0 .. kF8D-1 (youngest)
#pragma unroll
  for (int g = 0; g < 2; ++g) {
#pragma unroll
    for (int p = 0; p < kGroupSteps; ++p) issue_codes(g, p);
    issue_scales(g);
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int kk = 0; kk < kF8D; ++kk) issue_a(kk);

  // Loads per step: the activation DMA for step kk + kF8D first, then one
  // code DMA and, at a group's first step, the weight- and activation-scale
  // DMAs.  Younger than activation stage kk (issued first at step kk-4) are
  // the code and scale DMAs after it at step kk-4 and every load of steps
  // kk-3 .. kk-1 (two each, four at a group's first step): 9 at every step
  // (the four places of a group hold one four-load step between them).  In
  // group 0 the prologue's younger activation stages stand in for the steps
  // before 0: 3, 6, 7, 8.  A code group, needed eight steps after its first
  // DMA, is thereby never waited for early.
  static_assert(kF8D == 4 && kGroupSteps == 4, "wait counts below");
  auto main_loop = [&](auto vm_c) {
    constexpr int VM = decltype(vm_c)::value;
    auto group = [&](int g, auto n0, auto n1, auto n2, auto n3) {
      const char* cb = lds_c + (g % kGroupBufs) * kCodesGroup;
      const char* sb = lds_s + (g % kGroupBufs) * (BN * 8);
      const char* ab = lds_as + (g % kGroupBufs) * kAScalesGroup;
      auto step = [&](auto p_c, auto n_c) {
        constexpr int p = decltype(p_c)::value;
        const int kk = kGroupSteps * g + p;
        wait_and_barrier<decltype(n_c)::value>();
        issue_a(kk + kF8D);
        asm volatile("" ::: "memory");  // codes and scales after the step's activations
        issue_codes(g + 2, p);
        if constexpr (p == 0) issue_scales(g + 2);
        f8_step<VM>(lds_a + (kk % kF8A) * kStageA8, cb, sb, ab, p, arow, brow, half, acc);
      };
      step(std::integral_constant<int, 0>{}, n0);
      step(std::integral_constant<int, 1>{}, n1);
      step(std::integral_constant<int, 2>{}, n2);
      step(std::integral_constant<int, 3>{}, n3);
    };
    using C3 = std::integral_constant<int, 3>;
    using C6 = std::integral_constant<int, 6>;
    using C7 = std::integral_constant<int, 7>;
    using C8 = std::integral_constant<int, 8>;
    using C9 = std::integral_constant<int, 9>;
    if (ng > 0) group(0, C3{}, C6{}, C7{}, C8{});
    for (int g = 1; g < ng; ++g) group(g, C9{}, C9{}, C9{}, C9{});
  };
  if (vm == 2)
    main_loop(std::integral_constant<int, 2>{});
  else if (vm == 1)
    main_loop(std::integral_constant<int, 1>{});
  else
    main_loop(std::integral_constant<int, 0>{});
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue
  if (GATEUP) {
    // h = silu(g) * u as MXFP8: the wave's 32 columns are one scale block
    const int col = nbase + 32 * wn + cl;
    uint8_t* hq = reinterpret_cast<uint8_t*>(a.out);
    uint8_t* hs = reinterpret_cast<uint8_t*>(a.out_scale);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      if (mi < vm) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * half + (i & 3);
          const float g = acc[0][mi][i];
          const float h = silu_mul(g, acc[1][mi][i]);
          float amax = fabsf(h);
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
          const uint32_t sbyte = mxfp8_scale_byte(amax);
          const float inv = __uint_as_float((254u - sbyte) << 23);  // 2^(127 - sbyte)
          if (row < nrows) {
            const size_t r = (size_t)(row0 + row);
            hq[r * a.N + col] = (uint8_t)e4m3_byte(h * inv);
            if (cl == 0) hs[r * (a.N / 32) + col / 32] = (uint8_t)sbyte;
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      if (mi < vm) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * half + (i & 3);
          if (row < nrows) {
            const size_t orow = (size_t)(row0 + row) * a.N;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const int col = nbase + 64 * wn + 32 * m + cl;
              reinterpret_cast<float*>(a.out)[orow + col] = acc[m][mi][i];
            }
          }
        }
      }
    }
  }
}

// x [T][K] bf16 -> MXFP8: one thread per 32-element block.
__global__ __launch_bounds__(256) void quantize_mxfp8_kernel(const uint16_t* __restrict__ x, long long nblocks,
                                                             uint8_t* __restrict__ q, uint8_t* __restrict__ qs) {
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + 32 * b);
  float v[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 w = src[j];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[8 * j + 2 * t] = __uint_as_float(ww[t] << 16);
      v[8 * j + 2 * t + 1] = __uint_as_float(ww[t] & 0xffff0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const uint32_t sbyte = mxfp8_scale_byte(amax);
  const float inv = __uint_as_float((254u - sbyte) << 23);
  uint32_t out[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    out[j] = e4m3_byte(v[4 * j] * inv) | (e4m3_byte(v[4 * j + 1] * inv) << 8) |
             (e4m3_byte(v[4 * j + 2] * inv) << 16) | (e4m3_byte(v[4 * j + 3] * inv) << 24);
  u32x4* dst = reinterpret_cast<u32x4*>(q + 32 * b);
  dst[0] = u32x4{out[0], out[1], out[2], out[3]};
  dst[1] = u32x4{out[4], out[5], out[6], out[7]};
  qs[b] = (uint8_t)sbyte;
}

// x [T][K] bf16 -> the same shape in bf16, each value rounded to the MXFP8
// grid of its 32-element block (E4M3 code times the block's E8M0 scale, both
// chosen as quantize_mxfp8_kernel does): the activations of the FP8 path with
// NVFP4 weights, whose products then run on bf16 MFMA.  One thread per block.
__global__ __launch_bounds__(256) void round_mxfp8_kernel(const uint16_t* __restrict__ x, long long nblocks,
                                                          uint16_t* __restrict__ y) {
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + 32 * b);
  float v[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 w = src[j];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[8 * j + 2 * t] = __uint_as_float(ww[t] << 16);
      v[8 * j + 2 * t + 1] = __uint_as_float(ww[t] & 0xffff0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const uint32_t sbyte = mxfp8_scale_byte(amax);
  const float inv = __uint_as_float((254u - sbyte) << 23);
  const float sc = __uint_as_float(sbyte << 23);
  uint32_t out[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t lo = f32_to_bf16(e4m3_to_f32(e4m3_byte(v[2 * j] * inv)) * sc);
    const uint32_t hi = f32_to_bf16(e4m3_to_f32(e4m3_byte(v[2 * j + 1] * inv)) * sc);
    out[j] = lo | (hi << 16);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(y + 32 * b);
#pragma unroll
  for (int j = 0; j < 4; ++j) dst[j] = u32x4{out[4 * j], out[4 * j + 1], out[4 * j + 2], out[4 * j + 3]};
}

// K-steps of loads in flight (register budget of two waves per SIMD).
constexpr int kDepthDirect = 2;  // gg_direct_b_kernel, MX-FP4 weights

// 4-bit GEMMs whose K (d for gate/up, f for down) holds whole code groups
// use gg_mx_group_kernel; other MX-FP4 GEMMs fall back to gg_direct_b_kernel
// (NVFP4 layers with such K take the GEMV path).
bool mx_grouped(int K) { return K % (kGroupSteps * BK) == 0; }

// Output columns per tile: gate/up counts columns of each of W_gate, W_up.
int tile_cols(const Dims& dm, bool gateup) {
  const int K = gateup ? dm.d : dm.f;
  const int base = (dm.wfmt == kMXFP4 && !mx_grouped(K)) ? 256 : 128;  // direct-B: 256
  return gateup ? base : 2 * base;
}

template <bool GATEUP>
hipError_t launch_gg(const Dims& dm, const GGArgs& a, hipStream_t s) {
  const size_t max_tiles = grouped_gemm_max_mtiles(dm) * (size_t)a.ntiles;
  const dim3 grid((unsigned)((max_tiles + kXcds - 1) / kXcds * kXcds)), block(kThreads);
  if (GATEUP && dm.fp8 && dm.wfmt == kNVFP4)
    gg_mx_row_kernel<kNVFP4, true, true><<<grid, block, 0, s>>>(a);  // h on the MXFP8 grid
  else if (dm.wfmt == kNVFP4)
    gg_mx_row_kernel<kNVFP4, GATEUP><<<grid, block, 0, s>>>(a);
  else if (dm.wfmt == kMXFP4 && mx_grouped(a.K))
    gg_mx_group_kernel<kMXFP4, GATEUP><<<grid, block, 0, s>>>(a);
  else if (dm.wfmt == kMXFP4)
    gg_direct_b_kernel<kMXFP4, GATEUP, kDepthDirect><<<grid, block, 0, s>>>(a);
  else
    gg_dma_kernel<GATEUP><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool grouped_gemm_ok(const Dims& dm) {
  if (dm.act != kBF16 || dm.T < kGemmMinT) return false;
  if (dm.wfmt == kNVFP4) return mx_grouped(dm.d) && mx_grouped(dm.f);
  // bf16 and MX-FP4 take d, f >= 64 (multiples of 32: a K tail of 32 is handled)
  return (dm.wfmt == kBF16 || dm.wfmt == kMXFP4) && dm.d >= BK && dm.f >= BK;
}

size_t grouped_gemm_max_mtiles(const Dims& dm) {
  const size_t Tk = (size_t)dm.Tk();
  const size_t E = (size_t)dm.E;
  return Tk / kGemmBM + (Tk < E ? Tk : E) + 1;
}

hipError_t launch_gg_gate_up(const Dims& dm, const void* x, const Plan& p, const Weights& w,
                             void* h, hipStream_t s) {
  LaunchTimer tm("gg_gate_up", s);
  const int tc = tile_cols(dm, true);
  GGArgs a{x, p.sorted_src, w.wg, w.wu, w.sg, w.su, w.tg, w.tu, nullptr, nullptr, p.mtiles, p.num_mtiles, h,
           dm.d, dm.f, dm.k, (dm.f + tc - 1) / tc, dm.T};
  return launch_gg<true>(dm, a, s);
}

hipError_t launch_gg_down(const Dims& dm, const void* h, const Plan& p, const Weights& w,
                          float* y_sorted, hipStream_t s) {
  LaunchTimer tm("gg_down", s);
  const int tc = tile_cols(dm, false);
  GGArgs a{h, nullptr, w.wd, nullptr, w.sd, nullptr, w.td, nullptr, nullptr, nullptr, p.mtiles, p.num_mtiles,
           y_sorted,
           dm.f, dm.d, dm.k, (dm.d + tc - 1) / tc, dm.T};
  return launch_gg<false>(dm, a, s);
}

bool fp8_path_ok(const Dims& dm) {
  return dm.act == kBF16 && is_fp4(dm.wfmt) && mx_grouped(dm.d) && mx_grouped(dm.f);
}

hipError_t launch_round_mxfp8(const void* x, long long rows, int K, void* y, hipStream_t s) {
  LaunchTimer tm("round_mxfp8", s);
  const long long nb = rows * (K / 32);
  if (nb == 0) return hipSuccess;
  const dim3 grid((unsigned)((nb + 255) / 256)), block(256);
  round_mxfp8_kernel<<<grid, block, 0, s>>>(reinterpret_cast<const uint16_t*>(x), nb,
                                            reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8(const void* x, long long rows, int K, uint8_t* q, uint8_t* qs,
                                 hipStream_t s) {
  LaunchTimer tm("quantize_mxfp8", s);
  const long long nb = rows * (K / 32);
  if (nb == 0) return hipSuccess;
  const dim3 grid((unsigned)((nb + 255) / 256)), block(256);
  quantize_mxfp8_kernel<<<grid, block, 0, s>>>(reinterpret_cast<const uint16_t*>(x), nb, q, qs);
  return hipGetLastError();
}

hipError_t launch_gg_f8_gate_up(const Dims& dm, const uint8_t* xq, const uint8_t* xs, const Plan& p,
                                const Weights& w, uint8_t* hq, uint8_t* hs, hipStream_t s) {
  LaunchTimer tm("gg_gate_up", s);
  GGArgs a{xq, p.sorted_src, w.wg, w.wu, w.sg, w.su, nullptr, nullptr, xs, hs, p.mtiles, p.num_mtiles,
           hq, dm.d, dm.f, dm.k, dm.f / (BN / 2), dm.T};
  const size_t max_tiles = grouped_gemm_max_mtiles(dm) * (size_t)a.ntiles;
  const dim3 grid((unsigned)((max_tiles + kXcds - 1) / kXcds * kXcds)), block(kThreads);
  gg_f8f4_kernel<true><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gg_f8_down(const Dims& dm, const uint8_t* hq, const uint8_t* hs, const Plan& p,
                             const Weights& w, float* y_sorted, hipStream_t s) {
  LaunchTimer tm("gg_down", s);
  GGArgs a{hq, nullptr, w.wd, nullptr, w.sd, nullptr, nullptr, nullptr, hs, nullptr, p.mtiles,
           p.num_mtiles, y_sorted, dm.f, dm.d, dm.k, dm.d / BN, dm.T};
  const size_t max_tiles = grouped_gemm_max_mtiles(dm) * (size_t)a.ntiles;
  const dim3 grid((unsigned)((max_tiles + kXcds - 1) / kXcds * kXcds)), block(kThreads);
  gg_f8f4_kernel<false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

MOE_DBG_TAKE_DEFINE(dbg_take_grouped_gemm)

}  // namespace moe
