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
// Tile: 128 rows (one m-tile of an expert) x 4 waves; each wave owns two
// 32-column B operands (gate/up: the same 32 columns of W_gate and W_up, so
// the SwiGLU epilogue is wave-local; down: 64 consecutive columns of W_down).
// K advances 64 per step.  B (weights, read once from HBM) streams straight
// into registers D steps ahead (plain cached loads: the other m-tiles of the
// same panel read it from L2); A (activation rows, shared by the 4 waves)
// goes through a D-deep register ring into a double-buffered, XOR-swizzled
// LDS tile.  Both rings lead by D steps so that waiting for the oldest load
// never waits for younger ones.
//
// Tile order: logical tiles run expert by expert, n-tile by n-tile, m-tile
// by m-tile, and each XCD (blockIdx % 8 under round-robin dispatch) takes a
// contiguous range.  The m-tiles of one (expert, n-tile) panel therefore run
// together on one XCD and share the weight panel through its L2; the n-tiles
// of one expert follow each other there and reuse its activation rows.
#include "device.h"
#include "internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = kGemmBM;  // 128
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kXcds = 8;

struct GGArgs {
  const void* a_src;      // gate/up: x [T][K]; down: h [T*k][K] (bf16)
  const int* sorted_src;  // gate/up: row r reads x[sorted_src[r] / k]
  const void* w0;         // gate/up: W_gate; down: W_down   ([E][N][K] or codes)
  const void* w1;         // gate/up: W_up
  const uint8_t* s0;      // MX-FP4 scales of w0 / w1
  const uint8_t* s1;
  const int* mtiles;
  const int* num_mtiles;
  void* out;              // gate/up: h bf16 [T*k][N]; down: y_sorted fp32 [T*k][N]
  int K, N, k, ntiles;
};

template <int WF>
struct BRegs;
template <>
struct BRegs<kBF16> {  // 4 x 16 B per matrix per step: the lane's 32 K-values
  u32x4 v[2][4];
};
template <>
struct BRegs<kMXFP4> {  // 16 B of codes and one scale per matrix per step
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
    const float sc = e8m0_to_f32(b.s[m]);
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
    return __builtin_bit_cast(bf16x8_t, r);
  }
}

// LDS A tile: 128 rows x 128 B; 16-byte unit u of row r lives at unit
// u ^ (r & 7), so the 8 rows read together by a fragment hit 8 distinct
// bank groups.
__device__ __forceinline__ int a_off(int row, int unit) {
  return row * (BK * 2) + ((unit ^ (row & 7)) << 4);
}

template <int WF, bool GATEUP, int D>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GGArgs a) {
  __shared__ __align__(16) char lds[2][BM * BK * 2];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;

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
  const int half = lane >> 5;
  const int cl = lane & 31;
  int col0, col1;
  if (GATEUP) {
    col0 = ntile * 128 + wave * 32 + cl;
    col1 = col0;
  } else {
    col0 = ntile * 256 + wave * 64 + cl;
    col1 = col0 + 32;
  }
  const int c0c = min(col0, a.N - 1);
  const int c1c = min(col1, a.N - 1);
  const char* wbase0 = reinterpret_cast<const char*>(a.w0);
  const char* wbase1 = reinterpret_cast<const char*>(GATEUP ? a.w1 : a.w0);
  const char *p0, *p1;
  const uint8_t *q0 = nullptr, *q1 = nullptr;
  if constexpr (WF == kBF16) {
    p0 = wbase0 + ((size_t)e * a.N + c0c) * a.K * 2 + half * 64;
    p1 = wbase1 + ((size_t)e * a.N + c1c) * a.K * 2 + half * 64;
  } else {
    p0 = wbase0 + ((size_t)e * a.N + c0c) * (a.K / 2) + half * 16;
    p1 = wbase1 + ((size_t)e * a.N + c1c) * (a.K / 2) + half * 16;
    q0 = a.s0 + ((size_t)e * a.N + c0c) * (a.K / 32) + half;
    q1 = (GATEUP ? a.s1 : a.s0) + ((size_t)e * a.N + c1c) * (a.K / 32) + half;
  }

  // ---- A rows staged by this thread: row tid/2, units (tid&1)*4 .. +3
  const int arow = tid >> 1;
  const int aunit = (tid & 1) * 4;
  const int src_row = row0 + min(arow, nrows - 1);
  const size_t a_rb = (size_t)a.K * 2;
  const char* ap = reinterpret_cast<const char*>(a.a_src) +
                   (GATEUP ? (size_t)(a.sorted_src[src_row] / a.k) : (size_t)src_row) * a_rb +
                   aunit * 16;

  const int nk = a.K / BK;
  u32x4 areg[D][4];
  BRegs<WF> breg[D];
  auto load_a = [&](u32x4* r, int kk) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = ld16(ap + (size_t)kk * (BK * 2) + 16 * j);
  };
  auto store_a = [&](const u32x4* r, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(&lds[buf][a_off(arow, aunit + j)]) = r[j];
  };

  f32x16_t acc0[4], acc1[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    acc0[mi] = f32x16_t{};
    acc1[mi] = f32x16_t{};
  }

  // ---- prologue: A and B of steps 0..D-1 in flight; A(0) into LDS.
  // Every step issues the same loads (past the end they re-read the last
  // step), so the load sequence is branch-free and the compiler's wait
  // counts stay exact: waiting for the oldest ring entry never waits for the
  // younger ones.
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_a(areg[j], min(j, nk - 1));
    load_b<WF>(breg[j], p0, p1, q0, q1, min(j, nk - 1));
  }
  store_a(areg[0], 0);
  load_a(areg[0], min(D, nk - 1));
  __syncthreads();

  // ---- main loop, unrolled by D so ring slots are static.  A last partial
  // group (nk % D != 0) only skips the MFMAs.
  for (int kk0 = 0; kk0 < nk; kk0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int kk = kk0 + j;
      if (kk < nk) {
        const char* abuf = lds[kk & 1];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_t b0 = b_frag<WF>(breg[j], 0, s);
          const bf16x8_t b1 = b_frag<WF>(breg[j], 1, s);
#pragma unroll
          for (int mi = 0; mi < 4; ++mi) {
            const int row = mi * 32 + cl;
            const bf16x8_t af =
                *reinterpret_cast<const bf16x8_t*>(abuf + a_off(row, half * 4 + s));
            acc0[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b0, acc0[mi], 0, 0, 0);
            acc1[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b1, acc1[mi], 0, 0, 0);
          }
        }
      }
      load_b<WF>(breg[j], p0, p1, q0, q1, min(kk + D, nk - 1));
      const int jn = (j + 1) % D;
      store_a(areg[jn], (kk + 1) & 1);
      load_a(areg[jn], min(kk + 1 + D, nk - 1));
      __syncthreads();
    }
  }

  // ---- epilogue.  C layout of a 32x32 MFMA: lane holds column lane%32 and
  // rows 8*(i/4) + 4*(lane/32) + i%4 for i in 0..15.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = mi * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (row < nrows) {
        const size_t orow = (size_t)(row0 + row) * a.N;
        if (GATEUP) {
          if (col0 < a.N) {
            const float g = acc0[mi][i];
            const float u = acc1[mi][i];
            reinterpret_cast<uint16_t*>(a.out)[orow + col0] =
                f32_to_bf16(g / (1.0f + expf(-g)) * u);
          }
        } else {
          if (col0 < a.N) reinterpret_cast<float*>(a.out)[orow + col0] = acc0[mi][i];
          if (col1 < a.N) reinterpret_cast<float*>(a.out)[orow + col1] = acc1[mi][i];
        }
      }
    }
  }
}

#ifndef MOE_GG_DEPTH
#define MOE_GG_DEPTH 4
#endif
constexpr int kDepth = MOE_GG_DEPTH;  // K-steps of loads in flight

template <bool GATEUP>
hipError_t launch_gg(const Dims& dm, const GGArgs& a, hipStream_t s) {
  const size_t max_tiles = grouped_gemm_max_mtiles(dm) * (size_t)a.ntiles;
  const dim3 grid((unsigned)((max_tiles + kXcds - 1) / kXcds * kXcds)), block(kThreads);
  if (dm.wfmt == kMXFP4)
    grouped_gemm_kernel<kMXFP4, GATEUP, kDepth><<<grid, block, 0, s>>>(a);
  else
    grouped_gemm_kernel<kBF16, GATEUP, kDepth><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool grouped_gemm_ok(const Dims& dm) {
  return dm.act == kBF16 && (dm.wfmt == kBF16 || dm.wfmt == kMXFP4) && dm.T > kDecodeMaxT &&
         dm.d % BK == 0 && dm.f % BK == 0;
}

size_t grouped_gemm_max_mtiles(const Dims& dm) {
  const size_t Tk = (size_t)dm.Tk();
  const size_t E = (size_t)dm.E;
  return Tk / kGemmBM + (Tk < E ? Tk : E) + 1;
}

hipError_t launch_gg_gate_up(const Dims& dm, const void* x, const Plan& p, const Weights& w,
                             void* h, hipStream_t s) {
  LaunchTimer tm("gg_gate_up", s);
  GGArgs a{x, p.sorted_src, w.wg, w.wu, w.sg, w.su, p.mtiles, p.num_mtiles, h,
           dm.d, dm.f, dm.k, (dm.f + 127) / 128};
  return launch_gg<true>(dm, a, s);
}

hipError_t launch_gg_down(const Dims& dm, const void* h, const Plan& p, const Weights& w,
                          float* y_sorted, hipStream_t s) {
  LaunchTimer tm("gg_down", s);
  GGArgs a{h, nullptr, w.wd, nullptr, w.sd, nullptr, p.mtiles, p.num_mtiles, y_sorted,
           dm.f, dm.d, dm.k, (dm.d + 255) / 256};
  return launch_gg<false>(dm, a, s);
}

}  // namespace moe
