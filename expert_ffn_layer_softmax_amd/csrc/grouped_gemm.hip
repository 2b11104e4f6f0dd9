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
// Two tile schemes, both 128 rows (one m-tile of an expert) x 8 waves (two
// per SIMD), K advancing 64 per step:
//
// bf16 weights (gg_lds_kernel): 256 B-columns per tile (gate/up: 128
// columns of W_gate and the same 128 of W_up, so the SwiGLU epilogue is
// wave-local; down: 256 columns of W_down), K advancing 64 per step.  Both
// operands go through double-buffered, XOR-swizzled LDS tiles.  512 threads
// (8 waves, two per SIMD) fetch each step with 16-byte loads, 8 consecutive
// threads per 128-byte row segment, into a D-deep register ring: loads for a
// step are issued D steps before its MFMAs.  Every step issues the same loads
// (past the end they re-read the last step), so waiting for the oldest ring
// entry never waits for younger ones.  MX-FP4 weights are converted to bf16
// (block scale applied by the instruction) on their way into LDS.  Waves form
// a 2 (rows) x 4 (columns) grid, each owning 64 rows x (2 x 32) columns.
//
// MX-FP4 weights (gg_direct_b_kernel): h wave owns all
// 128 rows and two 32-column B operands: gate/up: the same 32 columns of
// W_gate and W_up (the SwiGLU epilogue stays wave-local), so a tile spans
// 256 columns of each; down: 64 consecutive columns of W_down, 512 per tile.
// K advances 64 per step.  A weight column belongs to exactly one wave, so
// the weights stream straight from memory into registers, D steps ahead; the
// activation rows, shared by all 8 waves, go through a D-deep register ring
// into a double-buffered, XOR-swizzled LDS tile (8 threads per 128-byte row
// segment, full cache lines).  Every step issues the same loads (past the end
// they re-read the last step), so waiting for the oldest ring entry never
// waits for younger ones.  Per substep a wave reads 4 A fragments from LDS for
// 8 MFMAs; B never touches LDS.
//
// The weights are 4x smaller there, so streaming them per wave into
// registers costs little and keeps LDS traffic to the shared activations.
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
constexpr int kThreads = 512;
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
    const float sc = e8m0_to_f32(b.s[m]);
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
    return __builtin_bit_cast(bf16x8_t, r);
  }
}

constexpr int BN = 256;                 // gg_lds_kernel: B-tile rows (weight columns) per tile
constexpr int kBPieces = BN * 8 / kThreads;   // bf16 B pieces per thread per step

// One step's global data held by a thread between its load and its LDS store.
template <int WF>
struct Stage;
template <>
struct Stage<kBF16> {
  u32x4 a[kAPieces];
  u32x4 b[kBPieces];
};
template <>
struct Stage<kMXFP4> {  // B: 16 B of codes (one 32-element block) + its scale
  u32x4 a[kAPieces];
  u32x4 b;
  uint32_t s;
};

template <int WF, bool GATEUP, int D>
__global__ __launch_bounds__(kThreads) void gg_lds_kernel(GGArgs a) {
  __shared__ __align__(16) char lds_a[2][BM * BK * 2];
  __shared__ __align__(16) char lds_b[2][BN * BK * 2];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int wm = wave >> 2;  // 0..1: rows 64*wm ..
  const int wn = wave & 3;   // 0..3: columns
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
  const int nbase = ntile * (GATEUP ? BN / 2 : BN);

  // ---- global sources of this thread's pieces
  const int unit = tid & 7;
  const size_t a_rb = (size_t)a.K * 2;
  const char* ap[kAPieces];
#pragma unroll
  for (int i = 0; i < kAPieces; ++i) {
    const int r = (tid >> 3) + i * (kThreads / 8);
    const int src = row0 + min(r, nrows - 1);
    ap[i] = reinterpret_cast<const char*>(a.a_src) +
            (GATEUP ? (size_t)(a.sorted_src[src] / a.k) : (size_t)src) * a_rb + unit * 16;
  }
  // B-tile row r -> weight matrix and column
  auto bcol = [&](int r, const void*& w, const uint8_t*& sc) {
    int col;
    if (GATEUP) {
      const bool up = r >= BN / 2;
      w = up ? a.w1 : a.w0;
      sc = up ? a.s1 : a.s0;
      col = nbase + (up ? r - BN / 2 : r);
    } else {
      w = a.w0;
      sc = a.s0;
      col = nbase + r;
    }
    return min(col, a.N - 1);
  };
  constexpr int NBP = (WF == kBF16) ? kBPieces : 1;
  const char* bp[NBP];
  const uint8_t* sp = nullptr;
  int b_unit0 = 0;  // MX-FP4: first LDS unit this thread's block fills
  if constexpr (WF == kBF16) {
#pragma unroll
    for (int i = 0; i < kBPieces; ++i) {
      const void* w;
      const uint8_t* sc;
      const int col = bcol((tid >> 3) + i * (kThreads / 8), w, sc);
      bp[i] = reinterpret_cast<const char*>(w) + ((size_t)e * a.N + col) * a_rb + unit * 16;
    }
  } else {
    const void* w;
    const uint8_t* sc;
    const int col = bcol(tid >> 1, w, sc);
    const int hb = tid & 1;  // which 32-element block of the step
    bp[0] = reinterpret_cast<const char*>(w) + ((size_t)e * a.N + col) * (a.K / 2) + hb * 16;
    sp = sc + ((size_t)e * a.N + col) * (a.K / 32) + hb;
    b_unit0 = hb * 4;
  }

  const int nk = a.K / BK;
  Stage<WF> ring[D];
  auto load_stage = [&](Stage<WF>& st, int kk) {
#pragma unroll
    for (int i = 0; i < kAPieces; ++i) st.a[i] = ld16(ap[i] + (size_t)kk * (BK * 2));
    if constexpr (WF == kBF16) {
#pragma unroll
      for (int i = 0; i < kBPieces; ++i) st.b[i] = ld16(bp[i] + (size_t)kk * (BK * 2));
    } else {
      st.b = ld16(bp[0] + (size_t)kk * (BK / 2));
      st.s = sp[2 * kk];
    }
  };
  auto store_stage = [&](const Stage<WF>& st, int buf) {
#pragma unroll
    for (int i = 0; i < kAPieces; ++i)
      *reinterpret_cast<u32x4*>(&lds_a[buf][t_off((tid >> 3) + i * (kThreads / 8), unit)]) = st.a[i];
    if constexpr (WF == kBF16) {
#pragma unroll
      for (int i = 0; i < kBPieces; ++i)
        *reinterpret_cast<u32x4*>(&lds_b[buf][t_off((tid >> 3) + i * (kThreads / 8), unit)]) = st.b[i];
    } else {
      const float scale = e8m0_to_f32(st.s);
      const uint32_t cw[4] = {st.b.x, st.b.y, st.b.z, st.b.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 r;
        r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], scale, 0));
        r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], scale, 1));
        r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], scale, 2));
        r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], scale, 3));
        *reinterpret_cast<u32x4*>(&lds_b[buf][t_off(tid >> 1, b_unit0 + j)]) = r;
      }
    }
  };

  // fragment rows of this lane
  int arow[2], brow[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) arow[mi] = 64 * wm + 32 * mi + cl;
#pragma unroll
  for (int m = 0; m < 2; ++m) brow[m] = GATEUP ? (m * (BN / 2) + 32 * wn + cl) : (64 * wn + 32 * m + cl);

  f32x16_t acc[2][2];  // [matrix / column subtile][row subtile]
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) acc[m][mi] = f32x16_t{};

  // ---- prologue: steps 0..D-1 in flight, step 0 into LDS
#pragma unroll
  for (int j = 0; j < D; ++j) load_stage(ring[j], min(j, nk - 1));
  store_stage(ring[0], 0);
  load_stage(ring[0], min(D, nk - 1));
  __syncthreads();

  // ---- main loop, unrolled by D so ring slots are static.  A last partial
  // group (nk % D != 0) only skips the MFMAs.
  for (int kk0 = 0; kk0 < nk; kk0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int kk = kk0 + j;
      if (kk < nk) {
        const char* abuf = lds_a[kk & 1];
        const char* bbuf = lds_b[kk & 1];
        // fragments one substep ahead of the MFMAs that consume them
        bf16x8_t af[2][2], bf[2][2];
        auto read_frags = [&](int s, bf16x8_t* a2, bf16x8_t* b2) {
#pragma unroll
          for (int mi = 0; mi < 2; ++mi)
            a2[mi] = *reinterpret_cast<const bf16x8_t*>(abuf + t_off(arow[mi], half * 4 + s));
#pragma unroll
          for (int m = 0; m < 2; ++m)
            b2[m] = *reinterpret_cast<const bf16x8_t*>(bbuf + t_off(brow[m], half * 4 + s));
        };
        read_frags(0, af[0], bf[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (s + 1 < 4) read_frags(s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
              acc[m][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][mi], bf[s & 1][m],
                                                                 acc[m][mi], 0, 0, 0);
        }
      }
      const int jn = (j + 1) % D;
      store_stage(ring[jn], (kk + 1) & 1);
      load_stage(ring[jn], min(kk + 1 + D, nk - 1));
      __syncthreads();
    }
  }

  // ---- epilogue.  C layout of a 32x32 MFMA: lane holds column lane%32 and
  // rows 8*(i/4) + 4*(lane/32) + i%4 for i in 0..15.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
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
            reinterpret_cast<uint16_t*>(a.out)[orow + col] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
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
            (GATEUP ? (size_t)(a.sorted_src[src] / a.k) : (size_t)src) * a_rb + unit * 16;
  }

  const int nk = a.K / BK;
  u32x4 aring[D][kAPieces];
  BRegs<WF> bring[D];
  auto load_a = [&](u32x4* r, int kk) {
#pragma unroll
    for (int i = 0; i < kAPieces; ++i) r[i] = ld16(ap[i] + (size_t)kk * (BK * 2));
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

  // ---- prologue: steps 0..D-1 in flight, step 0 into LDS
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_a(aring[j], min(j, nk - 1));
    load_b<WF>(bring[j], p0, p1, q0, q1, min(j, nk - 1));
  }
  store_a(aring[0], 0);
  load_a(aring[0], min(D, nk - 1));
  __syncthreads();

  // ---- main loop, unrolled by D so ring slots are static.  A last partial
  // group (nk % D != 0) only skips the MFMAs.
  for (int kk0 = 0; kk0 < nk; kk0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int kk = kk0 + j;
      if (kk < nk) {
        const char* abuf = lds_a[kk & 1];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bf16x8_t af[4];
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
            af[mi] = *reinterpret_cast<const bf16x8_t*>(abuf + t_off(32 * mi + cl, half * 4 + s));
          const bf16x8_t b0 = b_frag<WF>(bring[j], 0, s);
          const bf16x8_t b1 = b_frag<WF>(bring[j], 1, s);
#pragma unroll
          for (int mi = 0; mi < 4; ++mi) {
            acc[0][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], b0, acc[0][mi], 0, 0, 0);
            acc[1][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], b1, acc[1][mi], 0, 0, 0);
          }
        }
      }
      load_b<WF>(bring[j], p0, p1, q0, q1, min(kk + D, nk - 1));
      const int jn = (j + 1) % D;
      store_a(aring[jn], (kk + 1) & 1);
      load_a(aring[jn], min(kk + 1 + D, nk - 1));
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
            reinterpret_cast<uint16_t*>(a.out)[orow + col0] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
          }
        } else {
          if (col0 < a.N) reinterpret_cast<float*>(a.out)[orow + col0] = acc[0][mi][i];
          if (col1 < a.N) reinterpret_cast<float*>(a.out)[orow + col1] = acc[1][mi][i];
        }
      }
    }
  }
}

// K-steps of loads in flight (register budget of two waves per SIMD).
constexpr int kDepthLds = 2;     // gg_lds_kernel, bf16 weights
constexpr int kDepthDirect = 2;  // gg_direct_b_kernel, MX-FP4 weights

// Output columns per tile: gate/up counts columns of each of W_gate, W_up.
int tile_cols(const Dims& dm, bool gateup) {
  const int base = dm.wfmt == kMXFP4 ? 256 : 128;
  return gateup ? base : 2 * base;
}

template <bool GATEUP>
hipError_t launch_gg(const Dims& dm, const GGArgs& a, hipStream_t s) {
  const size_t max_tiles = grouped_gemm_max_mtiles(dm) * (size_t)a.ntiles;
  const dim3 grid((unsigned)((max_tiles + kXcds - 1) / kXcds * kXcds)), block(kThreads);
  if (dm.wfmt == kMXFP4)
    gg_direct_b_kernel<kMXFP4, GATEUP, kDepthDirect><<<grid, block, 0, s>>>(a);
  else
    gg_lds_kernel<kBF16, GATEUP, kDepthLds><<<grid, block, 0, s>>>(a);
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
  const int tc = tile_cols(dm, true);
  GGArgs a{x, p.sorted_src, w.wg, w.wu, w.sg, w.su, p.mtiles, p.num_mtiles, h,
           dm.d, dm.f, dm.k, (dm.f + tc - 1) / tc};
  return launch_gg<true>(dm, a, s);
}

hipError_t launch_gg_down(const Dims& dm, const void* h, const Plan& p, const Weights& w,
                          float* y_sorted, hipStream_t s) {
  LaunchTimer tm("gg_down", s);
  const int tc = tile_cols(dm, false);
  GGArgs a{h, nullptr, w.wd, nullptr, w.sd, nullptr, p.mtiles, p.num_mtiles, y_sorted,
           dm.f, dm.d, dm.k, (dm.d + tc - 1) / tc};
  return launch_gg<false>(dm, a, s);
}

}  // namespace moe
