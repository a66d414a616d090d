// Weight-streaming grouped GEMM for gfx950 (few rows per expert: decode, and
// any share whose expert weights dominate the bytes).
//
// When an expert meets only a few dozen activation rows, the GEMM is bound by
// reading the expert weights from HBM once, and what sets the achieved
// bandwidth is how the weight rows are streamed.  Measured on MI355X (decode
// gate/up shape, 768 MB of weights):
//  * 128-byte pieces of each weight row per K step (the LDS-tiled kernel's
//    stage) reach about 4.8 TB/s; 512-byte pieces about 5.5 TB/s;
//  * a workgroup barrier per K step, which ties every wave to the slowest one,
//    costs 5-10 %; so does a coarse workgroup (8 waves over 256 weight rows, one
//    per CU, against 4 waves over 128 rows, two per CU), through the idle waves
//    of a finishing workgroup and the last partial round of workgroups.
// This kernel therefore
//  * gives each workgroup one 16-row activation tile and 128 weight rows, two
//    workgroups per CU; the whole activation tile (16 rows x K, K <= 2048,
//    64 KB) is loaded into LDS once, XOR-swizzled by row, behind the only
//    barrier of the tile;
//  * lets each of the 4 waves stream its own 32 weight rows straight from HBM
//    into registers, already in MFMA operand layout (a weight element is used by
//    one wave only, so it never touches LDS), 512 bytes of each row per chunk,
//    the next chunk loading while the current one is multiplied;
//  * keeps the tile map and the groups of the LDS-tiled kernel (gemm_mfma.h):
//    for the gate/up GEMM each wave holds 16 gate rows and the 16 matching up
//    rows, so SwiGLU stays in registers.
// Experts with more than 16 rows take several row tiles; the tile order puts
// the row tiles of one weight tile next to each other on one XCD, so the
// repeated weight reads are served by its L2.
// fp8 codes are expanded per MFMA operand: code value x block scale, rounded
// once to bf16 (a 64-wide K piece of a 16-row subtile lies in one scale block).
//
// MFMA operand layout (v_mfma_f32_16x16x32_bf16): lane l supplies row l%16 and
// 8 consecutive K values of group l/16.  For bf16 weights K step s of a chunk
// uses k = 32s + 8g, as the LDS-tiled kernel does (the two give identical
// bits); for fp8 weights a 16-byte load holds two steps, so step s = 2p + q
// uses k = 64p + 16g + 8q.  A and B always use the same k.
#pragma once

#include <type_traits>

#include "gemm_mfma.h"

namespace dbomoe {

constexpr int kWsRows = 16;              // activation rows per tile
constexpr int kWsKMax = 2048;            // longest K whose activation tile fits in LDS
constexpr int kWsWaves = 4;
constexpr int kWsBN = 128;               // weight rows per column tile (32 per wave)

// LDS element offset of 16-byte chunk kc of activation row r (rows of `row`
// elements, a multiple of 128): chunks are XOR-swizzled by row inside runs of
// 16 (256 bytes), so the 16 rows one MFMA operand read touches hit distinct
// banks.
__device__ __forceinline__ int ws_lds(int r, int kc, int row) {
  return r * row + (((kc & ~15) | ((kc ^ r) & 15)) << 3);
}

// K offset, inside a chunk, of the 8 values lane group g holds at K step s.
template <bool FP8>
__device__ __forceinline__ int ws_koff(int s, int g) {
  if constexpr (FP8) return 64 * (s >> 1) + 16 * g + 8 * (s & 1);
  return 32 * s + 8 * g;
}

// One K chunk of NS steps from a wave's two weight subtiles: NS 16-byte loads
// per subtile for bf16, NS/2 for fp8 (each holds two steps).
template <int NS, bool FP8>
struct WsChunk {
  static constexpr int LOADS = FP8 ? NS / 2 : NS;
  static constexpr int STEPS = NS;
  u32x4_t b[2][LOADS];
};

// One wave's share of a column tile: 32 weight rows (gate/up: 16 gate rows and
// the 16 matching up rows; down: 32 consecutive rows) against TM 16-row
// activation subtiles held in LDS.  The host keeps every wave's rows inside
// the matrix (I % 64 == 0 for 64 gate/up columns per tile, H % 128 == 0).
template <int TM, int MODE, bool FP8>
struct WsWave {
  const uint8_t* bptr[2];
  const float* srow[2];
  int wrow[2];
  int frow, fg;
  f32x4_t acc[TM][2];

  __device__ __forceinline__ void init(const GemmGroup& g, const TileLoc& t) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    frow = lane & 15;
    fg = lane >> 4;
    if constexpr (MODE == MODE_GATEUP) {
      wrow[0] = t.nt * (kWsBN / 2) + wave * 16 + frow;     // gate
      wrow[1] = g.N + wrow[0];                              // matching up
    } else {
      wrow[0] = t.nt * kWsBN + wave * 32 + frow;
      wrow[1] = wrow[0] + 16;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const size_t row_elem = static_cast<size_t>(t.e) * g.b_estride + static_cast<size_t>(wrow[j]) * g.ldb;
      bptr[j] = FP8 ? static_cast<const uint8_t*>(g.B) + row_elem + 16 * fg
                    : reinterpret_cast<const uint8_t*>(static_cast<const bf16_t*>(g.B) + row_elem + 8 * fg);
      srow[j] = nullptr;
    }
    if constexpr (FP8) {
      const int kblocks = g.K / 128;
      const float* se = g.bscale + static_cast<size_t>(t.e) * (g.b_rows / 128) * kblocks;
#pragma unroll
      for (int j = 0; j < 2; ++j) srow[j] = se + static_cast<size_t>((wrow[j] - frow) / 128) * kblocks;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // The chunk of weights starting at K offset k0.
  template <class Ch>
  __device__ __forceinline__ void load(Ch& ch, int k0) const {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int l = 0; l < Ch::LOADS; ++l) {
        const size_t off = FP8 ? static_cast<size_t>(k0) + 64 * l : (static_cast<size_t>(k0) + 32 * l) * 2;
        ch.b[j][l] = *reinterpret_cast<const u32x4_t*>(bptr[j] + off);
      }
  }

  // MFMAs of the chunk at K offset k0; its activations sit in LDS columns
  // starting at k0 - kbase of rows `lrow` elements long.
  template <class Ch>
  __device__ __forceinline__ void compute(const Ch& ch, int k0, const bf16_t* sA, int lrow, int kbase) {
#pragma unroll
    for (int s = 0; s < Ch::STEPS; ++s) {
      const int kc = (k0 - kbase + ws_koff<FP8>(s, fg)) >> 3;
      bf16x8_t af[TM];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        af[tm] = *reinterpret_cast<const bf16x8_t*>(&sA[ws_lds(tm * 16 + frow, kc, lrow)]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8_t bv;
        if constexpr (FP8) {
          const u32x4_t& q = ch.b[j][s >> 1];
          const float sc = srow[j][(k0 + 64 * (s >> 1)) / 128];
          const int w0 = static_cast<int>(q[(s & 1) * 2]);
          const int w1 = static_cast<int>(q[(s & 1) * 2 + 1]);
          const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
          const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
          const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
          const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
          const u32x4_t u{cvt_bf16x2(f0[0] * sc, f0[1] * sc), cvt_bf16x2(f1[0] * sc, f1[1] * sc),
                          cvt_bf16x2(f2[0] * sc, f2[1] * sc), cvt_bf16x2(f3[0] * sc, f3[1] * sc)};
          bv = __builtin_bit_cast(bf16x8_t, u);
        } else {
          bv = __builtin_bit_cast(bf16x8_t, ch.b[j][s]);
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tm][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], bv, acc[tm][j], 0, 0, 0);
      }
    }
  }

  // Accumulator element r of lane l is (row 4*(l/16) + r, column l%16).
  __device__ __forceinline__ void store(const GemmGroup& g, const TileLoc& t) const {
    const int row_q = fg * 4;
    bf16_t* C = static_cast<bf16_t*>(g.C) + t.e * g.c_estride;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mr = t.m_off + tm * 16 + row_q + r;
        if (mr >= t.rows) continue;
        bf16_t* Cr = C + (t.row_begin + mr) * g.ldc;
        if constexpr (MODE == MODE_GATEUP) {
          Cr[wrow[0]] = f32_to_bf16(silu_f32(acc[tm][0][r]) * acc[tm][1][r]);
        } else {
          Cr[wrow[0]] = f32_to_bf16(acc[tm][0][r]);
          Cr[wrow[1]] = f32_to_bf16(acc[tm][1][r]);
        }
      }
  }
};

// ---------------------------------------------------------------------------
// Whole-K activation tile (K <= 2048), 16-row tiles.
// KS steps per full chunk, REM steps in a first, partial chunk (0 if K is a
// multiple of the chunk).  Every load and MFMA inside a chunk is
// unconditional, so the compiler can keep all of a chunk's loads in flight.
template <int KS, int REM, int MODE, bool FP8>
__device__ __forceinline__ void gemm_tile_ws(const GemmGroup& g, const TileLoc& t, bf16_t* sA) {
  constexpr int KC = KS * 32;                   // K per full chunk
  static_assert(!FP8 || (KS % 2 == 0 && REM % 2 == 0), "fp8 steps come in pairs");
  using Full = WsChunk<KS, FP8>;
  using Part = WsChunk<(REM > 0 ? REM : 2), FP8>;

  const int tid = threadIdx.x;
  const int K = g.K;
  const int lrow = (K + 127) & ~127;            // LDS row length: whole swizzle runs
  WsWave<kWsRows / 16, MODE, FP8> w;
  w.init(g, t);

  const int kp = REM * 32;                      // K where the full chunks start
  const int n_full = (K - kp) / KC;
  auto kfull = [&](int c) { return kp + c * KC; };
  Full b0, b1;
  Part bp;

  // Weights of the partial chunk and the first full chunk are issued ahead of
  // the activation tile, the second full chunk behind it.  Rows past the
  // tile's end read the tile's last row (never stored out).
  if constexpr (REM > 0) w.load(bp, 0);
  if (n_full > 0) w.load(b0, kfull(0));
  {
    constexpr int kThreads = kWsWaves * kWave;
    constexpr int kPer = kWsRows * kWsKMax / 8 / kThreads;   // 16-byte chunks per thread at K = kWsKMax
    const int chunks = K / 8;                               // per row
    const int total = kWsRows * chunks;
    const bf16_t* Ab = g.A + t.e * g.a_estride;
    u32x4_t v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * kThreads + tid;
      if (c < total) {
        int mr = t.m_off + c / chunks;
        mr = mr < t.rows ? mr : t.rows - 1;
        v[i] = *reinterpret_cast<const u32x4_t*>(Ab + (t.row_begin + mr) * g.lda + (c % chunks) * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * kThreads + tid;
      if (c < total) *reinterpret_cast<u32x4_t*>(&sA[ws_lds(c / chunks, c % chunks, lrow)]) = v[i];
    }
  }
  if (n_full > 1) w.load(b1, kfull(1));
  __syncthreads();                                          // activation tile complete; no barrier follows

  if constexpr (REM > 0) w.compute(bp, 0, sA, lrow, 0);
  // Steady state: both next chunks exist, so both loads are unconditional and
  // chunk c + 1 stays in flight while chunk c is multiplied.  The scheduling
  // barriers keep each chunk's loads where they are issued: the compiler would
  // otherwise sink them below the next chunk's MFMAs, and the wait for one
  // chunk would then also wait for the other.
  int c = 0;
  for (; c + 3 < n_full; c += 2) {
    w.compute(b0, kfull(c), sA, lrow, 0);
    __builtin_amdgcn_sched_barrier(0);
    w.load(b0, kfull(c + 2));
    __builtin_amdgcn_sched_barrier(0);
    w.compute(b1, kfull(c + 1), sA, lrow, 0);
    __builtin_amdgcn_sched_barrier(0);
    w.load(b1, kfull(c + 3));
    __builtin_amdgcn_sched_barrier(0);
  }
  const int left = n_full - c;                              // 0..3
  if (left == 3) {
    w.compute(b0, kfull(c), sA, lrow, 0);
    __builtin_amdgcn_sched_barrier(0);
    w.load(b0, kfull(c + 2));
    __builtin_amdgcn_sched_barrier(0);
    w.compute(b1, kfull(c + 1), sA, lrow, 0);
    w.compute(b0, kfull(c + 2), sA, lrow, 0);
  } else if (left == 2) {
    w.compute(b0, kfull(c), sA, lrow, 0);
    w.compute(b1, kfull(c + 1), sA, lrow, 0);
  } else if (left == 1) {
    w.compute(b0, kfull(c), sA, lrow, 0);
  }
  w.store(g, t);
}

// Dispatches on the partial chunk's step count (bf16 K is a multiple of 64,
// fp8 K of 128, so REM is even, and a multiple of 4 for fp8).
template <int KS, int MODE, bool FP8>
__device__ __forceinline__ void gemm_tile_ws_rem(const GemmGroup& g, const TileLoc& t, bf16_t* sA) {
  const int rem = (g.K / 32) % KS;
  switch (rem) {
    case 0: gemm_tile_ws<KS, 0, MODE, FP8>(g, t, sA); break;
    case 4: gemm_tile_ws<KS, 4, MODE, FP8>(g, t, sA); break;
    case 8: if constexpr (KS > 8) gemm_tile_ws<KS, 8, MODE, FP8>(g, t, sA); break;
    case 12: if constexpr (KS > 12) gemm_tile_ws<KS, 12, MODE, FP8>(g, t, sA); break;
    default:
      if constexpr (!FP8) {
        if (rem == 2) gemm_tile_ws<KS, 2, MODE, FP8>(g, t, sA);
        else gemm_tile_ws<KS, 6, MODE, FP8>(g, t, sA);
      }
      break;
  }
}

// Two workgroups of 4 waves per CU (the activation tile takes 64 KB of LDS).
template <int MODE, bool FP8>
__global__ __launch_bounds__(kWsWaves * kWave, 2) void k_gemm_ws(GemmParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[kWsRows * kWsKMax];
  int* s_loc = reinterpret_cast<int*>(&sA[0]);
  TileLoc t;
  if (!locate_tile<kWsRows>(p, s_loc, t)) return;
  __syncthreads();                                  // s_loc read by all before sA is filled
  if (FP8 && t.grp == 0)
    gemm_tile_ws_rem<16, MODE, FP8>(p.g[0], t, sA);
  else
    gemm_tile_ws_rem<8, MODE, false>(p.g[t.grp], t, sA);
}

}  // namespace dbomoe
