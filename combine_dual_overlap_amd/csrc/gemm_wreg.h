// Grouped GEMM for large experts (prefill) on gfx950: activations through LDS,
// weights straight into registers.
//
// With hundreds of rows per expert the GEMM is bound by the MFMA units, and
// what limits them is LDS traffic: a 64x64 wave tile that reads both operands
// from LDS needs about as many LDS bytes per clock as a CU can serve.  Here
// only the activations go through LDS; each wave streams its own weight rows
// from global memory into MFMA operand registers (a weight element is used by
// one wave only), so the LDS carries the activation tile once per stage in and
// once per wave out.
//
// Shape: one workgroup per CU, 4 waves, a 128-row activation tile and 256
// weight rows (64 per wave: for the gate/up GEMM 32 gate rows and the 32
// matching up rows, so SwiGLU stays in registers).  Each wave holds a 128 x 64
// block of fp32 accumulators (8 x 4 tiles of v_mfma_f32_16x16x32_bf16).
// K advances 64 per stage:
//  * activations: loaded into registers two stages ahead, stored into a
//    double-buffered, XOR-swizzled LDS tile one stage ahead, one barrier per
//    stage;
//  * weights: loaded three stages ahead into a four-deep register ring (fp8:
//    one 16-byte load per 16-row subtile per stage; bf16: two).
// Loads past the last stage re-read the last stage (clamped addresses, never
// used), so every load in the loop is unconditional and the compiler keeps
// all of them in flight.  Rows past the tile's end read the tile's last row
// and are never stored.
// fp8 codes are expanded per MFMA operand: code value x block scale, rounded
// once to bf16 (a stage's 64-wide K piece of a 16-row subtile lies in one
// scale block), and the lane layout is the weight-streaming kernel's
// (gemm_wstream.h): for bf16, K step s of a stage uses k = 32s + 8g; for fp8,
// the one 16-byte load holds both steps, step q using k = 16g + 8q.
#pragma once

#include "gemm_wstream.h"

namespace dbomoe {

constexpr int kWrRows = 128;             // activation rows per tile
constexpr int kWrWaveRows = 64;          // weight rows per wave
constexpr int kWrBN = 4 * kWrWaveRows;   // weight rows per column tile
constexpr int kWrBK = 64;                // K per stage

template <int MODE, bool FP8>
__device__ __forceinline__ void gemm_tile_wr(const GemmGroup& g, const TileLoc& t, bf16_t* sA) {
  constexpr int TM = kWrRows / 16;              // 8 activation subtiles
  constexpr int TN = kWrWaveRows / 16;          // 4 weight subtiles
  constexpr int BL = FP8 ? 1 : 2;               // 16-byte weight loads per subtile per stage
  constexpr int CPR = kWrBK / 8;                // 16-byte activation chunks per row per stage
  constexpr int CA = kWrRows * CPR / 256;       // per thread
  constexpr int ROW = kWrBK;                    // LDS row length (one swizzle run of 8 chunks x 2)
  static_assert(CA == 4, "activation staging");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int frow = lane & 15;
  const int fg = lane >> 4;
  const int K = g.K;
  const int n = K / kWrBK;                      // stages (K is a multiple of 64)

  // ---- weight rows of the wave's four subtiles
  int wrow[TN];
  if constexpr (MODE == MODE_GATEUP) {
    const int c0 = t.nt * (kWrBN / 2) + wave * (kWrWaveRows / 2);   // first output column of the wave
#pragma unroll
    for (int j = 0; j < TN / 2; ++j) {
      wrow[j] = c0 + 16 * j + frow;                                 // gate
      wrow[TN / 2 + j] = g.N + c0 + 16 * j + frow;                  // matching up
    }
  } else {
#pragma unroll
    for (int j = 0; j < TN; ++j) wrow[j] = t.nt * kWrBN + wave * kWrWaveRows + 16 * j + frow;
  }
  const uint8_t* bptr[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const size_t row_elem = static_cast<size_t>(t.e) * g.b_estride + static_cast<size_t>(wrow[j]) * g.ldb;
    bptr[j] = FP8 ? static_cast<const uint8_t*>(g.B) + row_elem + 16 * fg
                  : reinterpret_cast<const uint8_t*>(static_cast<const bf16_t*>(g.B) + row_elem + 8 * fg);
  }
  // fp8 scale rows: gate/up subtiles 0-1 share one 128-row block, 2-3 another;
  // the down GEMM's 64 rows lie in one block.
  const float* srow0 = nullptr;
  const float* srow1 = nullptr;
  if constexpr (FP8) {
    const int kblocks = K / 128;
    const float* se = g.bscale + static_cast<size_t>(t.e) * (g.b_rows / 128) * kblocks;
    srow0 = se + static_cast<size_t>((wrow[0] - frow) / 128) * kblocks;
    srow1 = se + static_cast<size_t>((wrow[TN - 1] - frow) / 128) * kblocks;
  }

  // ---- activation staging: thread tid moves chunk tid % CPR of rows tid / CPR + 32 i
  const int a_kc = tid % CPR;
  const int a_r0 = tid / CPR;
  const bf16_t* a_base = g.A + t.e * g.a_estride + t.row_begin * g.lda + a_kc * 8;
  int a_row[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    int mr = t.m_off + a_r0 + 32 * i;
    a_row[i] = mr < t.rows ? mr : t.rows - 1;
  }

  u32x4_t ra0[CA], ra1[CA];
  u32x4_t rb0[TN][BL], rb1[TN][BL], rb2[TN][BL], rb3[TN][BL];
  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto load_a = [&](int s, u32x4_t (&ra)[CA]) {
    const int64_t k0 = static_cast<int64_t>(min(s, n - 1)) * kWrBK;
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_base + a_row[i] * g.lda + k0);
  };
  auto store_a = [&](int buf, const u32x4_t (&ra)[CA]) {
#pragma unroll
    for (int i = 0; i < CA; ++i)
      *reinterpret_cast<u32x4_t*>(&sA[buf * kWrRows * ROW + lds_off(a_r0 + 32 * i, a_kc)]) = ra[i];
  };
  auto load_b = [&](int s, u32x4_t (&rb)[TN][BL]) {
    const size_t k0 = static_cast<size_t>(min(s, n - 1)) * kWrBK;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int l = 0; l < BL; ++l)
        rb[j][l] = *reinterpret_cast<const u32x4_t*>(bptr[j] + (FP8 ? k0 : (k0 + 32 * l) * 2));
  };
  auto compute = [&](int s, int buf, const u32x4_t (&rb)[TN][BL]) {
    float sc0 = 1.f, sc1 = 1.f;
    if constexpr (FP8) {
      sc0 = srow0[(s * kWrBK) / 128];
      sc1 = srow1[(s * kWrBK) / 128];
    }
    const bf16_t* A = sA + buf * kWrRows * ROW;
#pragma unroll
    for (int q = 0; q < kWrBK / 32; ++q) {
      bf16x8_t bv[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (FP8) {
          const float sc = (MODE == MODE_GATEUP && j >= TN / 2) ? sc1 : sc0;
          const int w0 = static_cast<int>(rb[j][0][2 * q]);
          const int w1 = static_cast<int>(rb[j][0][2 * q + 1]);
          const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
          const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
          const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
          const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
          const u32x4_t u{cvt_bf16x2(f0[0] * sc, f0[1] * sc), cvt_bf16x2(f1[0] * sc, f1[1] * sc),
                          cvt_bf16x2(f2[0] * sc, f2[1] * sc), cvt_bf16x2(f3[0] * sc, f3[1] * sc)};
          bv[j] = __builtin_bit_cast(bf16x8_t, u);
        } else {
          bv[j] = __builtin_bit_cast(bf16x8_t, rb[j][q]);
        }
      }
      // activation chunk of K step q for lane group fg: fp8 uses k = 16 fg + 8 q,
      // bf16 k = 32 q + 8 fg
      const int kc = FP8 ? 2 * fg + q : 4 * q + fg;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&A[lds_off(tm * 16 + frow, kc)]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[tm][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bv[j], acc[tm][j], 0, 0, 0);
      }
    }
  };

  // One stage: loads two (activations) and three (weights) stages ahead,
  // MFMAs of stage s, the activations of stage s + 1 into LDS, barrier.
  // Stages past the end keep the loads (clamped) and the barrier, skip the MFMAs.
  auto step = [&](int s, u32x4_t (&ra_cur)[CA], u32x4_t (&ra_next)[CA], const u32x4_t (&rb_cur)[TN][BL],
                  u32x4_t (&rb_ahead)[TN][BL]) {
    load_a(s + 2, ra_cur);
    load_b(s + 3, rb_ahead);
    __builtin_amdgcn_sched_barrier(0);
    if (s < n) compute(s, s & 1, rb_cur);
    __builtin_amdgcn_sched_barrier(0);
    store_a((s + 1) & 1, ra_next);
    __syncthreads();
  };

  load_a(0, ra0);
  load_b(0, rb0);
  load_b(1, rb1);
  load_a(1, ra1);
  load_b(2, rb2);
  store_a(0, ra0);
  __syncthreads();
  for (int s = 0; s < n; s += 4) {
    step(s, ra0, ra1, rb0, rb3);
    step(s + 1, ra1, ra0, rb1, rb0);
    step(s + 2, ra0, ra1, rb2, rb1);
    step(s + 3, ra1, ra0, rb3, rb2);
  }

  // ---- epilogue: accumulator element r of lane l is (row 4*(l/16) + r, column l%16)
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
#pragma unroll
        for (int j = 0; j < TN / 2; ++j)
          Cr[wrow[j]] = f32_to_bf16(silu_f32(acc[tm][j][r]) * acc[tm][TN / 2 + j][r]);
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) Cr[wrow[j]] = f32_to_bf16(acc[tm][j][r]);
      }
    }
}

// Column tiles of this kernel: 128 output columns (gate/up) or 256 (down).
inline int wr_col_tiles(int mode, int N) { return mode == MODE_GATEUP ? N / (kWrBN / 2) : N / kWrBN; }

template <int MODE, bool FP8>
__global__ __launch_bounds__(256, 1) void k_gemm_wr(GemmParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2 * kWrRows * kWrBK];
  int* s_loc = reinterpret_cast<int*>(&sA[0]);
  TileLoc t;
  if (!locate_tile<kWrRows>(p, s_loc, t)) return;
  __syncthreads();                                  // s_loc read by all before sA is filled
  if (FP8 && t.grp == 0)
    gemm_tile_wr<MODE, FP8>(p.g[0], t, sA);
  else
    gemm_tile_wr<MODE, false>(p.g[t.grp], t, sA);
}

}  // namespace dbomoe
