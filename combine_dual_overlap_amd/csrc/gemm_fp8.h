// fp8 x fp8 grouped expert GEMM for gfx950 (activations and weights E4M3 fn).
//
// The fp8 expert path that the fused SiLU-mul + fp8 quantisation op of
// "[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM" (CI discussion)
// feeds.  C[m, n] = sum_k A[m, k] B[n, k] with
//   A = activation codes times the row's per-128-column power-of-two scale,
//   B = weight codes times the weight's 128 x 128 block scale (fp32).
//
// Work decomposition (the tile map is the one of the bf16 kernel,
// locate_tile: device-side per-expert row counts, XCD-aware order)
//  * BM activation rows x 256 weight rows per workgroup, 8 waves.  For the
//    gate/up GEMM a tile holds 128 gate rows and the 128 matching up rows, so
//    the tile owns whole 128-column groups of h and can quantise h in its
//    epilogue (per-row amax over the tile's 128 h columns, exchanged in LDS).
//  * K advances 128 per stage: one E4M3 K block of 128 bytes per row, the
//    same LDS geometry as a 64-wide bf16 stage (16-byte chunks XOR-swizzled by
//    row), half the LDS bytes per flop.  Two-deep register ring of global loads,
//    double-buffered LDS, one barrier per stage, unconditional steady-state
//    loads (the last stages are peeled).
//  * One v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 tile per stage.  The
//    hardware applies the activation row's E8M0 byte (scale operand of A; the
//    B scale byte is 127 = 1.0).  The weight block scale changes with the K
//    block, so each stage's product is accumulated into fp32 as
//    acc += scale_w * p (promotion per K block).
//  * Operand lanes: lane l holds row (or weight row) l % 16 and the 32 bytes
//    [32 (l / 16), 32 (l / 16) + 32) of the stage's K block.  A and B use the
//    same K assignment, so every product pairs matching K indices.
//  * Two stagings of the same arithmetic: k_gemm_f8 moves each stage through a
//    two-deep register ring into double-buffered LDS; k_gemm_f8d (further down)
//    loads straight into three LDS stages with LDS DMA.  The host takes the
//    DMA variant for K <= 4096.
#pragma once

#include "fp8_act.h"
#include "gemm_mfma.h"

namespace dbomoe {

constexpr int kF8BK = 128;          // K per stage (= bytes per row per stage)
constexpr int kF8BN = 256;          // weight rows per column tile
constexpr int kF8Threads = 512;     // 8 waves
constexpr int kF8MaxK = 64 * 128;   // a weight scale row (K / 128 blocks) fits one register per lane
constexpr int kF8DmaMaxK = 4096;    // longest K given to the LDS-DMA variant

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Byte offset of 16-byte chunk c of LDS row r (rows of 128 bytes).
__device__ __forceinline__ int lds8_off(int r, int c) { return r * kF8BK + ((c ^ (r & 7)) << 4); }

struct F8Group {
  const uint8_t* A;       // activation codes [rows][K]
  const uint8_t* As;      // E8M0 bytes [rows][K / 128]
  const uint8_t* B;       // weight codes [experts][b_rows][K]
  const float* Bs;        // weight block scales [experts][b_rows / 128][K / 128]
  int K;                  // multiple of 128
  int N;                  // I (gate/up) or H (down)
  int b_rows;             // 2I or H
  int n_tiles;            // column tiles (I / 128 or H / 256)
  void* C;                // gate/up: h codes [rows][N]; down: bf16 [rows][N]
  uint8_t* Cs;            // gate/up: h E8M0 bytes [rows][N / 128]
};

struct F8Params {
  GemmParams loc;         // tile map only: offsets, E_loc, dense_rows, g[0].n_tiles
  F8Group g;
};

template <int BM>
struct F8Shape {
  static constexpr int WAVES_M = BM == 128 ? 2 : 1;
  static constexpr int WAVES_N = 8 / WAVES_M;
  static constexpr int WM = BM / WAVES_M;          // 64
  static constexpr int WN = kF8BN / WAVES_N;       // 64 (BM 128) or 32 (BM 64)
  static constexpr int TM = WM / 16;
  static constexpr int TN = WN / 16;
  static_assert(BM == 64 || BM == 128, "row tile");
};

// LDS row of the weight tile -> weight row inside the expert's matrix.
template <int MODE>
__device__ __forceinline__ int f8_b_row(const F8Group& g, int nt, int r) {
  if constexpr (MODE == MODE_GATEUP)
    return r < kF8BN / 2 ? nt * (kF8BN / 2) + r : g.N + nt * (kF8BN / 2) + (r - kF8BN / 2);
  else
    return nt * kF8BN + r;
}

// First LDS weight row of the wave's tn-th 16-column MFMA tile.
template <int MODE, int WN, int TN>
__device__ __forceinline__ int f8_b_lds_row(int wn, int tn) {
  if constexpr (MODE == MODE_GATEUP)
    return tn < TN / 2 ? wn * (WN / 2) + tn * 16 : kF8BN / 2 + wn * (WN / 2) + (tn - TN / 2) * 16;
  else
    return wn * WN + tn * 16;
}

template <int BM, int MODE>
__device__ __forceinline__ void gemm_tile_f8(const F8Group& g, const TileLoc& t, uint8_t (*sA)[BM * kF8BK],
                                             uint8_t (*sB)[kF8BN * kF8BK]) {
  using S = F8Shape<BM>;
  constexpr int TM = S::TM, TN = S::TN, WM = S::WM, WN = S::WN;
  constexpr int CA = BM * (kF8BK / 16) / kF8Threads;     // 16-byte A chunks per thread
  constexpr int CB = kF8BN * (kF8BK / 16) / kF8Threads;  // 16-byte B chunks per thread
  static_assert(CA >= 1 && CB >= 1, "chunking");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / S::WAVES_N;
  const int wn = wave % S::WAVES_N;
  const int K = g.K;
  const int KT = K / kF8BK;
  // K walked from a per-weight-tile starting stage (see the bf16 kernel): the
  // loads and the scales of loop stage kt are those of K block stage_k(kt).
  const int kt_rot = __builtin_amdgcn_readfirstlane(rotation_start(t.e * g.n_tiles + t.nt, KT));
  auto stage_k = [&](int kt) {
    const int ks = kt + kt_rot;
    return ks >= KT ? ks - KT : ks;
  };
  const int KB = K / 128;
  const int nt = t.nt;

  // Per-thread chunk c = tid + i * 512 sits in tile row tid / 8 + 64 i with the
  // same 16-byte column tid % 8, so its LDS offset is the i = 0 offset plus
  // i * 64 rows (the XOR swizzle depends on the row only through row & 7), and
  // its global address is the i = 0 address plus a workgroup-uniform step.
  // Addresses are 32-bit offsets from workgroup-uniform bases (a tile's rows
  // and an expert's matrix are each < 4 GiB).
  const int r0 = tid / (kF8BK / 16);
  const int kc0 = tid % (kF8BK / 16);
  const int lds0 = lds8_off(r0, kc0);
  constexpr int kLdsStep = (kF8Threads / (kF8BK / 16)) * kF8BK;   // 64 rows
  const uint8_t* a_base = g.A + (t.row_begin + t.m_off) * static_cast<int64_t>(K);
  uint32_t a_off[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    int r = r0 + i * (kF8Threads / (kF8BK / 16));
    r = t.m_off + r < t.rows ? r : t.rows - 1 - t.m_off;
    a_off[i] = static_cast<uint32_t>(r) * static_cast<uint32_t>(K) + kc0 * 16;
  }
  const uint8_t* be = g.B + static_cast<size_t>(t.e) * g.b_rows * K;
  const uint32_t b_off0 = static_cast<uint32_t>(f8_b_row<MODE>(g, nt, r0)) * static_cast<uint32_t>(K) + kc0 * 16;
  // weight row of chunk i minus that of chunk 0 (uniform)
  auto b_step = [&](int i) -> uint32_t {
    return static_cast<uint32_t>(f8_b_row<MODE>(g, nt, i * (kF8Threads / (kF8BK / 16))) - f8_b_row<MODE>(g, nt, 0)) *
           static_cast<uint32_t>(K);
  };
  // E8M0 bytes of the activation rows this lane feeds to the MFMA (row l % 16
  // of each 16-row subtile; rows past the expert's end read its last row).
  const int frag_row = lane & 15;
  const uint8_t* as_base = g.As + t.row_begin * static_cast<int64_t>(KB);
  const int as_row0 = t.m_off + wm * WM + frag_row;
  // Weight block scales: gate and up blocks (gate/up) or the wave's 128-row block (down).
  const float* bs_e = g.Bs + static_cast<size_t>(t.e) * (g.b_rows / 128) * KB;
  const float* ws0;
  const float* ws1;
  if constexpr (MODE == MODE_GATEUP) {
    ws0 = bs_e + static_cast<size_t>(nt) * KB;
    ws1 = bs_e + static_cast<size_t>(g.N / 128 + nt) * KB;
  } else {
    ws0 = bs_e + static_cast<size_t>((nt * kF8BN + wn * WN) / 128) * KB;
    ws1 = ws0;
  }

  // The two weight scale rows, one K block per lane (K <= 64 blocks), picked
  // per stage with v_readlane: the K loop issues no scalar memory loads,
  // whose completion counter the LDS reads share (a wait for an LDS read
  // would otherwise also wait for a scale load in flight).
  float wsv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) wsv[j] = (j == 0 ? ws0 : ws1)[min(lane, KB - 1)];
  auto wscale = [&](int j, int kb) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsv[j]), kb));
  };

  u32x4_t ra0[CA], rb0[CB], ra1[CA], rb1[CB];
  uint32_t sa0[TM], sa1[TM];
  auto load_data = [&](int kt, u32x4_t* ra, u32x4_t* rb) {
    const uint32_t k0 = static_cast<uint32_t>(stage_k(kt)) * kF8BK;
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_base + (a_off[i] + k0));
#pragma unroll
    for (int i = 0; i < CB; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(be + (b_off0 + b_step(i) + k0));
  };
  auto load_scales = [&](int kt, uint32_t* sa) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int mr = min(as_row0 + tm * 16, t.rows - 1);
      sa[tm] = as_base[static_cast<uint32_t>(mr) * static_cast<uint32_t>(KB) + stage_k(kt)];
    }
  };
  auto store_stage = [&](int buf, const u32x4_t* ra, const u32x4_t* rb) {
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4_t*>(&sA[buf][lds0 + i * kLdsStep]) = ra[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) *reinterpret_cast<u32x4_t*>(&sB[buf][lds0 + i * kLdsStep]) = rb[i];
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int frag_q = lane >> 4;             // 32-byte K slice of the stage
  const int tm_valid = __builtin_amdgcn_readfirstlane(
      max(0, min(TM, (t.rows - t.m_off - wm * WM + 15) / 16)));
  auto frag = [&](const uint8_t* base, int row) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(base + lds8_off(row, 2 * frag_q));
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(base + lds8_off(row, 2 * frag_q + 1));
    return i32x8_t{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                   static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                   static_cast<int>(hi[2]), static_cast<int>(hi[3])};
  };
  // One 16-row subtile at a time, two MFMAs at a time, each pair followed by
  // its promotion into the accumulators, so at most two products are live
  // (the scheduling barriers keep the compiler from hoisting later MFMAs).
  auto compute_stage = [&](int buf, const uint32_t* sa, int kt_c) {
    const int kb = stage_k(kt_c);
    const float sw[2] = {wscale(0, kb), wscale(1, kb)};
    i32x8_t bfv[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) bfv[tn] = frag(sB[buf], f8_b_lds_row<MODE, WN, TN>(wn, tn) + frag_row);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      if (tm < tm_valid) {
        const i32x8_t af = frag(sA[buf], wm * WM + tm * 16 + frag_row);
        // two MFMAs at a time, then their promotion (bounds the live products)
#pragma unroll
        for (int tn0 = 0; tn0 < TN; tn0 += 2) {
          f32x4_t pr[2];
#pragma unroll
          for (int j = 0; j < 2; ++j)
            pr[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af, bfv[tn0 + j], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, static_cast<int>(sa[tm]), 0, 127);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[tm][tn0 + j] += pr[j] * ((MODE == MODE_GATEUP && tn0 + j >= TN / 2) ? sw[1] : sw[0]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Two-deep register ring (see the bf16 kernel): stage s is loaded into slot
  // s % 2 two stages before its MFMAs and stored to LDS buffer s % 2 one stage
  // before them; steady-state loads are unconditional.  A slot's scales are
  // reloaded right after the MFMAs that used them (one stage ahead).
  load_data(0, ra0, rb0);
  load_scales(0, sa0);
  if (KT > 1) {
    load_data(1, ra1, rb1);
    load_scales(1, sa1);
  }
  store_stage(0, ra0, rb0);
  __syncthreads();
  int kt = 0;
  for (; kt + 3 < KT; kt += 2) {
    load_data(kt + 2, ra0, rb0);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage(0, sa0, kt);
    load_scales(kt + 2, sa0);
    store_stage(1, ra1, rb1);
    __syncthreads();
    load_data(kt + 3, ra1, rb1);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage(1, sa1, kt + 1);
    load_scales(kt + 3, sa1);
    store_stage(0, ra0, rb0);
    __syncthreads();
  }
  const int left = KT - kt;                 // 1, 2 or 3 stages; stage kt is in LDS buffer 0
  if (left == 3) {
    load_data(kt + 2, ra0, rb0);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage(0, sa0, kt);
    load_scales(kt + 2, sa0);
    store_stage(1, ra1, rb1);
    __syncthreads();
    compute_stage(1, sa1, kt + 1);
    store_stage(0, ra0, rb0);
    __syncthreads();
    compute_stage(0, sa0, kt + 2);
  } else if (left == 2) {
    compute_stage(0, sa0, kt);
    store_stage(1, ra1, rb1);
    __syncthreads();
    compute_stage(1, sa1, kt + 1);
  } else {
    compute_stage(0, sa0, kt);
  }

  // Epilogue.  Accumulator element r of lane l in a 16x16 tile is
  // (row 4*(l/16) + r, column l%16).
  const int col_in = lane & 15;
  const int row_q = (lane >> 4) * 4;
  if constexpr (MODE == MODE_GATEUP) {
    // h = silu(gate) * up, then per row: amax over the tile's 128 h columns
    // (this wave's WN/2 columns in registers and lanes, the other waves'
    // through LDS), E8M0 scale, E4M3 codes.
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN / 2; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[tm][tn][r] = silu_f32(acc[tm][tn][r]) * acc[tm][tn + TN / 2][r];
    float* s_amax = reinterpret_cast<float*>(&sA[0][0]);   // [WAVES_N][BM]
    __syncthreads();                                       // every wave is done with the LDS tiles
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = 0.f;
#pragma unroll
        for (int tn = 0; tn < TN / 2; ++tn) m = fmaxf(m, fabsf(acc[tm][tn][r]));
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
        if (col_in == 0) s_amax[wn * BM + wm * WM + tm * 16 + row_q + r] = m;
      }
    __syncthreads();
    uint8_t* Cq = static_cast<uint8_t*>(g.C);
    const int groups = g.N / kQGroup;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = wm * WM + tm * 16 + row_q + r;
        const int mr = t.m_off + lr;
        float m = 0.f;
#pragma unroll
        for (int w = 0; w < S::WAVES_N; ++w) m = fmaxf(m, s_amax[w * BM + lr]);
        const uint32_t b = e8m0_for_amax(m);
        const float inv = e8m0_inv_scale(b);
        if (mr < t.rows) {
          const int64_t row = t.row_begin + mr;
#pragma unroll
          for (int tn = 0; tn < TN / 2; ++tn) {
            const int col = nt * (kF8BN / 2) + wn * (WN / 2) + tn * 16 + col_in;
            Cq[row * g.N + col] = fp8_rne1(acc[tm][tn][r] * inv);
          }
          if (wn == 0 && col_in == 0) g.Cs[row * groups + nt] = static_cast<uint8_t>(b);
        }
      }
  } else {
    bf16_t* C = static_cast<bf16_t*>(g.C);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int col = nt * kF8BN + wn * WN + tn * 16 + col_in;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mr = t.m_off + wm * WM + tm * 16 + row_q + r;
          if (mr < t.rows) C[(t.row_begin + mr) * g.N + col] = f32_to_bf16(acc[tm][tn][r]);
        }
      }
  }
}

template <int BM, int MODE>
__global__ __launch_bounds__(kF8Threads, 2) void k_gemm_f8(F8Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kF8BK];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kF8BN * kF8BK];
  int* s_loc = reinterpret_cast<int*>(&sA[0][0]);   // tile location, before sA holds A tiles
  TileLoc t;
  if (!locate_tile<BM>(p.loc, s_loc, t)) return;
  __syncthreads();                                  // s_loc read by all before sA is filled
  gemm_tile_f8<BM, MODE>(p.g, t, sA, sB);
}



// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane l's bytes land at LDS address lds_addr + 16 l.  Issued as inline
// assembly so that the compiler does not wait for every such load before each
// LDS read (it cannot tell the three stage buffers apart); the kernel counts
// them itself with s_waitcnt.  The assembly sets M0, which the compiler does
// not use anywhere in these kernels (checked in the generated code).

// ---------------------------------------------------------------------------
// The same GEMM with the staging through LDS DMA: three LDS stages of BM + 256
// rows (the A rows, then the weight rows), each 8-row group loaded by one wave
// instruction whose lanes take the row's 16-byte chunks in swizzled order, so
// no register ring and no LDS store instructions.  The activation scale bytes
// of the tile sit in LDS for the whole K.  Stage kt + 2 is issued once the
// barrier of stage kt shows every wave done with the buffer it overwrites.
// Bitwise equal to k_gemm_f8.  Measured standalone (MI355X, 128-row tiles):
// Qwen3-shaped prefill gate/up 304.5 -> 270.5 us, down 184.5 -> 170.0 us;
// R1-shaped share down 157.1 -> 132.1 us, but gate/up (K = 7168) 193.2 ->
// 232.2 us, so it is used for K <= 4096 only.
template <int BM> struct F8DmaShape {
  static constexpr int ROWS = BM + kF8BN;            // A rows then B rows
  static constexpr int STAGE = ROWS * kF8BK;         // bytes per LDS stage
  static constexpr int NQ = ROWS / 8 / 8;            // 8-row groups per wave per stage
};

template <int BM, int MODE>
__device__ __forceinline__ void gemm_tile_f8d(const F8Group& g, const TileLoc& t, uint8_t* sT, uint8_t* s_as) {
  using S = F8Shape<BM>;
  using D = F8DmaShape<BM>;
  constexpr int TM = S::TM, TN = S::TN, WM = S::WM, WN = S::WN, NQ = D::NQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;
  const int K = g.K, KT = K / kF8BK, KB = K / 128, nt = t.nt;
  const int kt_rot = __builtin_amdgcn_readfirstlane(rotation_start(t.e * g.n_tiles + t.nt, KT));
  auto stage_k = [&](int kt) { const int ks = kt + kt_rot; return ks >= KT ? ks - KT : ks; };

  // activation scale bytes of the tile's rows, whole K (rows past the end: last row)
  for (int i = tid; i < BM * KB; i += kF8Threads) {
    const int r = i / KB, kb = i % KB;
    const int mr = min(t.m_off + r, t.rows - 1);
    s_as[r * KB + kb] = g.As[(t.row_begin + mr) * static_cast<int64_t>(KB) + kb];
  }
  // global source of each of this wave's 8-row groups (lane: row l/8, logical chunk (l%8)^(l/8))
  const uint8_t* a_base = g.A + (t.row_begin + t.m_off) * static_cast<int64_t>(K);
  const uint8_t* be = g.B + static_cast<size_t>(t.e) * g.b_rows * K;
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;
  const uint8_t* src[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int R = 8 * (wave + 8 * i) + lrow;           // row of the combined tile
    if (R < BM) {
      const int r = t.m_off + R < t.rows ? R : t.rows - 1 - t.m_off;
      src[i] = a_base + static_cast<int64_t>(r) * K + 16 * lchunk;
    } else {
      src[i] = be + static_cast<size_t>(f8_b_row<MODE>(g, nt, R - BM)) * K + 16 * lchunk;
    }
  }
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(sT))));
  auto issue = [&](int kt, int buf) {
    const uint32_t k0 = static_cast<uint32_t>(stage_k(kt)) * kF8BK;
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      lds_dma16(lds_base + buf * D::STAGE + (wave + 8 * i) * 8 * kF8BK, src[i] + k0);
  };

  const float* bs_e = g.Bs + static_cast<size_t>(t.e) * (g.b_rows / 128) * KB;
  const float* ws0;
  const float* ws1;
  if constexpr (MODE == MODE_GATEUP) {
    ws0 = bs_e + static_cast<size_t>(nt) * KB;
    ws1 = bs_e + static_cast<size_t>(g.N / 128 + nt) * KB;
  } else {
    ws0 = bs_e + static_cast<size_t>((nt * kF8BN + wn * WN) / 128) * KB;
    ws1 = ws0;
  }
  float wsv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) wsv[j] = (j == 0 ? ws0 : ws1)[min(lane, KB - 1)];
  auto wscale = [&](int j, int kb) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsv[j]), kb)); };
  __syncthreads();                           // s_as complete; compiler loads above waited for

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int frag_row = lane & 15, frag_q = lane >> 4;
  const int tm_valid = __builtin_amdgcn_readfirstlane(max(0, min(TM, (t.rows - t.m_off - wm * WM + 15) / 16)));
  auto frag = [&](const uint8_t* base, int row) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(base + lds8_off(row, 2 * frag_q));
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(base + lds8_off(row, 2 * frag_q + 1));
    return i32x8_t{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]), static_cast<int>(lo[3]),
                   static_cast<int>(hi[0]), static_cast<int>(hi[1]), static_cast<int>(hi[2]), static_cast<int>(hi[3])};
  };
  auto compute_stage = [&](const uint8_t* st, int kt_c) {
    const int kb = stage_k(kt_c);
    const float sw[2] = {wscale(0, kb), wscale(1, kb)};
    i32x8_t bfv[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) bfv[tn] = frag(st, BM + f8_b_lds_row<MODE, WN, TN>(wn, tn) + frag_row);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      if (tm < tm_valid) {
        const int ar = wm * WM + tm * 16 + frag_row;
        const i32x8_t af = frag(st, ar);
        const int sa = s_as[ar * KB + kb];
#pragma unroll
        for (int tn0 = 0; tn0 < TN; tn0 += 2) {
          f32x4_t pr[2];
#pragma unroll
          for (int j = 0; j < 2; ++j)
            pr[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfv[tn0 + j], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                       0, sa, 0, 127);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[tm][tn0 + j] += pr[j] * ((MODE == MODE_GATEUP && tn0 + j >= TN / 2) ? sw[1] : sw[0]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // every compiler-issued load (scale rows, scale bytes) completes here, so the
  // compiler sees nothing outstanding inside the loop and inserts no vmcnt wait
  // of its own there; only the LDS DMA below is in flight, counted by hand.
  __builtin_amdgcn_s_waitcnt(0);
  issue(0, 0);
  if (KT > 1) issue(1, 1);
  int buf = 0;
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT)
      __builtin_amdgcn_s_waitcnt(0xF70 | NQ);   // stage kt landed; stage kt + 1 may be in flight
    else
      __builtin_amdgcn_s_waitcnt(0xF70);
    __syncthreads();
    if (kt + 2 < KT) issue(kt + 2, buf == 0 ? 2 : buf - 1);
    compute_stage(sT + buf * D::STAGE, kt);
    buf = buf == 2 ? 0 : buf + 1;
  }

  const int col_in = lane & 15;
  const int row_q = (lane >> 4) * 4;
  if constexpr (MODE == MODE_GATEUP) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN / 2; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[tm][tn][r] = silu_f32(acc[tm][tn][r]) * acc[tm][tn + TN / 2][r];
    float* s_amax = reinterpret_cast<float*>(sT);
    __syncthreads();
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = 0.f;
#pragma unroll
        for (int tn = 0; tn < TN / 2; ++tn) m = fmaxf(m, fabsf(acc[tm][tn][r]));
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
        if (col_in == 0) s_amax[wn * BM + wm * WM + tm * 16 + row_q + r] = m;
      }
    __syncthreads();
    uint8_t* Cq = static_cast<uint8_t*>(g.C);
    const int groups = g.N / kQGroup;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = wm * WM + tm * 16 + row_q + r;
        const int mr = t.m_off + lr;
        float m = 0.f;
#pragma unroll
        for (int w = 0; w < S::WAVES_N; ++w) m = fmaxf(m, s_amax[w * BM + lr]);
        const uint32_t b = e8m0_for_amax(m);
        const float inv = e8m0_inv_scale(b);
        if (mr < t.rows) {
          const int64_t row = t.row_begin + mr;
#pragma unroll
          for (int tn = 0; tn < TN / 2; ++tn) {
            const int col = nt * (kF8BN / 2) + wn * (WN / 2) + tn * 16 + col_in;
            Cq[row * g.N + col] = fp8_rne1(acc[tm][tn][r] * inv);
          }
          if (wn == 0 && col_in == 0) g.Cs[row * groups + nt] = static_cast<uint8_t>(b);
        }
      }
  } else {
    bf16_t* C = static_cast<bf16_t*>(g.C);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int col = nt * kF8BN + wn * WN + tn * 16 + col_in;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mr = t.m_off + wm * WM + tm * 16 + row_q + r;
          if (mr < t.rows) C[(t.row_begin + mr) * g.N + col] = f32_to_bf16(acc[tm][tn][r]);
        }
      }
  }
}

template <int BM, int MODE>
__global__ __launch_bounds__(kF8Threads, 2) void k_gemm_f8d(F8Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sT[3 * F8DmaShape<BM>::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t s_as[BM * (kF8DmaMaxK / 128)];
  int* s_loc = reinterpret_cast<int*>(sT);
  TileLoc t;
  if (!locate_tile<BM>(p.loc, s_loc, t)) return;
  __syncthreads();
  gemm_tile_f8d<BM, MODE>(p.g, t, sT, s_as);
}

}  // namespace dbomoe
