// LDS-tiled bf16 MFMA "NT" GEMM for gfx950, shared by the router logits and the
// two grouped expert GEMMs.  C[m, n] = sum_k A[m, k] * B[n, k]: both operands
// are K-contiguous rows, which is how activations ([rows, H]) and the expert
// weights ([2I, H] and [H, I]) are stored, so no operand is ever transposed.
//
// Work decomposition
//  * Row tiles of BM rows per expert (the grouped GEMM's "M tiles"), column
//    tiles of BN = 128 weight rows; for the gate/up GEMM a column tile holds 64
//    gate rows and the 64 matching up rows, so SwiGLU is applied in registers.
//  * A launch covers up to two groups of tiles: group 0 is the routed experts,
//    whose per-expert row counts live on the device (every workgroup rebuilds
//    the tile map from `offsets` with one wave prefix scan, so the host launches
//    a worst-case grid and surplus workgroups exit at once); group 1 is E1 dense
//    experts over a fixed number of rows (the always-on shared experts, whose
//    down projection is cut into K chunks with one output slab each), so their
//    tiles run in the same launch instead of as a small grid of their own.
//    Group 1 tiles come first in the tile order, so they start with the launch.
//  * Workgroup b runs on XCD b % 8; the logical tile index is remapped so each
//    XCD walks a contiguous run of tiles.  Inside an expert the row tiles of one
//    column tile come first, then the next column tile, so row tiles that share
//    a weight tile run at the same time on one XCD and read it through its L2.
//  * 4 waves; each wave owns a WM x WN block made of 16x16 MFMA tiles
//    (v_mfma_f32_16x16x32_bf16, fp32 accumulators).  K advances BK per stage
//    (64; 128 for the 32-row decode tile when K allows).
//  * Two ways to stage a K slice.  gemm_tile: global loads run two stages
//    ahead of the MFMAs in a register ring and are stored into a
//    double-buffered LDS tile (one barrier per stage).  gemm_tile_dma: LDS DMA
//    (global_load_lds_dwordx4) writes the slices straight into a ring of LDS
//    buffers.  Either way LDS rows are BK elements with the 16-byte chunks
//    XOR-swizzled by row, so the rows an MFMA fragment read touches spread over
//    the banks without padding.
//  * The epilogue stages each wave's outputs through LDS and stores whole
//    16-byte pieces of output rows.
//  * fp8 e4m3 weights, on the register path, are expanded on their way to
//    LDS: code value times its 128x128 block scale, rounded once to bf16 (the
//    stage's K slice lies in one scale block, and so do the 64 gate or 64 up
//    rows of a tile).  The 64- and 128-row fp8 tiles of routed experts use
//    gemm_fp8w.h instead, which never rounds a weight.
#pragma once

#include <type_traits>

#include "common.h"

namespace dbomoe {

constexpr int kBK = 64;                  // K elements per LDS stage
constexpr int kLdsStride = kBK;          // bf16 elements per LDS row (chunks XOR-swizzled)
constexpr int kBN = 128;                 // weight rows per column tile (32-row tiles: 64)

// LDS element offset of 16-byte chunk c (8 bf16) of tile row r.
// With BK-wide stages the rows are BK elements long; the swizzle is the same.
template <int BK>
__device__ __forceinline__ int lds_off_k(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }
__device__ __forceinline__ int lds_off(int r, int c) { return lds_off_k<kLdsStride>(r, c); }

enum GemmMode { MODE_ROUTER = 0, MODE_GATEUP = 1, MODE_DOWN = 2 };

// One group of tiles: the same K, N and weight layout for every expert in it.
struct GemmGroup {
  const bf16_t* A;        // activation rows
  int64_t lda;            // elements between rows of A
  const void* B;          // [experts][b_rows][ldb] bf16 or fp8 codes
  int64_t ldb;            // elements between weight rows
  const float* bscale;    // fp8: [experts][b_rows/128][K/128], else NULL
  int K;                  // reduction length (multiple of 64; of 128 for fp8)
  int N;                  // output columns: E (router), I (gate/up), H (down)
  int b_rows;             // weight rows per expert
  int n_tiles;            // column tiles
  void* C;                // output rows (fp32 for the router, bf16 otherwise)
  int64_t ldc;
  // Per-expert element strides of A, B and C (group 1's dense experts: A and
  // B column offsets of a K chunk, C slab offset); group 0 uses b_estride only.
  int64_t a_estride, b_estride, c_estride;
};

struct GemmParams {
  GemmGroup g[2];
  const int32_t* offsets; // group 0: [E_loc+1] device offsets, or NULL (one expert of dense_rows rows)
  int E_loc;
  int64_t dense_rows;
  int64_t rows1;          // group 1: rows of each of its dense experts (0 = no group 1)
  int E1;                 // group 1: number of dense experts
  const float* bias;      // router logit bias or NULL (unused with split-K)
  int64_t split_c;        // router split-K: blockIdx.y selects K range [y*K, (y+1)*K)
                          // and output slab C + y*split_c
};

template <int BM, int WAVES_M, int WAVES_N, int BN = kBN>
struct TileShape {
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int TM = WM / 16;
  static constexpr int TN = WN / 16;
  static_assert(WAVES_M * WAVES_N == 4 || WAVES_M * WAVES_N == 8, "4 or 8 waves per workgroup");
  static_assert(TM >= 1 && TN >= 2 && TN % 2 == 0, "wave tile shape");
};

struct TileLoc {
  int grp, e, rows, m_off, nt;
  int64_t row_begin;
};

// Locates this workgroup's tile.  Returns false for a surplus workgroup.
template <int BM>
__device__ __forceinline__ bool locate_tile(const GemmParams& p, int* s_loc, TileLoc& t) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int t4[4], o4[4], n4[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ex = lane * 4 + i;
      int n = 0, o = 0;
      if (p.offsets) {
        if (ex < p.E_loc) {
          o = p.offsets[ex];
          n = p.offsets[ex + 1] - o;
        }
      } else if (ex == 0) {
        n = static_cast<int>(p.dense_rows);
      }
      o4[i] = o;
      n4[i] = n;
      t4[i] = (n + BM - 1) / BM;
      sum += t4[i];
    }
    const int incl = wave_incl_scan(sum);
    const int total0 = __shfl(incl, 63, kWave);
    const int tiles0 = total0 * p.g[0].n_tiles;
    const int mt1 = static_cast<int>((p.rows1 + BM - 1) / BM);
    const int tiles1 = p.rows1 > 0 ? p.E1 * mt1 * p.g[1].n_tiles : 0;
    const int R = tiles1 + tiles0;
    const int per = (R + 7) / 8;
    const int b = blockIdx.x;
    const int L = (b & 7) * per + (b >> 3);
    const bool valid = (b >> 3) < per && L < R;
    if (lane == 0) {
      s_loc[0] = valid ? 1 : 0;
      if (valid && L < tiles1) {    // group 1: dense experts, expert-major
        const int per_e = mt1 * p.g[1].n_tiles;
        const int L1 = L % per_e;
        s_loc[1] = 1;
        s_loc[2] = L / per_e;
        s_loc[3] = L1 % mt1;
        s_loc[4] = L1 / mt1;
      }
    }
    if (valid && L >= tiles1) {
      // Expert e owns tiles [nt0 * rt_before(e), nt0 * rt_through(e)), row
      // tile fastest: the row tiles sharing a weight tile run back to back.
      const int L0 = L - tiles1;
      const int nt0 = p.g[0].n_tiles;
      const int excl = incl - sum;
      if (L0 >= excl * nt0 && L0 < incl * nt0) {
        int acc = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (L0 >= acc * nt0 && L0 < (acc + t4[i]) * nt0) {
            const int local = L0 - acc * nt0;
            s_loc[1] = 0;
            s_loc[2] = lane * 4 + i;
            s_loc[3] = local % t4[i];
            s_loc[4] = local / t4[i];
            s_loc[5] = o4[i];          // the expert's first row and row count, so
            s_loc[6] = n4[i];          // no workgroup reads the offsets twice
          }
          acc += t4[i];
        }
      }
    }
  }
  __syncthreads();
  if (!s_loc[0]) return false;
  t.grp = s_loc[1];
  t.e = s_loc[2];
  t.m_off = s_loc[3] * BM;
  t.nt = s_loc[4];
  if (t.grp == 1) {
    t.row_begin = 0;
    t.rows = static_cast<int>(p.rows1);
  } else if (p.offsets) {
    t.row_begin = s_loc[5];
    t.rows = s_loc[6];
  } else {
    t.row_begin = 0;
    t.rows = static_cast<int>(p.dense_rows);
  }
  return true;
}

// LDS row of weight tile row r -> weight row inside the expert's matrix
// (tiles of BN weight rows).
template <int MODE, int BN = kBN>
__device__ __forceinline__ int b_global_row(const GemmGroup& g, int nt, int r) {
  if constexpr (MODE == MODE_GATEUP) {
    return r < BN / 2 ? nt * (BN / 2) + r : g.N + nt * (BN / 2) + (r - BN / 2);
  } else if constexpr (MODE == MODE_ROUTER) {
    const int gr = nt * BN + r;
    return gr < g.N ? gr : g.N - 1;
  } else {
    return nt * BN + r;
  }
}

// First LDS weight row of the wave's tn-th 16-column MFMA tile.
template <int MODE, int WN, int TN, int BN = kBN>
__device__ __forceinline__ int b_lds_row(int wn, int tn) {
  if constexpr (MODE == MODE_GATEUP) {
    return tn < TN / 2 ? wn * (WN / 2) + tn * 16 : BN / 2 + wn * (WN / 2) + (tn - TN / 2) * 16;
  } else {
    return wn * WN + tn * 16;
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// First K stage of the tile with index `tile` (its stages are visited in the
// order start, start + 1, ..., KT - 1, 0, ..., start - 1).  Consecutive tiles
// start 5 stages apart.
__device__ __forceinline__ int rotation_start(int tile, int KT) {
  return KT > 1 ? static_cast<int>((static_cast<uint32_t>(tile) * 5u) % static_cast<uint32_t>(KT)) : 0;
}

__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = static_cast<__bf16>(a);     // v_cvt_pk_bf16_f32: round to nearest even
  v[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, v);
}

// 16 fp8 e4m3 codes -> 16 bf16 of (code value * s), one rounding each.
__device__ __forceinline__ void fp8x16_to_bf16x16(const u32x4_t& q, float s, u32x4_t& lo, u32x4_t& hi) {
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int v = static_cast<int>(q[w]);
    const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
    const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
    out[2 * w] = cvt_bf16x2(f01[0] * s, f01[1] * s);
    out[2 * w + 1] = cvt_bf16x2(f23[0] * s, f23[1] * s);
  }
  lo = u32x4_t{out[0], out[1], out[2], out[3]};
  hi = u32x4_t{out[4], out[5], out[6], out[7]};
}

// Epilogue of a tile: gate/up applies SiLU(gate) * up and rounds h to bf16;
// down rounds y to bf16; the router writes fp32 logits (+ bias).
// bf16 outputs go through LDS (`scratch`, the tile's free activation buffers,
// at least BM x BN bf16): each wave writes its block row-major with the
// 16-byte chunks of a row XOR-swizzled by the row, then reads it back 16 bytes
// per lane and stores whole 16-byte pieces of output rows.  An accumulator
// lane holds 4 rows of one column, so storing straight from the registers
// takes one 2-byte store per element (measured: the Qwen3-shaped down GEMM
// spent a quarter of its time on them).
template <int BM, int WAVES_M, int WAVES_N, int MODE, int BN>
__device__ __forceinline__ void store_tile(const GemmGroup& g, const TileLoc& t, const GemmParams& p,
                                           const f32x4_t (&acc)[TileShape<BM, WAVES_M, WAVES_N, BN>::TM]
                                                                [TileShape<BM, WAVES_M, WAVES_N, BN>::TN],
                                           bf16_t* scratch) {
  using S = TileShape<BM, WAVES_M, WAVES_N, BN>;
  constexpr int TM = S::TM, TN = S::TN, WM = S::WM, WN = S::WN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int nt = t.nt;
  const int col_in = lane & 15;
  const int row_q = (lane >> 4) * 4;
  if constexpr (MODE == MODE_ROUTER) {
    float* C = static_cast<float*>(g.C) + blockIdx.y * p.split_c;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int col = nt * BN + wn * WN + tn * 16 + col_in;
        if (col < g.N) {
          const float b = p.bias ? p.bias[col] : 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int mr = t.m_off + wm * WM + tm * 16 + row_q + r;
            if (mr < t.rows) C[(t.row_begin + mr) * g.ldc + col] = acc[tm][tn][r] + b;
          }
        }
      }
  } else {
    constexpr int OW = MODE == MODE_GATEUP ? WN / 2 : WN;     // output columns of a wave
    constexpr int OT = OW / 16;                                // 16-column MFMA tiles of it
    constexpr int CPR = OW / 8;                                // 16-byte chunks per output row
    static_assert(CPR >= 2 && (CPR & (CPR - 1)) == 0, "epilogue chunking");
    bf16_t* W = scratch + wave * WM * OW;
    auto woff = [](int r, int c) { return r * OW + (((c >> 3) ^ (r & (CPR - 1))) << 3) + (c & 7); };
    __syncthreads();                              // every wave is done reading the stage buffers
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < OT; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v;
          if constexpr (MODE == MODE_GATEUP)
            v = silu_f32(acc[tm][tn][r]) * acc[tm][tn + TN / 2][r];
          else
            v = acc[tm][tn][r];
          W[woff(tm * 16 + row_q + r, tn * 16 + col_in)] = f32_to_bf16(v);
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    bf16_t* C = static_cast<bf16_t*>(g.C) + t.e * g.c_estride;
    const int col0 = MODE == MODE_GATEUP ? nt * (BN / 2) + wn * OW : nt * BN + wn * OW;
#pragma unroll
    for (int i = 0; i < (WM * CPR + 63) / 64; ++i) {
      const int ch = lane + 64 * i;
      if (WM * CPR % 64 != 0 && ch >= WM * CPR) break;
      const int rr = ch / CPR, cc = ch % CPR;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&W[rr * OW + ((cc ^ (rr & (CPR - 1))) << 3)]);
      const int mr = t.m_off + wm * WM + rr;
      if (mr < t.rows)
        *reinterpret_cast<u32x4_t*>(&C[(t.row_begin + mr) * g.ldc + col0 + cc * 8]) = v;
    }
  }
}

template <int BM, int WAVES_M, int WAVES_N, int MODE, bool FP8, int BN, int BK>
__device__ __forceinline__ void gemm_tile(const GemmGroup& g, const TileLoc& t, const GemmParams& p,
                                          bf16_t (*sA)[BM * BK], bf16_t (*sB)[BN * BK]) {
  using S = TileShape<BM, WAVES_M, WAVES_N, BN>;
  constexpr int TM = S::TM, TN = S::TN, WM = S::WM, WN = S::WN;
  constexpr int CA = BM * (BK / 8) / 256;              // 16-byte A chunks per thread
  constexpr int CB = FP8 ? BN * (BK / 16) / 256        // 16-byte B chunks per thread
                         : BN * (BK / 8) / 256;
  static_assert(CA >= 1 && CB >= 1, "chunking");
  static_assert(!FP8 || 128 % BK == 0, "an fp8 stage must lie inside one 128-wide scale block");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int K = g.K;
  const int KT = K / BK;
  // With 32-row tiles (decode: the GEMM streams weights) each column tile
  // walks K from its own starting stage, wrapping around: tiles that stream
  // their weights at the same K offset at the same time hit the same HBM
  // channels.  Measured with 1408 tiles reading 128 bytes of each of 128 rows
  // per step: 4.46 TB/s in lockstep, 5.54 TB/s rotated; decode gate/up
  // 157.7 -> 150.8 us.  Larger row tiles share activation tiles across column
  // tiles through L2 and ran 1-4 % slower rotated, so they keep K in order.
  const int kt_rot = BM <= 32 ? __builtin_amdgcn_readfirstlane(rotation_start(t.e * g.n_tiles + t.nt, KT)) : 0;
  const int64_t ksplit = static_cast<int64_t>(blockIdx.y) * K;   // 0 unless router split-K
  const int nt = t.nt;

  // Global source addresses of this thread's chunks (K offset added per stage).
  const bf16_t* a_src[CA];
  int a_lds[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + i * 256;
    const int r = c / (BK / 8);
    const int kc = c % (BK / 8);
    int mr = t.m_off + r;
    mr = mr < t.rows ? mr : t.rows - 1;
    a_src[i] = g.A + t.e * g.a_estride + (t.row_begin + mr) * g.lda + ksplit + kc * 8;
    a_lds[i] = lds_off_k<BK>(r, kc);
  }
  const size_t expert_elems = static_cast<size_t>(g.b_estride);
  const uint8_t* b_src[CB];
  int b_lds[CB], b_lds2[CB];
  bool b_up[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + i * 256;
    const int r = FP8 ? c / (BK / 16) : c / (BK / 8);
    const int kc = FP8 ? c % (BK / 16) : c % (BK / 8);
    const int gr = b_global_row<MODE, BN>(g, nt, r);
    b_up[i] = r >= BN / 2;
    if constexpr (FP8) {
      b_src[i] = static_cast<const uint8_t*>(g.B) + static_cast<size_t>(t.e) * expert_elems +
                 static_cast<size_t>(gr) * g.ldb + ksplit + kc * 16;
      b_lds[i] = lds_off_k<BK>(r, 2 * kc);          // 16 fp8 codes -> two 8-element bf16 chunks
      b_lds2[i] = lds_off_k<BK>(r, 2 * kc + 1);
    } else {
      b_src[i] = reinterpret_cast<const uint8_t*>(static_cast<const bf16_t*>(g.B) +
                                                  static_cast<size_t>(t.e) * expert_elems +
                                                  static_cast<size_t>(gr) * g.ldb + ksplit + kc * 8);
      b_lds[i] = lds_off_k<BK>(r, kc);
      b_lds2[i] = b_lds[i];
    }
  }
  // fp8 scale rows of this column tile (gate rows / up rows, or the one row block)
  const float* srow0 = nullptr;
  const float* srow1 = nullptr;
  if constexpr (FP8) {
    const int kblocks = K / 128;
    const float* se = g.bscale + static_cast<size_t>(t.e) * (g.b_rows / 128) * kblocks;
    if constexpr (MODE == MODE_GATEUP) {
      srow0 = se + static_cast<size_t>((nt * (BN / 2)) / 128) * kblocks;
      srow1 = se + static_cast<size_t>((g.N + nt * (BN / 2)) / 128) * kblocks;
    } else {
      srow0 = se + static_cast<size_t>((nt * BN) / 128) * kblocks;
      srow1 = srow0;
    }
  }

  // fp8: the two scale rows, one K block per lane (lane l holds blocks l and
  // l + 64), picked per stage with v_readlane.  A scalar memory load inside the
  // K loop would share its completion counter with the LDS reads, so every
  // wait for an LDS read would also wait for the scale load in flight.
  float scv[2][2] = {{1.f, 1.f}, {1.f, 1.f}};
  if constexpr (FP8) {
    const int kblocks = K / 128;
    const int lane_l = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float* row = j == 0 ? srow0 : srow1;
      scv[j][0] = row[min(lane_l, kblocks - 1)];
      scv[j][1] = row[min(lane_l + 64, kblocks - 1)];
    }
  }
  u32x4_t ra0[CA], rb0[CB], ra1[CA], rb1[CB];
  float sc0[2] = {1.f, 1.f}, sc1[2] = {1.f, 1.f};
  auto load_stage = [&](int kt, u32x4_t* ra, u32x4_t* rb, float* sc) {
    int ks = kt + kt_rot;
    ks = ks >= KT ? ks - KT : ks;
    const int k0 = ks * BK;
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const size_t kb = FP8 ? static_cast<size_t>(k0) : static_cast<size_t>(k0) * 2;
      rb[i] = *reinterpret_cast<const u32x4_t*>(b_src[i] + kb);
    }
    if constexpr (FP8) {
      const int blk = k0 / 128;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float v = blk < 64 ? scv[j][0] : scv[j][1];
        sc[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), blk & 63));
      }
    }
  };
  auto store_stage = [&](int buf, const u32x4_t* ra, const u32x4_t* rb, const float* sc) {
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4_t*>(&sA[buf][a_lds[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      if constexpr (FP8) {
        u32x4_t lo, hi;
        fp8x16_to_bf16x16(rb[i], (MODE == MODE_GATEUP && b_up[i]) ? sc[1] : sc[0], lo, hi);
        *reinterpret_cast<u32x4_t*>(&sB[buf][b_lds[i]]) = lo;
        *reinterpret_cast<u32x4_t*>(&sB[buf][b_lds2[i]]) = hi;
      } else {
        *reinterpret_cast<u32x4_t*>(&sB[buf][b_lds[i]]) = rb[i];
      }
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int frag_row = lane & 15;
  const int frag_c = lane >> 4;             // 16-byte chunk within the 32-wide K step
  // 16-row subtiles of this wave that hold rows of the expert: the last row
  // tile of an expert is usually partial, and its empty subtiles skip their
  // LDS reads and MFMAs (a wave-uniform count).
  const int tm_valid = __builtin_amdgcn_readfirstlane(
      max(0, min(TM, (t.rows - t.m_off - wm * WM + 15) / 16)));
  auto compute_stage = [&](int buf) {
    if (tm_valid == 0) return;            // no rows for this wave in this tile
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      bf16x8_t af[TM], bfv[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        if (tm < tm_valid)
          af[tm] = *reinterpret_cast<const bf16x8_t*>(
              &sA[buf][lds_off_k<BK>(wm * WM + tm * 16 + frag_row, kk * 4 + frag_c)]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        bfv[tn] = *reinterpret_cast<const bf16x8_t*>(
            &sB[buf][lds_off_k<BK>(b_lds_row<MODE, WN, TN, BN>(wn, tn) + frag_row, kk * 4 + frag_c)]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        if (tm < tm_valid)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], bfv[tn], acc[tm][tn], 0, 0, 0);
    }
  };

  // Two-deep register ring: stage s is loaded into ring slot s % 2 two stages
  // before its MFMAs and stored to LDS buffer s % 2 one stage before them.
  // The steady-state loop issues its loads unconditionally (the last stages
  // are peeled), and scheduling barriers keep them ahead of the MFMAs: with a
  // conditional or sunk load the compiler's wait for one stage also waits for
  // the stage issued after it, and the ring degenerates to one stage.
  load_stage(0, ra0, rb0, sc0);
  if (KT > 1) load_stage(1, ra1, rb1, sc1);
  store_stage(0, ra0, rb0, sc0);
  __syncthreads();
  int kt = 0;
  // A wave whose row subtiles all hold rows (every wave of a full row tile)
  // runs the steady state without the per-subtile branches, so the stage is
  // one basic block the compiler schedules as a whole (prefill gate/up
  // 402 -> 379 us standalone, bitwise equal).  Both loops run the same
  // barriers, so waves of one workgroup may take different ones.
  auto compute_full = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      bf16x8_t af[TM], bfv[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        af[tm] = *reinterpret_cast<const bf16x8_t*>(
            &sA[buf][lds_off_k<BK>(wm * WM + tm * 16 + frag_row, kk * 4 + frag_c)]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        bfv[tn] = *reinterpret_cast<const bf16x8_t*>(
            &sB[buf][lds_off_k<BK>(b_lds_row<MODE, WN, TN, BN>(wn, tn) + frag_row, kk * 4 + frag_c)]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], bfv[tn], acc[tm][tn], 0, 0, 0);
    }
  };
  if (tm_valid == TM) {
    for (; kt + 3 < KT; kt += 2) {
      load_stage(kt + 2, ra0, rb0, sc0);
      __builtin_amdgcn_sched_barrier(0);
      compute_full(0);
      store_stage(1, ra1, rb1, sc1);
      __syncthreads();
      load_stage(kt + 3, ra1, rb1, sc1);
      __builtin_amdgcn_sched_barrier(0);
      compute_full(1);
      store_stage(0, ra0, rb0, sc0);
      __syncthreads();
    }
  } else {
    for (; kt + 3 < KT; kt += 2) {
      load_stage(kt + 2, ra0, rb0, sc0);
      __builtin_amdgcn_sched_barrier(0);
      compute_stage(0);
      store_stage(1, ra1, rb1, sc1);
      __syncthreads();
      load_stage(kt + 3, ra1, rb1, sc1);
      __builtin_amdgcn_sched_barrier(0);
      compute_stage(1);
      store_stage(0, ra0, rb0, sc0);
      __syncthreads();
    }
  }
  const int left = KT - kt;                 // 1, 2 or 3 stages; stage kt is in LDS buffer 0
  if (left == 3) {
    load_stage(kt + 2, ra0, rb0, sc0);
    __builtin_amdgcn_sched_barrier(0);
    compute_stage(0);
    store_stage(1, ra1, rb1, sc1);
    __syncthreads();
    compute_stage(1);
    store_stage(0, ra0, rb0, sc0);
    __syncthreads();
    compute_stage(0);
  } else if (left == 2) {
    compute_stage(0);
    store_stage(1, ra1, rb1, sc1);
    __syncthreads();
    compute_stage(1);
  } else {
    compute_stage(0);
  }

  store_tile<BM, WAVES_M, WAVES_N, MODE, BN>(g, t, p, acc, &sA[0][0]);
}

// One LDS DMA (global_load_lds_dwordx4): each lane's 16 bytes land at
// lds_addr + 16 * lane, so one wave instruction fills 1 KB of LDS.  Written as
// inline assembly with its completion counted by hand (s_waitcnt vmcnt): the
// compiler's own accounting would wait for every DMA in flight before any
// LDS read.  No register is written, so nothing the compiler owns is in flight.
__device__ __forceinline__ void lds_dma16(uint32_t lds_addr, const void* gptr) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(a), "v"(gptr) : "memory");
}

// s_waitcnt vmcnt(N): vmcnt is 6 bits, its low 4 in bits 3:0 and its high 2
// in bits 15:14; expcnt (6:4) and lgkmcnt (11:8) at their maxima, not waited for.
// One 4-byte LDS DMA (global_load_lds_dword): lane l's word lands at
// lds_addr + 4 * lane.
__device__ __forceinline__ void lds_dma4(uint32_t lds_addr, const void* gptr) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(a), "v"(gptr) : "memory");
}

template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}

// Waits until at most n stages of this wave's DMAs (NDMA each) are in flight.
template <int NDMA, int MAXN>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) {
      wait_vmcnt<MAXN * NDMA>();
      return;
    }
    wait_stages<NDMA, MAXN - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// gemm_tile with both operands staged by LDS DMA (bf16 activations and bf16
// weights): no register ring and no LDS stores sit on the load path.  A
// synthetic stage probe on MI355X (128 x 128 tile, 64-wide K stages, two
// workgroups per CU, L2-resident data) ran 1.05-1.16 PFLOP/s with register
// staging and LDS stores and 1.41-1.52 PFLOP/s with DMA staging.  The same
// arithmetic as gemm_tile, so the outputs are bitwise equal.
// A stage is BK wide (CPR = BK / 8 16-byte chunks per row); each DMA fills
// 64 / CPR rows: lane l carries row R = first row + l / CPR and that row's
// chunk (l % CPR) ^ (R & 7), so the chunks land in the XOR-swizzled order
// the fragment reads expect.  Ring of NBUF stages (stage kt in buffer kt % NBUF):
// stage kt issues stage kt + NBUF - 1 into the buffer stage kt - 1 used,
// computes, waits for this wave's DMAs of stage kt + 1 and meets the others
// at the barrier.  ROT: each weight tile walks K from its own starting stage
// (the 32-row decode tiles, as gemm_tile does).
template <int BM, int BN, int BK, int NBUF> struct DmaLds {
  static constexpr int A = BM * BK * 2, B = BN * BK * 2, bytes = NBUF * (A + B);
};

template <int MODE, int BM, int BN, int BK, int NBUF, bool ROT, int WAVES_N = 2>
__device__ __forceinline__ void gemm_tile_dma(const GemmGroup& g, const TileLoc& t, const GemmParams& p,
                                              uint8_t* lds) {
  constexpr int WAVES_M = 2, NW = WAVES_M * WAVES_N;
  using S = TileShape<BM, WAVES_M, WAVES_N, BN>;
  constexpr int TM = S::TM, TN = S::TN, WM = S::WM, WN = S::WN;
  constexpr int CPR = BK / 8, RPD = 64 / CPR;              // chunks per row, rows per DMA
  constexpr int NQA = BM / RPD / NW, NQB = BN / RPD / NW;  // DMAs per wave per stage
  constexpr int NDMA = NQA + NQB;
  constexpr int A_BYTES = DmaLds<BM, BN, BK, NBUF>::A, B_BYTES = DmaLds<BM, BN, BK, NBUF>::B;
  static_assert(NQA >= 1 && NQB >= 1 && NQA * NW * RPD == BM && NQB * NW * RPD == BN, "DMA split");
  static_assert(NBUF >= 2 && (NBUF - 2) * NDMA < 64, "ring");
  static_assert(NW * WM * (MODE == MODE_GATEUP ? WN / 2 : WN) * 2 <= NBUF * A_BYTES, "epilogue scratch");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int K = g.K, KT = K / BK, nt = t.nt;
  const int kt_rot = ROT ? __builtin_amdgcn_readfirstlane(rotation_start(t.e * g.n_tiles + t.nt, KT)) : 0;

  uint8_t* sA = lds;
  uint8_t* sB = lds + NBUF * A_BYTES;
  const uint32_t lds_a = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(lds)));
  const uint32_t lds_b = lds_a + NBUF * A_BYTES;

  // the swizzle takes the tile row R (a DMA's first row is a multiple of RPD,
  // which is not a multiple of 8 for 128-wide stages)
  const int lrow = lane / CPR, lpos = lane % CPR;
  const bf16_t* a_src[NQA];
  const bf16_t* b_src[NQB];
#pragma unroll
  for (int i = 0; i < NQA; ++i) {
    const int R = RPD * (wave * NQA + i) + lrow;
    int mr = t.m_off + R;
    mr = mr < t.rows ? mr : t.rows - 1;
    a_src[i] = g.A + t.e * g.a_estride + (t.row_begin + mr) * g.lda + (lpos ^ (R & 7)) * 8;
  }
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const int R = RPD * (wave * NQB + i) + lrow;
    b_src[i] = static_cast<const bf16_t*>(g.B) + static_cast<size_t>(t.e) * g.b_estride +
               static_cast<size_t>(b_global_row<MODE, BN>(g, nt, R)) * g.ldb + (lpos ^ (R & 7)) * 8;
  }
  __builtin_amdgcn_s_waitcnt(0);     // only hand-counted DMAs in flight from here
  auto issue = [&](int kt) {
    int ks = kt + kt_rot;
    ks = ks >= KT ? ks - KT : ks;
    const int k0 = ks * BK, buf = kt % NBUF;
#pragma unroll
    for (int i = 0; i < NQA; ++i) lds_dma16(lds_a + buf * A_BYTES + (wave * NQA + i) * 1024, a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < NQB; ++i) lds_dma16(lds_b + buf * B_BYTES + (wave * NQB + i) * 1024, b_src[i] + k0);
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int frag_row = lane & 15, frag_c = lane >> 4;
  const int tm_valid = __builtin_amdgcn_readfirstlane(
      max(0, min(TM, (t.rows - t.m_off - wm * WM + 15) / 16)));
  auto compute = [&](int kt, auto full) {
    if (!decltype(full)::value && tm_valid == 0) return;   // no rows for this wave
    const bf16_t* A = reinterpret_cast<const bf16_t*>(sA + (kt % NBUF) * A_BYTES);
    const bf16_t* B = reinterpret_cast<const bf16_t*>(sB + (kt % NBUF) * B_BYTES);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      bf16x8_t af[TM], bfv[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        if (decltype(full)::value || tm < tm_valid)
          af[tm] = *reinterpret_cast<const bf16x8_t*>(&A[lds_off_k<BK>(wm * WM + tm * 16 + frag_row, kk * 4 + frag_c)]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        bfv[tn] = *reinterpret_cast<const bf16x8_t*>(
            &B[lds_off_k<BK>(b_lds_row<MODE, WN, TN, BN>(wn, tn) + frag_row, kk * 4 + frag_c)]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        if (decltype(full)::value || tm < tm_valid)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], bfv[tn], acc[tm][tn], 0, 0, 0);
    }
  };

  const int pre = min(NBUF - 1, KT);
  for (int s = 0; s < pre; ++s) issue(s);
  wait_stages<NDMA, NBUF - 2>(pre - 1);
  __syncthreads();
  auto stage = [&](int kt, auto full) {
    if (kt + NBUF - 1 < KT) issue(kt + NBUF - 1);
    compute(kt, full);
    wait_stages<NDMA, NBUF - 2>(min(KT - 1, kt + NBUF - 1) - (kt + 1));
    __syncthreads();
  };
  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;
  if (tm_valid == TM) {
    for (int kt = 0; kt < KT; ++kt) stage(kt, Full{});
  } else {
    for (int kt = 0; kt < KT; ++kt) stage(kt, Part{});
  }
  store_tile<BM, WAVES_M, WAVES_N, MODE, BN>(g, t, p, acc, reinterpret_cast<bf16_t*>(sA));
}

// Waves per SIMD each tile shape is built for: 4 for the 32-row tile with
// 64-wide K stages (24 KB of LDS), 3 with 128-wide stages (48 KB: three
// workgroups share a CU), 3 for 64 rows, 2 for 128 rows.
template <int BM, int BK> struct MinWaves {
  static constexpr int value = BM == 32 ? (BK == 64 ? 4 : 3) : BM == 64 ? 3 : 2;
};

template <int BM, int WAVES_M, int WAVES_N, int MODE, bool FP8, int BN = kBN, int BK = kBK>
__global__ __launch_bounds__(256, (MinWaves<BM, BK>::value)) void k_gemm_nt(GemmParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * BK];
  int* s_loc = reinterpret_cast<int*>(&sA[0][0]);   // tile location, before sA holds A tiles
  TileLoc t;
  if (!locate_tile<BM>(p, s_loc, t)) return;
  __syncthreads();                                  // s_loc read by all before sA is filled
  if (FP8 && t.grp == 0)
    gemm_tile<BM, WAVES_M, WAVES_N, MODE, FP8, BN, BK>(p.g[0], t, p, sA, sB);
  else
    gemm_tile<BM, WAVES_M, WAVES_N, MODE, false, BN, BK>(p.g[t.grp], t, p, sA, sB);
}

// bf16 tiles with DMA staging; both groups (a dense group of shared experts
// runs through the same tile).  2 x WAVES_N waves (MINW: waves per SIMD).
template <int MODE, int BM = 128, int BN = kBN, int BK = kBK, int NBUF = 2, bool ROT = false, int MINW = 2,
          int WAVES_N = 2>
__global__ __launch_bounds__(2 * WAVES_N * 64, MINW) void k_gemm_dma(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[DmaLds<BM, BN, BK, NBUF>::bytes];
  int* s_loc = reinterpret_cast<int*>(lds);
  TileLoc t;
  if (!locate_tile<BM>(p, s_loc, t)) return;
  __syncthreads();                                  // s_loc read by all before the ring is filled
  gemm_tile_dma<MODE, BM, BN, BK, NBUF, ROT, WAVES_N>(p.g[t.grp], t, p, lds);
}

// Worst-case number of row tiles: sum_e ceil(n_e / BM) <= ceil(cap / BM) + E_loc.
inline int64_t max_row_tiles(int64_t cap_rows, int E_loc, int BM, bool dense) {
  if (dense) return (cap_rows + BM - 1) / BM;
  return (cap_rows + BM - 1) / BM + E_loc;
}

inline int64_t gemm_grid(int64_t tiles) { return (tiles + 7) / 8 * 8; }

// fp32 SIMT variant of the same tiling (fp32 activations and weights only, one
// group per launch): 32 rows x 128 weight rows per workgroup, K staged 32 at a
// time through LDS, each thread owns 2 rows x 8 columns (gate/up: 2 rows x 4
// gate + 4 up columns).
template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_nt_f32(GemmParams p) {
  constexpr int BM = 32, BKF = 32;
  __shared__ float sA[BM][BKF + 1];
  __shared__ float sB[kBN][BKF + 1];
  __shared__ int s_loc[8];
  TileLoc t;
  if (!locate_tile<BM>(p, s_loc, t)) return;
  const GemmGroup& g = p.g[0];

  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t ksplit = static_cast<int64_t>(blockIdx.y) * g.K;
  const float* A = reinterpret_cast<const float*>(g.A) + ksplit;
  const float* B = static_cast<const float*>(g.B) + static_cast<size_t>(t.e) * g.b_estride + ksplit;
  float acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < g.K; k0 += BKF) {
#pragma unroll
    for (int i = 0; i < BM * BKF / 256; ++i) {
      const int c = tid + i * 256;
      const int r = c / BKF, kc = c % BKF;
      int mr = t.m_off + r;
      mr = mr < t.rows ? mr : t.rows - 1;
      sA[r][kc] = A[(t.row_begin + mr) * g.lda + k0 + kc];
    }
#pragma unroll
    for (int i = 0; i < kBN * BKF / 256; ++i) {
      const int c = tid + i * 256;
      const int r = c / BKF, kc = c % BKF;
      sB[r][kc] = B[static_cast<size_t>(b_global_row<MODE>(g, t.nt, r)) * g.ldb + k0 + kc];
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < BKF; ++kk) {
      const float a0 = sA[ty][kk], a1 = sA[ty + 16][kk];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // gate/up: j < 4 -> gate rows tx+16j, j >= 4 -> the matching up rows
        const int br = (MODE == MODE_GATEUP) ? (j < 4 ? tx + 16 * j : kBN / 2 + tx + 16 * (j - 4))
                                             : tx + 16 * j;
        const float b = sB[br][kk];
        acc[0][j] += a0 * b;
        acc[1][j] += a1 * b;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int mr = t.m_off + ty + 16 * i;
    if (mr >= t.rows) continue;
    float* C = static_cast<float*>(g.C) + blockIdx.y * p.split_c + (t.row_begin + mr) * g.ldc;
    if constexpr (MODE == MODE_GATEUP) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gt = acc[i][j], u = acc[i][j + 4];
        C[t.nt * (kBN / 2) + tx + 16 * j] = gt / (1.0f + expf(-gt)) * u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = t.nt * kBN + tx + 16 * j;
        if (MODE == MODE_ROUTER && col >= g.N) continue;
        C[col] = acc[i][j] + ((MODE == MODE_ROUTER && p.bias) ? p.bias[col] : 0.f);
      }
    }
  }
}

}  // namespace dbomoe
