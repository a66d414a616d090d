// LDS-tiled bf16 MFMA "NT" GEMM for gfx950, shared by the router logits and the
// two grouped expert GEMMs.  C[m, n] = sum_k A[m, k] * B[n, k]: both operands
// are K-contiguous rows, which is how activations ([rows, H]) and the expert
// weights ([2I, H] and [H, I]) are stored, so no operand is ever transposed.
//
// Work decomposition
//  * Row tiles of BM rows per expert (the grouped GEMM's "M tiles"), column
//    tiles of BN = 128 weight rows; for the gate/up GEMM a column tile holds 64
//    gate rows and the 64 matching up rows, so SwiGLU is applied in registers.
//  * Per-expert row counts are on the device: every workgroup rebuilds the
//    tile map from `offsets` with one wave prefix scan, so the host launches a
//    worst-case grid and surplus workgroups exit at once.
//  * Workgroup b runs on XCD b % 8; the logical tile index is remapped so each
//    XCD walks a contiguous run of tiles (column tiles of one row tile, then the
//    next row tile of the same expert), keeping the A rows and the weight tile a
//    neighbour needs in that XCD's L2.
//  * 4 waves; each wave owns a WM x WN block made of 16x16 MFMA tiles
//    (v_mfma_f32_16x16x32_bf16, fp32 accumulators).  K advances 64 per stage;
//    global loads for stage k+1 are issued before the MFMAs of stage k and land
//    in the other half of a double-buffered LDS tile (one barrier per stage).
//  * fp8 e4m3 weights are converted to bf16 once per workgroup on their way to
//    LDS (exact: every e4m3 value is a bf16 value); the per-128x128-block fp32
//    scale multiplies the fp32 partial sum of each 128-wide K block.
#pragma once

#include "common.h"

namespace dbomoe {

constexpr int kBK = 64;                  // K elements per LDS stage
constexpr int kLdsStride = kBK + 8;      // bf16 elements per LDS row (16 B pad: spreads banks)
constexpr int kBN = 128;                 // weight rows per column tile

enum GemmMode { MODE_ROUTER = 0, MODE_GATEUP = 1, MODE_DOWN = 2 };

struct GemmParams {
  const bf16_t* A;        // activation rows
  int64_t lda;            // elements between rows of A
  const void* B;          // [E_loc][b_rows][ldb] bf16 or fp8 codes
  int64_t ldb;            // elements between weight rows
  const float* bscale;    // fp8: [E_loc][b_rows/128][K/128]
  int K;                  // reduction length (multiple of 64; of 128 for fp8)
  int N;                  // output columns: E (router), I (gate/up), H (down)
  int b_rows;             // weight rows per expert
  const int32_t* offsets; // [E_loc+1] or NULL (dense: one expert with dense_rows rows)
  int E_loc;
  int64_t dense_rows;
  void* C;                // output rows (fp32 for the router, bf16 otherwise)
  int64_t ldc;
  const float* bias;      // logit bias or NULL (router without split-K only)
  int n_tiles;            // column tiles
  int64_t split_c;        // router split-K: blockIdx.y selects K range [y*K, (y+1)*K)
                          // and output slab C + y*split_c
};

template <int BM, int WAVES_M, int WAVES_N>
struct TileShape {
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = kBN / WAVES_N;
  static constexpr int TM = WM / 16;
  static constexpr int TN = WN / 16;
  static_assert(WAVES_M * WAVES_N == 4, "4 waves per workgroup");
  static_assert(TM >= 1 && TN >= 2 && TN % 2 == 0, "wave tile shape");
};

// Locates this workgroup's tile.  Returns false for a surplus workgroup.
template <int BM>
__device__ __forceinline__ bool locate_tile(const GemmParams& p, int* s_loc, int& e, int64_t& row_begin,
                                            int& rows, int& m_off, int& nt) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int t4[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ex = lane * 4 + i;
      int n = 0;
      if (p.offsets) {
        if (ex < p.E_loc) n = p.offsets[ex + 1] - p.offsets[ex];
      } else if (ex == 0) {
        n = static_cast<int>(p.dense_rows);
      }
      t4[i] = (n + BM - 1) / BM;
      sum += t4[i];
    }
    const int incl = wave_incl_scan(sum);
    const int total = __shfl(incl, 63, kWave);
    const int R = total * p.n_tiles;
    const int per = (R + 7) / 8;
    const int b = blockIdx.x;
    const int L = (b & 7) * per + (b >> 3);
    const bool valid = (b >> 3) < per && L < R;
    if (lane == 0) s_loc[0] = valid ? 1 : 0;
    if (valid) {
      const int mt = L / p.n_tiles;
      const int excl = incl - sum;
      if (mt >= excl && mt < incl) {
        int acc = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (mt >= acc && mt < acc + t4[i]) {
            const int ex = lane * 4 + i;
            s_loc[1] = ex;
            s_loc[2] = mt - acc;
            s_loc[3] = L % p.n_tiles;
          }
          acc += t4[i];
        }
      }
    }
  }
  __syncthreads();
  if (!s_loc[0]) return false;
  e = s_loc[1];
  m_off = s_loc[2] * BM;
  nt = s_loc[3];
  if (p.offsets) {
    row_begin = p.offsets[e];
    rows = p.offsets[e + 1] - p.offsets[e];
  } else {
    row_begin = 0;
    rows = static_cast<int>(p.dense_rows);
  }
  return true;
}

// LDS row of weight tile row r -> weight row inside the expert's matrix.
template <int MODE>
__device__ __forceinline__ int b_global_row(const GemmParams& p, int nt, int r) {
  if constexpr (MODE == MODE_GATEUP) {
    return r < kBN / 2 ? nt * (kBN / 2) + r : p.N + nt * (kBN / 2) + (r - kBN / 2);
  } else if constexpr (MODE == MODE_ROUTER) {
    const int g = nt * kBN + r;
    return g < p.N ? g : p.N - 1;
  } else {
    return nt * kBN + r;
  }
}

// First LDS weight row of the wave's tn-th 16-column MFMA tile.
template <int MODE, int WN, int TN>
__device__ __forceinline__ int b_lds_row(int wn, int tn) {
  if constexpr (MODE == MODE_GATEUP) {
    return tn < TN / 2 ? wn * (WN / 2) + tn * 16 : kBN / 2 + wn * (WN / 2) + (tn - TN / 2) * 16;
  } else {
    return wn * WN + tn * 16;
  }
}

__device__ __forceinline__ void fp8x16_to_bf16x16(const u32x4_t& q, u32x4_t& lo, u32x4_t& hi) {
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int v = static_cast<int>(q[w]);
    const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
    const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
    out[2 * w] = __builtin_amdgcn_perm(__float_as_uint(f01[1]), __float_as_uint(f01[0]), 0x07060302u);
    out[2 * w + 1] = __builtin_amdgcn_perm(__float_as_uint(f23[1]), __float_as_uint(f23[0]), 0x07060302u);
  }
  lo = u32x4_t{out[0], out[1], out[2], out[3]};
  hi = u32x4_t{out[4], out[5], out[6], out[7]};
}

template <int BM, int WAVES_M, int WAVES_N, int MODE, bool FP8>
__global__ __launch_bounds__(256) void k_gemm_nt(GemmParams p) {
  using S = TileShape<BM, WAVES_M, WAVES_N>;
  constexpr int TM = S::TM, TN = S::TN, WM = S::WM, WN = S::WN;
  constexpr int CA = BM * (kBK / 8) / 256;              // 16-byte A chunks per thread
  constexpr int CB = FP8 ? kBN * (kBK / 16) / 256       // 16-byte B chunks per thread
                         : kBN * (kBK / 8) / 256;
  static_assert(CA >= 1 && CB >= 1, "chunking");

  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * kLdsStride];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][kBN * kLdsStride];
  __shared__ int s_loc[4];

  int e, rows, m_off, nt;
  int64_t row_begin;
  if (!locate_tile<BM>(p, s_loc, e, row_begin, rows, m_off, nt)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int K = p.K;
  const int KT = K / kBK;
  const int64_t ksplit = static_cast<int64_t>(blockIdx.y) * K;   // 0 unless router split-K

  // Global source addresses of this thread's chunks (K offset added per stage).
  const bf16_t* a_src[CA];
  int a_lds[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + i * 256;
    const int r = c / (kBK / 8);
    const int kc = c % (kBK / 8);
    int mr = m_off + r;
    mr = mr < rows ? mr : rows - 1;
    a_src[i] = p.A + (row_begin + mr) * p.lda + ksplit + kc * 8;
    a_lds[i] = r * kLdsStride + kc * 8;
  }
  const size_t expert_elems = static_cast<size_t>(p.b_rows) * p.ldb;
  const uint8_t* b_src[CB];
  int b_lds[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + i * 256;
    if constexpr (FP8) {
      const int r = c / (kBK / 16);
      const int kc = c % (kBK / 16);
      const int gr = b_global_row<MODE>(p, nt, r);
      b_src[i] = static_cast<const uint8_t*>(p.B) + static_cast<size_t>(e) * expert_elems +
                 static_cast<size_t>(gr) * p.ldb + ksplit + kc * 16;
      b_lds[i] = r * kLdsStride + kc * 16;
    } else {
      const int r = c / (kBK / 8);
      const int kc = c % (kBK / 8);
      const int gr = b_global_row<MODE>(p, nt, r);
      b_src[i] = reinterpret_cast<const uint8_t*>(static_cast<const bf16_t*>(p.B) +
                                                  static_cast<size_t>(e) * expert_elems +
                                                  static_cast<size_t>(gr) * p.ldb + ksplit + kc * 8);
      b_lds[i] = r * kLdsStride + kc * 8;
    }
  }

  u32x4_t ra[CA], rb[CB];
  auto load_stage = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const size_t kb = FP8 ? static_cast<size_t>(k0) : static_cast<size_t>(k0) * 2;
      rb[i] = *reinterpret_cast<const u32x4_t*>(b_src[i] + kb);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4_t*>(&sA[buf][a_lds[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      if constexpr (FP8) {
        u32x4_t lo, hi;
        fp8x16_to_bf16x16(rb[i], lo, hi);
        *reinterpret_cast<u32x4_t*>(&sB[buf][b_lds[i]]) = lo;
        *reinterpret_cast<u32x4_t*>(&sB[buf][b_lds[i] + 8]) = hi;
      } else {
        *reinterpret_cast<u32x4_t*>(&sB[buf][b_lds[i]]) = rb[i];
      }
    }
  };

  f32x4_t acc[TM][TN];
  f32x4_t part[FP8 ? TM : 1][FP8 ? TN : 1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (FP8) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) part[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // fp8 scale rows of this column tile
  const float* srow0 = nullptr;
  const float* srow1 = nullptr;
  if constexpr (FP8) {
    const int kblocks = K / 128;
    const float* se = p.bscale + static_cast<size_t>(e) * (p.b_rows / 128) * kblocks;
    if constexpr (MODE == MODE_GATEUP) {
      srow0 = se + static_cast<size_t>((nt * (kBN / 2)) / 128) * kblocks;
      srow1 = se + static_cast<size_t>((p.N + nt * (kBN / 2)) / 128) * kblocks;
    } else {
      srow0 = se + static_cast<size_t>((nt * kBN) / 128) * kblocks;
      srow1 = srow0;
    }
  }

  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int frag_row = lane & 15;
  const int frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_stage(kt + 1);
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      bf16x8_t af[TM], bfv[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        af[tm] = *reinterpret_cast<const bf16x8_t*>(
            &sA[cur][(wm * WM + tm * 16 + frag_row) * kLdsStride + kk * 32 + frag_k]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        bfv[tn] = *reinterpret_cast<const bf16x8_t*>(
            &sB[cur][(b_lds_row<MODE, WN, TN>(wn, tn) + frag_row) * kLdsStride + kk * 32 + frag_k]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          if constexpr (FP8)
            part[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], bfv[tn], part[tm][tn], 0, 0, 0);
          else
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], bfv[tn], acc[tm][tn], 0, 0, 0);
        }
    }
    if constexpr (FP8) {
      if (kt & 1) {
        const int kb = kt >> 1;
        const float s0 = srow0[kb];
        const float s1 = srow1[kb];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            const float s = (MODE == MODE_GATEUP && tn >= TN / 2) ? s1 : s0;
            acc[tm][tn] += s * part[tm][tn];
            part[tm][tn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
      }
    }
    if (kt + 1 < KT) store_stage(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator element r of lane l in a 16x16 tile is
  // (row 4*(l/16) + r, column l%16).
  const int col_in = lane & 15;
  const int row_q = (lane >> 4) * 4;
  if constexpr (MODE == MODE_GATEUP) {
    bf16_t* C = static_cast<bf16_t*>(p.C);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN / 2; ++tn) {
        const int col = nt * (kBN / 2) + wn * (WN / 2) + tn * 16 + col_in;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mr = m_off + wm * WM + tm * 16 + row_q + r;
          if (mr < rows) {
            const float g = acc[tm][tn][r];
            const float u = acc[tm][tn + TN / 2][r];
            C[(row_begin + mr) * p.ldc + col] = f32_to_bf16(silu_f32(g) * u);
          }
        }
      }
  } else if constexpr (MODE == MODE_DOWN) {
    bf16_t* C = static_cast<bf16_t*>(p.C);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int col = nt * kBN + wn * WN + tn * 16 + col_in;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mr = m_off + wm * WM + tm * 16 + row_q + r;
          if (mr < rows) C[(row_begin + mr) * p.ldc + col] = f32_to_bf16(acc[tm][tn][r]);
        }
      }
  } else {
    float* C = static_cast<float*>(p.C) + blockIdx.y * p.split_c;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int col = nt * kBN + wn * WN + tn * 16 + col_in;
        if (col < p.N) {
          const float b = p.bias ? p.bias[col] : 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int mr = m_off + wm * WM + tm * 16 + row_q + r;
            if (mr < rows) C[(row_begin + mr) * p.ldc + col] = acc[tm][tn][r] + b;
          }
        }
      }
  }
}

// Worst-case number of row tiles: sum_e ceil(n_e / BM) <= ceil(cap / BM) + E_loc.
inline int64_t max_row_tiles(int64_t cap_rows, int E_loc, int BM, bool dense) {
  if (dense) return (cap_rows + BM - 1) / BM;
  return (cap_rows + BM - 1) / BM + E_loc;
}

inline int64_t gemm_grid(int64_t row_tiles, int n_tiles) {
  const int64_t g = row_tiles * n_tiles;
  return (g + 7) / 8 * 8;
}

// fp32 SIMT variant of the same tiling (fp32 activations and weights only):
// 32 rows x 128 weight rows per workgroup, K staged 32 at a time through LDS,
// each thread owns 2 rows x 8 columns (gate/up: 2 rows x 4 gate + 4 up columns).
template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_nt_f32(GemmParams p) {
  constexpr int BM = 32, BKF = 32;
  __shared__ float sA[BM][BKF + 1];
  __shared__ float sB[kBN][BKF + 1];
  __shared__ int s_loc[4];
  int e, rows, m_off, nt;
  int64_t row_begin;
  if (!locate_tile<BM>(p, s_loc, e, row_begin, rows, m_off, nt)) return;

  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t ksplit = static_cast<int64_t>(blockIdx.y) * p.K;
  const float* A = reinterpret_cast<const float*>(p.A) + ksplit;
  const float* B = static_cast<const float*>(p.B) + static_cast<size_t>(e) * p.b_rows * p.ldb + ksplit;
  float acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < p.K; k0 += BKF) {
#pragma unroll
    for (int i = 0; i < BM * BKF / 256; ++i) {
      const int c = tid + i * 256;
      const int r = c / BKF, kc = c % BKF;
      int mr = m_off + r;
      mr = mr < rows ? mr : rows - 1;
      sA[r][kc] = A[(row_begin + mr) * p.lda + k0 + kc];
    }
#pragma unroll
    for (int i = 0; i < kBN * BKF / 256; ++i) {
      const int c = tid + i * 256;
      const int r = c / BKF, kc = c % BKF;
      sB[r][kc] = B[static_cast<size_t>(b_global_row<MODE>(p, nt, r)) * p.ldb + k0 + kc];
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
    const int mr = m_off + ty + 16 * i;
    if (mr >= rows) continue;
    float* C = static_cast<float*>(p.C) + blockIdx.y * p.split_c + (row_begin + mr) * p.ldc;
    if constexpr (MODE == MODE_GATEUP) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float g = acc[i][j], u = acc[i][j + 4];
        C[nt * (kBN / 2) + tx + 16 * j] = g / (1.0f + expf(-g)) * u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = nt * kBN + tx + 16 * j;
        if (MODE == MODE_ROUTER && col >= p.N) continue;
        C[col] = acc[i][j] + ((MODE == MODE_ROUTER && p.bias) ? p.bias[col] : 0.f);
      }
    }
  }
}

}  // namespace dbomoe
