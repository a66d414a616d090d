// Grouped expert GEMM for bf16 activations x fp8 e4m3 weights with 128 x 128
// block scales (the expert compute of "[Core/DBO][1/N] Add Dual-Batch Overlap
// mechanism to VLLM", performance discussion, for the fp8 checkpoint of
// "[Perf] Fix DBO overlap: capture DeepEP event before yield", Test Plan).
//
// Every operand is staged by LDS DMA (global_load_lds_dwordx4, counted by
// hand): activation rows as bf16, weight rows as their fp8 codes, in a ring of
// three 64-wide K stages, so two stages are in flight while the MFMAs of the
// third run, and no register ring or LDS store sits on the load path.
//
// The weights stay fp8 in LDS.  Each wave converts its fragments exactly to
// bf16 when it reads them (every e4m3 value is a bf16 value) and the MFMAs sum
// code value x activation over one 128-wide K block into a block accumulator;
// at the end of the block the fp32 accumulator takes s x block (one fma), s
// being the block's scale.  This is the block-scaled product as defined, with
// no rounding of the weights: code value x s is never formed.
//
// K order: within a 64-wide stage, lane group q = lane / 16 of an MFMA
// supplies K offsets 16q + 8kk .. 16q + 8kk + 7 for the stage's MFMA step kk
// (0 or 1), for both operands, so one 16-byte LDS read of a weight row feeds
// both steps.  A reduction is the same sum in any order of its terms.
//
// Tile: BM (64 or 128) rows x 128 weight rows (gate/up: 64 gate + the 64
// matching up rows), 2 x 2 waves, each a (BM/2) x 64 block of 16x16x32 bf16
// MFMAs.  Group 0 (routed experts) only.
#pragma once

#include "gemm_mfma.h"

namespace dbomoe {

// LDS byte offset of 16-byte chunk q (0..3) of row r of an fp8 weight stage
// (64-byte rows).  The chunk index is XORed with two bits of the row so that
// the 16 rows a fragment read touches, 8 or 16 lanes at a time, fall in
// distinct banks.  The swizzle works on whole 16-byte chunks, which is what a
// DMA lane writes.
__device__ __forceinline__ int w8_swz(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1); }
__device__ __forceinline__ int w8_off(int r, int q) { return r * 64 + ((q ^ w8_swz(r)) << 4); }

// 16 e4m3 codes -> the bf16 operands of two MFMA steps (codes 0..7, 8..15),
// exact: v_cvt_scalef32_pk_bf16_fp8 with scale 1 (it applies only the scale's
// exponent, here 0).
__device__ __forceinline__ void fp8x16_to_bf16_exact(const u32x4_t& c, bf16x8_t& lo, bf16x8_t& hi) {
  uint32_t o[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    o[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w], 1.f, false));
    o[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w], 1.f, true));
  }
  lo = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
  hi = __builtin_bit_cast(bf16x8_t, u32x4_t{o[4], o[5], o[6], o[7]});
}

constexpr int kW8Buf = 3;                                      // LDS stages in the ring
template <int BM> struct W8Lds {
  static constexpr int A = BM * kBK * 2;                       // activation stage
  static constexpr int B = kBN * kBK;                          // fp8 weight stage
  static constexpr int bytes = kW8Buf * (A + B);               // 72 KB (BM 128), 48 KB (BM 64)
};
// K blocks a wave can hold scales for (two per lane)
constexpr int kW8MaxKBlocks = 128;

template <int MODE, int BM>
__device__ __forceinline__ void gemm_tile_fp8w(const GemmGroup& g, const TileLoc& t, const GemmParams& p,
                                               uint8_t* lds) {
  constexpr int BN = kBN, BK = kBK, WAVES_M = 2, WAVES_N = 2;
  using S = TileShape<BM, WAVES_M, WAVES_N, BN>;
  constexpr int TM = S::TM, TN = S::TN, WM = S::WM, WN = S::WN;
  constexpr int A_BYTES = W8Lds<BM>::A, B_BYTES = W8Lds<BM>::B;
  constexpr int NQA = BM / 8 / 4;            // activation DMAs per wave per stage (8 rows each)
  constexpr int NQB = BN / 16 / 4;           // weight DMAs per wave per stage (16 rows each)
  constexpr int NDMA = NQA + NQB;
  static_assert(NQA >= 1 && NQB >= 1 && NDMA < 16, "DMA split");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int K = g.K, KT = K / BK, nt = t.nt;

  uint8_t* sA = lds;
  uint8_t* sB = lds + kW8Buf * A_BYTES;
  const uint32_t lds_a = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(lds)));
  const uint32_t lds_b = lds_a + kW8Buf * A_BYTES;

  // Activation DMA i of this wave fills tile rows 8 (wave NQA + i) .. + 7:
  // lane l takes row l / 8 of the group and its 16-byte chunk (l % 8) ^ (l / 8),
  // the XOR-swizzled order of lds_off_k (rows past the expert: its last row).
  const int lrow = lane >> 3, lchunk = (lane & 7) ^ lrow;
  const bf16_t* a_src[NQA];
#pragma unroll
  for (int i = 0; i < NQA; ++i) {
    int mr = t.m_off + 8 * (wave * NQA + i) + lrow;
    mr = mr < t.rows ? mr : t.rows - 1;
    a_src[i] = g.A + (t.row_begin + mr) * g.lda + lchunk * 8;
  }
  // Weight DMA i of this wave fills weight-tile rows 16 (wave NQB + i) .. + 15:
  // lane l lands at chunk l % 4 of row l / 4, which holds chunk (l % 4) ^ swz.
  const uint8_t* b_src[NQB];
#pragma unroll
  for (int i = 0; i < NQB; ++i) {
    const int r = 16 * (wave * NQB + i) + (lane >> 2);
    const int qlog = (lane & 3) ^ w8_swz(r);
    b_src[i] = static_cast<const uint8_t*>(g.B) + static_cast<size_t>(t.e) * g.b_estride +
               static_cast<size_t>(b_global_row<MODE, BN>(g, nt, r)) * g.ldb + qlog * 16;
  }
  // Block scales of this column tile: the gate and up row blocks (or the one
  // row block of a down tile), K block j in lane j % 64 of slot j / 64.
  const int kblocks = K / 128;
  const float* se = g.bscale + static_cast<size_t>(t.e) * (g.b_rows / 128) * kblocks;
  const float* srow0;
  const float* srow1;
  if constexpr (MODE == MODE_GATEUP) {
    srow0 = se + static_cast<size_t>((nt * (BN / 2)) / 128) * kblocks;
    srow1 = se + static_cast<size_t>((g.N + nt * (BN / 2)) / 128) * kblocks;
  } else {
    srow0 = se + static_cast<size_t>((nt * BN) / 128) * kblocks;
    srow1 = srow0;
  }
  float scv[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float* row = j == 0 ? srow0 : srow1;
    scv[j][0] = row[min(lane, kblocks - 1)];
    scv[j][1] = row[min(lane + 64, kblocks - 1)];
  }
  // Every load the compiler issued has completed: inside the loop only the
  // DMAs are in flight, and their waits are counted by hand.
  __builtin_amdgcn_s_waitcnt(0);

  auto issue = [&](int kt, int buf) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < NQA; ++i) lds_dma16(lds_a + buf * A_BYTES + (wave * NQA + i) * 1024, a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < NQB; ++i) lds_dma16(lds_b + buf * B_BYTES + (wave * NQB + i) * 1024, b_src[i] + k0);
  };

  f32x4_t acc[TM][TN], blk[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      blk[i][j] = acc[i][j];
    }
  const int frag_row = lane & 15, q = lane >> 4;
  const int tm_valid = __builtin_amdgcn_readfirstlane(
      max(0, min(TM, (t.rows - t.m_off - wm * WM + 15) / 16)));
  int b_off[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) b_off[tn] = w8_off(b_lds_row<MODE, WN, TN, BN>(wn, tn) + frag_row, q);

  // MFMAs of one stage into the block accumulator (FIRST: the block's first
  // stage, whose first step starts from zero).
  auto compute = [&](int buf, auto first, auto full) {
    const bf16_t* A = reinterpret_cast<const bf16_t*>(sA + buf * A_BYTES);
    const uint8_t* B = sB + buf * B_BYTES;
    bf16x8_t blo[TN], bhi[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      fp8x16_to_bf16_exact(*reinterpret_cast<const u32x4_t*>(B + b_off[tn]), blo[tn], bhi[tn]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t af[TM];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        if (decltype(full)::value || tm < tm_valid)
          af[tm] = *reinterpret_cast<const bf16x8_t*>(&A[lds_off_k<BK>(wm * WM + tm * 16 + frag_row, 2 * q + kk)]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        if (decltype(full)::value || tm < tm_valid)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            const f32x4_t c = (decltype(first)::value && kk == 0) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : blk[tm][tn];
            blk[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], kk == 0 ? blo[tn] : bhi[tn], c, 0, 0, 0);
          }
    }
  };
  // acc += s * blk for K block kb
  auto scale_block = [&](int kb, auto full) {
    float s[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float v = kb < 64 ? scv[j][0] : scv[j][1];
      s[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kb & 63));
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      if (decltype(full)::value || tm < tm_valid)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const float sc = (MODE == MODE_GATEUP && tn >= TN / 2) ? s[1] : s[0];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[tm][tn][r] = __builtin_fmaf(sc, blk[tm][tn][r], acc[tm][tn][r]);
        }
  };

  // Ring: stage kt lives in buffer kt % 3.  Stage kt issues the DMAs of stage
  // kt + 2 into the buffer stage kt - 1 used (every wave left it at the
  // previous barrier), runs its MFMAs, waits for its own DMAs of stage kt + 1
  // (those of kt + 2 may stay in flight) and meets the others at the barrier.
  issue(0, 0);
  if (KT > 1) issue(1, 1);
  if (KT > 1)
    wait_vmcnt<NDMA>();
  else
    wait_vmcnt<0>();
  __syncthreads();
  auto stage = [&](int kt, int buf, int buf2, auto first, auto full) {
    if (kt + 2 < KT) issue(kt + 2, buf2);
    compute(buf, first, full);
    if (!decltype(first)::value) scale_block(kt >> 1, full);
    if (kt + 2 < KT)
      wait_vmcnt<NDMA>();
    else
      wait_vmcnt<0>();
    __syncthreads();
  };
  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;
  // KT is even (K is a multiple of 128): two stages per K block.
  auto run = [&](auto full) {
    int buf = 0;                               // kt % 3
    for (int kt = 0; kt < KT; kt += 2) {
      const int b1 = buf == 2 ? 0 : buf + 1, b2 = b1 == 2 ? 0 : b1 + 1;
      stage(kt, buf, b2, True{}, full);        // stage kt + 2 goes to (kt + 2) % 3 = b2
      const int b3 = b2 == 2 ? 0 : b2 + 1;
      stage(kt + 1, b1, b3, False{}, full);
      buf = b2;
    }
  };
  if (tm_valid == TM)
    run(True{});
  else
    run(False{});
  store_tile<BM, WAVES_M, WAVES_N, MODE, BN>(g, t, p, acc, reinterpret_cast<bf16_t*>(sA));
}

// Group 0 only (a launch without a dense group of shared experts); K a
// multiple of 128 with at most kW8MaxKBlocks blocks.
template <int MODE, int BM>
__global__ __launch_bounds__(256, (BM == 128 ? 2 : 3)) void k_gemm_fp8w(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[W8Lds<BM>::bytes];
  int* s_loc = reinterpret_cast<int*>(lds);
  TileLoc t;
  if (!locate_tile<BM>(p, s_loc, t)) return;
  __syncthreads();                                  // s_loc read by all before the ring is filled
  gemm_tile_fp8w<MODE, BM>(p.g[0], t, p, lds);
}

}  // namespace dbomoe
