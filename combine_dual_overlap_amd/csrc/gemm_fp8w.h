// Grouped expert GEMM for bf16 activations x fp8 e4m3 weights with 128 x 128
// block scales (the expert compute of "[Core/DBO][1/N] Add Dual-Batch Overlap
// mechanism to VLLM", performance discussion, for the fp8 checkpoint of
// "[Perf] Fix DBO overlap: capture DeepEP event before yield", Test Plan).
//
// Every operand is staged by LDS DMA (global_load_lds_dwordx4, counted by
// hand): activation rows as bf16, weight rows as their fp8 codes, in a ring of
// 64-wide K stages (three: two stages are in flight while the MFMAs of the
// third run), and no register ring or LDS store sits on the load path.
//
// The weights stay fp8 in LDS.  Each wave converts its fragments exactly to
// bf16 when it reads them (every e4m3 value is a bf16 value), so the MFMAs
// sum code value x activation over each 128-wide K block; code value x s is
// never formed or rounded.  The block scale s is applied in one of two ways:
//  * block accumulator: the block's MFMAs sum into a block accumulator, and at
//    the end of the block the fp32 accumulator takes s x block (one fma);
//  * one accumulator (ONE_ACC): the accumulator is kept in units of the
//    current K block's scale: entering block b it is multiplied by
//    s_prev / s_b, the block's MFMAs add into it directly, and the last
//    block's scale is applied at the end.  Mathematically the same sum, with
//    one fp32 rounding per block boundary (relative 2^-24 each); it needs
//    the partial sums divided by a block scale to stay within the fp32 range.
//    A block whose scale is zero contributes nothing: the weight codes of the
//    columns it scales are masked to zero for that block (every code read is
//    ANDed with its scale row's mask, no branch; a tile without a zero scale
//    runs a copy of the loop without the mask).  Half the accumulator registers (156 against
//    224 VGPRs at 128 rows), which with a two-stage ring (49 KB of LDS) lets
//    three workgroups share a CU instead of two.
//
// K order: within a 64-wide stage, lane group q = lane / 16 of an MFMA
// supplies K offsets 16q + 8kk .. 16q + 8kk + 7 for the stage's MFMA step kk
// (0 or 1), for both operands, so one 16-byte LDS read of a weight row feeds
// both steps.  The same terms are summed, in another order than the plain
// K order (every tile shape of this kernel uses this one, so they agree bit
// for bit).
//
// Tile: BM (64 or 128) rows x BN (128 or 256) weight rows (gate/up: BN/2
// gate + the BN/2 matching up rows; a 256-row down tile spans two scale row
// blocks, each wave's columns within one), WAVES_M x WAVES_N waves (2 x 2 or
// 2 x 4), each a block of 16x16x32 bf16 MFMAs.  Group 0 (routed experts) only.
#pragma once

#include "gemm_mfma.h"

namespace dbomoe {

// LDS byte offset of 16-byte chunk q (0..3) of row r of an fp8 weight stage
// (64-byte rows).  The chunk index is XORed with two bits of the row so that
// the rows one 16-byte fragment read touches spread over the banks (distinct
// banks for any 8 consecutive lanes, and for 16 at 64 banks).  The swizzle
// works on whole 16-byte chunks, which is what a DMA lane writes.  Measured in
// the layer: LDS instructions active 2.4 % of the wave cycles, about half of
// those cycles bank conflicts (the DMA writes included); not a limit.
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

// Waits until at most n of this wave's DMAs are in flight, n counted at run
// time (DMAs complete in issue order); n above MAXN waits for MAXN, which is
// only stricter.
template <int MAXN>
__device__ __forceinline__ void wait_dmas(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) {
      wait_vmcnt<MAXN>();
      return;
    }
    wait_dmas<MAXN - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// K blocks of one tile's scale rows (one 64-lane dword DMA per row)
constexpr int kW8MaxKBlocks = 64;
template <int BM, int NBUF, int BN = kBN> struct W8Lds {
  static constexpr int A = BM * kBK * 2;                       // activation stage
  static constexpr int B = BN * kBK;                           // fp8 weight stage
  static constexpr int S = 2 * kW8MaxKBlocks * 4;              // two scale rows
  static constexpr int bytes = NBUF * (A + B) + S;
};

template <int MODE, int BM, int WAVES_M, int WAVES_N, int NBUF, bool ONE_ACC, int BN>
__device__ __forceinline__ void gemm_tile_fp8w(const GemmGroup& g, const TileLoc& t, const GemmParams& p,
                                               uint8_t* lds) {
  static_assert(BN == 128 || BN == 256, "128 or 256 weight rows");
  constexpr int BK = kBK, NW = WAVES_M * WAVES_N;
  using S = TileShape<BM, WAVES_M, WAVES_N, BN>;
  constexpr int TM = S::TM, TN = S::TN, WM = S::WM, WN = S::WN;
  constexpr int A_BYTES = W8Lds<BM, NBUF, BN>::A, B_BYTES = W8Lds<BM, NBUF, BN>::B;
  constexpr int NQA = BM / 8 / NW;           // activation DMAs per wave per stage (8 rows each)
  constexpr int NQB = BN / 16 / NW;          // weight DMAs per wave per stage (16 rows each)
  constexpr int NDMA = NQA + NQB;
  static_assert(NQA >= 1 && NQB >= 1 && NQA * NW * 8 == BM && NQB * NW * 16 == BN, "DMA split");
  static_assert(NBUF >= 2 && (NBUF - 2) * NDMA < 64, "ring depth");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int K = g.K, KT = K / BK, nt = t.nt;

  uint8_t* sA = lds;
  uint8_t* sB = lds + NBUF * A_BYTES;
  const uint32_t lds_a = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(lds)));
  const uint32_t lds_b = lds_a + NBUF * A_BYTES;

  // Activation DMA i of this wave fills tile rows 8 (wave NQA + i) .. + 7:
  // lane l takes row l / 8 of the group and its 16-byte chunk (l % 8) ^ (l / 8),
  // the XOR-swizzled order of lds_off_k (rows past the expert: its last row).
  // Only the first na of them carry a row of the tile; the others are not
  // issued, and the LDS rows they would fill feed only output rows that are
  // never stored (an output row depends on its own activation row alone).  So
  // a wave issues nd = na + NQB DMAs per stage, a count fixed for the tile.
  const int na = __builtin_amdgcn_readfirstlane(
      max(0, min(NQA, (t.rows - t.m_off - 8 * wave * NQA + 7) / 8)));
  const int nd = na + NQB;
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
  // row block of a down tile), staged into LDS by wave 0 ahead of the first
  // stage (one dword DMA per row, lane j carrying K block j), so they arrive
  // with the first stage instead of costing a memory round trip of their own.
  const int kblocks = K / 128;
  const float* se = g.bscale + static_cast<size_t>(t.e) * (g.b_rows / 128) * kblocks;
  const float* srow0;
  const float* srow1;
  if constexpr (MODE == MODE_GATEUP) {
    srow0 = se + static_cast<size_t>((nt * (BN / 2)) / 128) * kblocks;
    srow1 = se + static_cast<size_t>((g.N + nt * (BN / 2)) / 128) * kblocks;
  } else {
    srow0 = se + static_cast<size_t>((nt * BN) / 128) * kblocks;
    srow1 = BN == 256 ? srow0 + kblocks : srow0;   // a 256-row tile spans two row blocks
  }
  const float* sS = reinterpret_cast<const float*>(lds + NBUF * (A_BYTES + B_BYTES));
  // Every load the compiler issued has completed: inside the loop only the
  // DMAs are in flight, and their waits are counted by hand.
  __builtin_amdgcn_s_waitcnt(0);
  if (wave == 0) {
    const uint32_t lds_s = lds_a + NBUF * (A_BYTES + B_BYTES);
    lds_dma4(lds_s, srow0 + min(lane, kblocks - 1));
    lds_dma4(lds_s + kW8MaxKBlocks * 4, srow1 + min(lane, kblocks - 1));
  }

  auto issue = [&](int kt, int buf) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < NQA; ++i)
      if (i < na) lds_dma16(lds_a + buf * A_BYTES + (wave * NQA + i) * 1024, a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < NQB; ++i) lds_dma16(lds_b + buf * B_BYTES + (wave * NQB + i) * 1024, b_src[i] + k0);
  };

  f32x4_t acc[TM][TN], blk[TM][TN];   // blk: block accumulator (unused with ONE_ACC)
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      blk[i][j] = acc[i][j];
    }
  // ONE_ACC: per scale row (gate, up; a down tile uses the first), the scale
  // the accumulator is expressed in and whether the current block's is nonzero
  float unit[2] = {1.f, 1.f};
  uint32_t code_mask[2] = {~0u, ~0u};
  // the scale row of fragment tn: gate or up half of a gate/up tile, or the
  // 128-row block of a 256-row down tile that the wave's columns fall in
  auto half = [&](int tn) {
    if constexpr (MODE == MODE_GATEUP) return tn >= TN / 2 ? 1 : 0;
    else return BN == 256 ? (wn * WN) / 128 : 0;
  };
  const int frag_row = lane & 15, q = lane >> 4;
  const int tm_valid = __builtin_amdgcn_readfirstlane(
      max(0, min(TM, (t.rows - t.m_off - wm * WM + 15) / 16)));
  int b_off[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) b_off[tn] = w8_off(b_lds_row<MODE, WN, TN, BN>(wn, tn) + frag_row, q);

  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;
  // MFMAs of one stage into the block accumulator (FIRST: the block's first
  // stage, whose first step starts from zero).
  auto compute = [&](int buf, auto first, auto full, auto mask) {
    // a wave with no rows in this tile (the last row tile of an expert) only
    // stages its share of the DMAs and meets the barriers
    if (!decltype(full)::value && tm_valid == 0) return;
    const bf16_t* A = reinterpret_cast<const bf16_t*>(sA + buf * A_BYTES);
    const uint8_t* B = sB + buf * B_BYTES;
    bf16x8_t blo[TN], bhi[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      u32x4_t c = *reinterpret_cast<const u32x4_t*>(B + b_off[tn]);
      if constexpr (ONE_ACC && decltype(mask)::value) c &= code_mask[half(tn)];
      fp8x16_to_bf16_exact(c, blo[tn], bhi[tn]);
    }
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
            if constexpr (ONE_ACC) {
              acc[tm][tn] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], kk == 0 ? blo[tn] : bhi[tn], acc[tm][tn], 0, 0, 0);
            } else {
              const f32x4_t c = (decltype(first)::value && kk == 0) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : blk[tm][tn];
              blk[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], kk == 0 ? blo[tn] : bhi[tn], c, 0, 0, 0);
            }
          }
    }
  };
  // ONE_ACC, entering K block kb: the accumulator into units of its scale
  auto enter_block = [&](int kb, auto full) {
    if (!decltype(full)::value && tm_valid == 0) return;
    float r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float sb = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sS[h * kW8MaxKBlocks + kb])));
      const bool live = sb != 0.f;
      code_mask[h] = live ? ~0u : 0u;
      r[h] = live ? unit[h] / sb : 1.f;
      unit[h] = live ? sb : unit[h];
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      if (decltype(full)::value || tm < tm_valid)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[tm][tn][e] *= r[half(tn)];
  };
  // acc += s * blk for K block kb
  auto scale_block = [&](int kb, auto full) {
    if (!decltype(full)::value && tm_valid == 0) return;
    const float s[2] = {sS[kb], sS[kW8MaxKBlocks + kb]};
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      if (decltype(full)::value || tm < tm_valid)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const float sc = s[half(tn)];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[tm][tn][r] = __builtin_fmaf(sc, blk[tm][tn][r], acc[tm][tn][r]);
        }
  };

  // Ring of NBUF stages: stage kt lives in buffer kt % NBUF.  Stage kt issues
  // the DMAs of stage kt + NBUF - 1 into the buffer stage kt - 1 used (every
  // wave left it at the previous barrier), runs its MFMAs, waits for its own
  // nd DMAs of stage kt + 1 (later stages may stay in flight) and meets the
  // other waves at the barrier.  The wait before the first stage also covers
  // wave 0's scale DMAs, which were issued before any stage.
  const int pre = min(NBUF - 1, KT);
  for (int s = 0; s < pre; ++s) issue(s, s);
  wait_dmas<(NBUF - 2) * NDMA>((pre - 1) * nd);
  __syncthreads();
  auto stage = [&](int kt, int buf, auto first, auto full, auto mask) {
    const int ahead = kt + NBUF - 1;
    if (ahead < KT) issue(ahead, buf == 0 ? NBUF - 1 : buf - 1);
    if constexpr (ONE_ACC) {
      if (decltype(first)::value) enter_block(kt >> 1, full);
    }
    compute(buf, first, full, mask);
    if constexpr (!ONE_ACC) {
      if (!decltype(first)::value) scale_block(kt >> 1, full);
    }
    wait_dmas<(NBUF - 2) * NDMA>((min(KT - 1, ahead) - (kt + 1)) * nd);
    __syncthreads();
  };
  // KT is even (K is a multiple of 128): two stages per K block.
  auto run = [&](auto full, auto mask) {
    int buf = 0;                               // kt % NBUF
    for (int kt = 0; kt < KT; kt += 2) {
      const int b1 = buf == NBUF - 1 ? 0 : buf + 1;
      stage(kt, buf, True{}, full, mask);
      stage(kt + 1, b1, False{}, full, mask);
      buf = b1 == NBUF - 1 ? 0 : b1 + 1;
    }
  };
  // ONE_ACC: only a tile whose scale rows hold a zero runs the loop that masks
  // the codes (the mask costs ~3 % of the gate/up GEMM); the scale rows are in
  // LDS since the wait and barrier above.
  bool any_zero = false;
  if constexpr (ONE_ACC) {
    const bool z = lane < kblocks && (sS[lane] == 0.f || sS[kW8MaxKBlocks + lane] == 0.f);
    any_zero = __ballot(z) != 0;
  }
  if (tm_valid == TM) {
    if (any_zero)
      run(True{}, True{});
    else
      run(True{}, False{});
  } else {
    if (any_zero)
      run(False{}, True{});
    else
      run(False{}, False{});
  }
  if constexpr (ONE_ACC) {   // into real units: the last nonzero block scale
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tm][tn][e] *= unit[half(tn)];
  }
  store_tile<BM, WAVES_M, WAVES_N, MODE, BN>(g, t, p, acc, reinterpret_cast<bf16_t*>(sA));
}

// Waves per SIMD a shape runs at: workgroups per CU from its LDS (160 KB per
// CU) times its waves, over 4 SIMDs (at most 4: the register budget of a wave
// is 512 / waves per SIMD).
template <int BM, int NW, int NBUF, int BN = kBN> struct W8Occ {
  static constexpr int wgs = (160 * 1024) / W8Lds<BM, NBUF, BN>::bytes;
  static constexpr int w = wgs * NW / 4;
  static constexpr int value = w < 1 ? 1 : w > 4 ? 4 : w;
};

// Group 0 only (a launch without a dense group of shared experts); K a
// multiple of 128 with at most kW8MaxKBlocks blocks.
template <int MODE, int BM, int WAVES_M = 2, int WAVES_N = 2, int NBUF = 3, bool ONE_ACC = false, int BN = kBN>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64, (W8Occ<BM, WAVES_M * WAVES_N, NBUF, BN>::value))
void k_gemm_fp8w(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[W8Lds<BM, NBUF, BN>::bytes];
  int* s_loc = reinterpret_cast<int*>(lds);
  TileLoc t;
  if (!locate_tile<BM>(p, s_loc, t)) return;
  __syncthreads();                                  // s_loc read by all before the ring is filled
  gemm_tile_fp8w<MODE, BM, WAVES_M, WAVES_N, NBUF, ONE_ACC, BN>(p.g[0], t, p, lds);
}

}  // namespace dbomoe
