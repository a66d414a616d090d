// Grouped SwiGLU expert FFN for gfx950: gate/up GEMM with SiLU-mul fused into
// its epilogue, then the down GEMM, each over all local experts in one launch.
//
// The expert compute of "[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to
// VLLM" (performance discussion: batched MoE GEMM + act-and-mul).  Reading:
// W13 = [gate rows 0..I) ; up rows I..2I)], h = silu(gate) * up rounded to the
// activation dtype, y = h W2^T.  With fp8 activations (the fused SiLU-mul +
// fp8 quantisation op of the same page, CI discussion) the rows arrive as E4M3
// codes with per-128-column E8M0 scales and h is quantised the same way
// (gemm_fp8.h, fp8_act.h).
#include <cmath>

#include "gemm_fp8.h"
#include "gemm_fp8w.h"

namespace dbomoe {

// Rows per expert under roughly uniform routing are about Poisson(mean): size
// the row tile for the likely largest expert, so most experts take one row
// tile (their weights stream once) and large experts get the big MFMA tile.
// An expert a row or two past a tile boundary streams its weights once more
// for a nearly empty tile, which costs more than the idle MFMA rows of the
// larger tile: at 64 +- 8 rows per expert (the R1-shaped share) 128-row tiles
// against 64 took the DBO layer from 0.969 to 0.933 ms (gate/up 286 -> 267 us,
// down 144 -> 137 us).
static int choose_tile_m(int64_t mean_rows) {
  const double m = static_cast<double>(mean_rows);
  const double est_max = m + 3.0 * std::sqrt(m) + 1.0;
  if (est_max <= 32) return 32;
  if (est_max <= 64) return 64;
  return 128;
}

// Row tiles of 32, 64 or 128 rows.
// The 32-row tile takes 64 weight rows per column tile (2 x 2 waves of 16 x
// 32): twice the tiles of 128-row-wide columns, so the last partial round of
// workgroups is shorter (decode gate/up with the shared experts 145.5 ->
// 140.9 us, down 75.0 -> 73.1 us, standalone).  When K allows, it stages K
// 128 wide (256 contiguous bytes of each weight row per stage, three
// workgroups per CU): decode gate/up 146.0 -> 144.4 us in the layer; 256
// wide (one workgroup per CU) was slower, 168.8 us.
static int col_tile_rows(int bm) { return bm == 32 ? 64 : kBN; }

// True if every group of the launch has a K that is a multiple of bk.
static bool k_multiple_of(const GemmParams& g, int bk) {
  return g.g[0].K % bk == 0 && (g.rows1 == 0 || g.g[1].K % bk == 0);
}

// K blocks of the launch's routed group within what k_gemm_fp8w stages per
// scale row.
static bool fp8w_fits(const GemmParams& g) { return g.g[0].K / 128 <= kW8MaxKBlocks; }

template <int MODE, bool FP8>
static void launch_mfma(int bm, dim3 grid, hipStream_t s, const GemmParams& g, bool full_tiles = false,
                        bool wide = false) {
  // bf16 weights, 128-row tiles: activation and weight tiles staged by LDS
  // DMA (bitwise equal to the register-staged kernel; measured
  // standalone on the skewed-layer shapes: gate/up 401 -> 367 us, down 217 ->
  // 197 us).  The down GEMM runs 8 waves per tile, 2 x 4 at 4 per SIMD: the
  // skewed layer (DBO) 1.096 -> 1.078 ms, down 180 -> 169 us; 2 x 4 gate/up
  // tiles gained nothing there (330 -> 333 us).
  if (!FP8 && bm == 128 && k_multiple_of(g, kBK)) {
    if (MODE == MODE_DOWN)
      hipLaunchKernelGGL((k_gemm_dma<MODE, 128, kBN, kBK, 2, false, 4, 4>), grid, dim3(512), 0, s, g);
    else
      hipLaunchKernelGGL((k_gemm_dma<MODE>), grid, dim3(256), 0, s, g);
    return;
  }
  // fp8 weights, 64- or 128-row tiles, no dense group: fp8 codes staged by LDS
  // DMA, converted exactly at fragment read, block scales applied to the fp32
  // block sums (gemm_fp8w.h).  Measured standalone against the register path
  // (which expands value(code) x scale to bf16 before LDS): Qwen3-shaped
  // prefill gate/up 373.8 -> 310.2 us, down 229.1 -> 206.2 us; R1-shaped share
  // gate/up (K = 7168, 64-row tiles) 333.5 -> 283.3 us.  The 128-row down
  // GEMM (short K, many column tiles) runs 8 waves per tile, 2 x 4, at 4 waves
  // per SIMD: Qwen3-shaped prefill down 193 -> 178 us in the layer.  2 x 2
  // stays faster for gate/up (308.2 against 329.7 us standalone) and for the
  // 64-row down tiles of the R1-shaped share in the layer (148.5 against
  // 166.7 us, although 141.5 against 154.5 us standalone).
  // With full_tiles (about 128 rows per expert or more: full 128-row tiles,
  // MFMA-bound) the tiles keep one accumulator (ONE_ACC) and a two-stage ring,
  // three 2 x 2 workgroups per CU: Qwen3-shaped prefill layer (DBO) 1.015 ->
  // 0.957 ms, gate/up 287 -> 266 us, down 165 -> 157 us.  On the R1-shaped
  // share (64 rows per expert, weight streaming) the two-stage ring lost
  // (gate/up 258 -> 285 us), so it keeps the block accumulator and three
  // stages.  Tiles of 64 and 128 rows of one launch take the same arithmetic,
  // so the row tile does not change the result.
  // wide (128-row gate/up tiles with the block accumulator, i.e. the
  // weight-streaming R1-shaped share): tiles of 256 weight rows (128 gate + 128
  // up), 8 waves of 64 x 64, a four-stage ring (128 KB, one workgroup per CU):
  // the same waves and weight bytes in flight per CU as two 128-row tiles,
  // with half the activation re-reads (each expert's rows are read by 16
  // column tiles instead of 32).  R1-shaped gate/up 252 -> 233 us, layer
  // (DBO) 0.886 -> 0.840 ms; three stages 235 us.
  if (FP8 && (bm == 64 || bm == 128) && g.rows1 == 0 && fp8w_fits(g)) {
    if (wide && MODE == MODE_GATEUP) {
      if constexpr (MODE == MODE_GATEUP)
        hipLaunchKernelGGL((k_gemm_fp8w<MODE, 128, 2, 4, 4, false, 256>), grid, dim3(512), 0, s, g);
    } else if (full_tiles) {
      if (bm == 128)
        hipLaunchKernelGGL((k_gemm_fp8w<MODE, 128, 2, 2, 2, true>), grid, dim3(256), 0, s, g);
      else
        hipLaunchKernelGGL((k_gemm_fp8w<MODE, 64, 2, 2, 3, true>), grid, dim3(256), 0, s, g);
    } else if (MODE == MODE_DOWN && bm == 128) {
      hipLaunchKernelGGL((k_gemm_fp8w<MODE, 128, 2, 4>), grid, dim3(512), 0, s, g);
    } else if (bm == 128) {
      hipLaunchKernelGGL((k_gemm_fp8w<MODE, 128>), grid, dim3(256), 0, s, g);
    } else {
      hipLaunchKernelGGL((k_gemm_fp8w<MODE, 64>), grid, dim3(256), 0, s, g);
    }
    return;
  }
  if (bm == 32 && k_multiple_of(g, 2 * kBK))
    hipLaunchKernelGGL((k_gemm_nt<32, 2, 2, MODE, FP8, 64, 2 * kBK>), grid, dim3(256), 0, s, g);
  else if (bm == 32)
    hipLaunchKernelGGL((k_gemm_nt<32, 2, 2, MODE, FP8, 64>), grid, dim3(256), 0, s, g);
  else if (bm == 64)
    hipLaunchKernelGGL((k_gemm_nt<64, 2, 2, MODE, FP8>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((k_gemm_nt<128, 2, 2, MODE, FP8>), grid, dim3(256), 0, s, g);
}

static GemmGroup gate_up_group(const void* x, int32_t H, int32_t I, const void* w13, const float* s13, void* h) {
  GemmGroup g{};
  g.A = static_cast<const bf16_t*>(x);
  g.lda = H;
  g.B = w13;
  g.ldb = H;
  g.bscale = s13;
  g.K = H;
  g.N = I;
  g.b_rows = 2 * I;
  g.n_tiles = I / (kBN / 2);
  g.C = h;
  g.ldc = I;
  g.b_estride = static_cast<int64_t>(g.b_rows) * g.ldb;
  return g;
}

static GemmGroup down_group(const void* h, int32_t H, int32_t I, const void* w2, const float* s2, void* y) {
  GemmGroup g{};
  g.A = static_cast<const bf16_t*>(h);
  g.lda = I;
  g.B = w2;
  g.ldb = I;
  g.bscale = s2;
  g.K = I;
  g.N = H;
  g.b_rows = H;
  g.n_tiles = H / kBN;
  g.C = y;
  g.ldc = H;
  g.b_estride = static_cast<int64_t>(g.b_rows) * g.ldb;
  return g;
}

int dense_down_chunks(moe_dtype act, int32_t I1, int32_t I) {
  if (act == MOE_F32 || I1 <= 0 || I <= 0) return 1;
  for (int d = (I1 + I - 1) / I; d > 1; --d)
    if (I1 % (d * kBK) == 0) return d;
  return 1;
}

// fp32 path: one SIMT launch per group and GEMM.
static moe_status launch_ffn_f32(const FfnArgs& a, hipStream_t s) {
  auto run = [&](const void* x, const int32_t* offsets, int E_loc, int64_t rows, int32_t I, const void* w13,
                 const void* w2, void* h, void* y) -> moe_status {
    GemmParams p{};
    p.offsets = offsets;
    p.E_loc = E_loc;
    p.dense_rows = rows;
    p.g[0] = gate_up_group(x, a.H, I, w13, nullptr, h);
    const int64_t row_tiles = max_row_tiles(rows, E_loc, 32, offsets == nullptr);
    hipLaunchKernelGGL(k_gemm_nt_f32<MODE_GATEUP>, dim3(static_cast<unsigned>(gemm_grid(row_tiles * p.g[0].n_tiles))),
                       dim3(256), 0, s, p);
    DBOMOE_CHECK_LAUNCH();
    p.g[0] = down_group(h, a.H, I, w2, nullptr, y);
    hipLaunchKernelGGL(k_gemm_nt_f32<MODE_DOWN>, dim3(static_cast<unsigned>(gemm_grid(row_tiles * p.g[0].n_tiles))),
                       dim3(256), 0, s, p);
    DBOMOE_CHECK_LAUNCH();
    return MOE_OK;
  };
  if (a.t0 && hipEventRecord(a.t0, s) != hipSuccess) return MOE_ERR_HIP;
  moe_status st = MOE_OK;
  if (a.cap_rows > 0) st = run(a.x, a.offsets, a.E_loc, a.cap_rows, a.I, a.w13, a.w2, a.h, a.y);
  if (st == MOE_OK && a.rows1 > 0) st = run(a.x1, nullptr, 1, a.rows1, a.I1, a.w13_1, a.w2_1, a.h1, a.y1);
  if (st != MOE_OK) return st;
  if (a.t1 && hipEventRecord(a.t1, s) != hipSuccess) return MOE_ERR_HIP;
  if (a.t2 && hipEventRecord(a.t2, s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

// Worst-case tiles of one grouped GEMM launch (the grid is sized for it;
// surplus workgroups exit at once).
static int64_t tiles_max(int bm, int64_t cap_rows, int E_loc, bool dense, int n_tiles0, int64_t rows1, int E1,
                         int n_tiles1) {
  const int64_t rt1 = rows1 > 0 ? (rows1 + bm - 1) / bm : 0;
  const int64_t rt0 = cap_rows > 0 ? max_row_tiles(cap_rows, E_loc, bm, dense) : 0;
  return rt0 * n_tiles0 + E1 * rt1 * n_tiles1;
}

// ---- fp8 activations ------------------------------------------------------

size_t ffn_fp8_ws_bytes(int64_t cap_rows, int32_t I) {
  return align_up(static_cast<size_t>(cap_rows) * I, 256) + align_up(static_cast<size_t>(cap_rows) * (I / kQGroup), 256);
}

moe_status check_ffn_fp8_shapes(int32_t H, int32_t I, int32_t E_loc, const float* s13, const float* s2) {
  if (H <= 0 || I <= 0 || E_loc < 1) return MOE_ERR_INVALID_ARG;
  if (E_loc > 256) return MOE_ERR_UNSUPPORTED;
  if (H % kF8BN || I % kQGroup) return MOE_ERR_UNSUPPORTED;
  if (H > kF8MaxK || I > kF8MaxK) return MOE_ERR_UNSUPPORTED;
  if (!s13 || !s2) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Row tile of the fp8 kernel: 64 or 128 (8 waves; 64 rows is its smallest
// tile).  Its cost per tile hardly depends on how many of the rows are
// filled, so 128-row tiles win as soon as experts are likely to exceed 64
// rows (measured: R1-shaped share with about 64 rows per expert, gate/up
// 188 us with 128-row tiles, 293 us with 64).
static int f8_tile_m(int tile_m, int64_t rows_hint) {
  if (tile_m > 0) return tile_m >= 128 ? 128 : 64;
  const double m = static_cast<double>(rows_hint);
  return m + 3.0 * std::sqrt(m) + 1.0 <= 64 ? 64 : 128;
}

// LDS-DMA staging for K <= 4096, the register ring beyond (measured, see
// gemm_fp8.h).
template <int MODE>
static void launch_f8(int bm, dim3 grid, hipStream_t s, const F8Params& p) {
  const bool dma = p.g.K <= kF8DmaMaxK;
  if (bm == 128) {
    if (dma)
      hipLaunchKernelGGL((k_gemm_f8d<128, MODE>), grid, dim3(kF8Threads), 0, s, p);
    else
      hipLaunchKernelGGL((k_gemm_f8<128, MODE>), grid, dim3(kF8Threads), 0, s, p);
  } else {
    if (dma)
      hipLaunchKernelGGL((k_gemm_f8d<64, MODE>), grid, dim3(kF8Threads), 0, s, p);
    else
      hipLaunchKernelGGL((k_gemm_f8<64, MODE>), grid, dim3(kF8Threads), 0, s, p);
  }
}

// Routed experts through the fp8 kernel; the shared experts (weights in the
// activation dtype) through the bf16 kernel as a dense group of their own.
static moe_status launch_ffn_fp8(const FfnArgs& a, hipStream_t s) {
  const bool dense = a.offsets == nullptr;
  const int bm = f8_tile_m(a.tile_m, a.rows_hint);
  uint8_t* hq = static_cast<uint8_t*>(a.h);
  uint8_t* hs = hq + align_up(static_cast<size_t>(a.cap_rows) * a.I, 256);
  F8Params p1{};
  p1.loc.offsets = a.offsets;
  p1.loc.E_loc = a.E_loc;
  p1.loc.dense_rows = a.cap_rows;
  p1.loc.g[0].n_tiles = a.I / (kF8BN / 2);
  p1.g = F8Group{static_cast<const uint8_t*>(a.x), a.xs, static_cast<const uint8_t*>(a.w13), a.s13,
                 a.H, a.I, 2 * a.I, a.I / (kF8BN / 2), hq, hs};
  F8Params p2 = p1;
  p2.loc.g[0].n_tiles = a.H / kF8BN;
  p2.g = F8Group{hq, hs, static_cast<const uint8_t*>(a.w2), a.s2, a.I, a.H, a.H, a.H / kF8BN, a.y, nullptr};
  const dim3 grid1(static_cast<unsigned>(gemm_grid(tiles_max(bm, a.cap_rows, a.E_loc, dense, p1.loc.g[0].n_tiles, 0, 0, 0))));
  const dim3 grid2(static_cast<unsigned>(gemm_grid(tiles_max(bm, a.cap_rows, a.E_loc, dense, p2.loc.g[0].n_tiles, 0, 0, 0))));

  // shared experts: group 1 only (group 0 keeps no tiles)
  GemmParams q1{}, q2{};
  int bm_sh = 0;
  dim3 gs1, gs2;
  if (a.rows1 > 0) {
    bm_sh = choose_tile_m(a.rows1);
    q1.rows1 = a.rows1;
    q1.E1 = 1;
    q1.g[1] = gate_up_group(a.x1, a.H, a.I1, a.w13_1, nullptr, a.h1);
    q2 = q1;
    const int n_ch = dense_down_chunks(MOE_BF16, a.I1, a.I);
    const int Kc = a.I1 / n_ch;
    GemmGroup gd = down_group(a.h1, a.H, a.I1, a.w2_1, nullptr, a.y1);
    gd.K = Kc;
    gd.a_estride = Kc;
    gd.b_estride = Kc;
    gd.c_estride = a.rows1 * a.H;
    q2.g[1] = gd;
    q2.E1 = n_ch;
    const int bn = col_tile_rows(bm_sh);
    q1.g[1].n_tiles = q1.g[1].N / (bn / 2);
    q2.g[1].n_tiles = q2.g[1].N / bn;
    gs1 = dim3(static_cast<unsigned>(gemm_grid(tiles_max(bm_sh, 0, 1, true, 0, a.rows1, q1.E1, q1.g[1].n_tiles))));
    gs2 = dim3(static_cast<unsigned>(gemm_grid(tiles_max(bm_sh, 0, 1, true, 0, a.rows1, q2.E1, q2.g[1].n_tiles))));
  }

  if (a.t0 && hipEventRecord(a.t0, s) != hipSuccess) return MOE_ERR_HIP;
  if (a.cap_rows > 0) {
    launch_f8<MODE_GATEUP>(bm, grid1, s, p1);
    DBOMOE_CHECK_LAUNCH();
  }
  if (a.rows1 > 0) {
    launch_mfma<MODE_GATEUP, false>(bm_sh, gs1, s, q1);
    DBOMOE_CHECK_LAUNCH();
  }
  if (a.t1 && hipEventRecord(a.t1, s) != hipSuccess) return MOE_ERR_HIP;
  if (a.cap_rows > 0) {
    launch_f8<MODE_DOWN>(bm, grid2, s, p2);
    DBOMOE_CHECK_LAUNCH();
  }
  if (a.rows1 > 0) {
    launch_mfma<MODE_DOWN, false>(bm_sh, gs2, s, q2);
    DBOMOE_CHECK_LAUNCH();
  }
  if (a.t2 && hipEventRecord(a.t2, s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status launch_ffn(const FfnArgs& a, hipStream_t s) {
  if (a.cap_rows == 0 && a.rows1 == 0) return MOE_OK;
  if (a.xs) return launch_ffn_fp8(a, s);
  if (a.act == MOE_F32) return launch_ffn_f32(a, s);
  const bool fp8 = a.wdt == MOE_FP8_E4M3FN;
  const bool dense = a.offsets == nullptr;
  const int bm = a.tile_m > 0 ? a.tile_m : choose_tile_m(a.rows_hint);

  GemmParams p1{};
  p1.offsets = a.offsets;
  p1.E_loc = a.E_loc;
  p1.dense_rows = a.cap_rows;
  p1.rows1 = a.rows1;
  p1.E1 = 1;
  p1.g[0] = gate_up_group(a.x, a.H, a.I, a.w13, a.s13, a.h);
  GemmParams p2 = p1;
  p2.g[0] = down_group(a.h, a.H, a.I, a.w2, a.s2, a.y);
  if (a.rows1 > 0) {
    p1.g[1] = gate_up_group(a.x1, a.H, a.I1, a.w13_1, nullptr, a.h1);
    // The dense down projection in n_ch K chunks, each a dense expert of the
    // group writing its own output slab (summed by the combine).
    const int n_ch = dense_down_chunks(a.act, a.I1, a.I);
    const int Kc = a.I1 / n_ch;
    GemmGroup gd = down_group(a.h1, a.H, a.I1, a.w2_1, nullptr, a.y1);
    gd.K = Kc;
    gd.a_estride = Kc;
    gd.b_estride = Kc;
    gd.c_estride = a.rows1 * a.H;
    p2.g[1] = gd;
    p2.E1 = n_ch;
  }
  {                              // column tiles of the LDS-tiled kernel's width
    const int bn = col_tile_rows(bm);
    p1.g[0].n_tiles = p1.g[0].N / (bn / 2);
    p2.g[0].n_tiles = p2.g[0].N / bn;
    if (a.rows1 > 0) {
      p1.g[1].n_tiles = p1.g[1].N / (bn / 2);
      p2.g[1].n_tiles = p2.g[1].N / bn;
    }
  }
  const dim3 grid1(static_cast<unsigned>(gemm_grid(
      tiles_max(bm, a.cap_rows, a.E_loc, dense, p1.g[0].n_tiles, a.rows1, p1.E1, p1.g[1].n_tiles))));
  const dim3 grid2(static_cast<unsigned>(gemm_grid(
      tiles_max(bm, a.cap_rows, a.E_loc, dense, p2.g[0].n_tiles, a.rows1, p2.E1, p2.g[1].n_tiles))));
  if (a.cap_rows == 0) {   // only the dense group: group 0 keeps no tiles
    p1.offsets = p2.offsets = nullptr;
    p1.dense_rows = p2.dense_rows = 0;
  }
  const bool fp8_launch = fp8 && a.cap_rows > 0;

  const bool full_tiles = a.rows_hint >= 128;
  // 256-wide gate/up tiles for the 128-row block-accumulator launches (see launch_mfma)
  const bool wide = fp8_launch && !full_tiles && bm == 128 && a.rows1 == 0 && fp8w_fits(p1);
  dim3 grid1w = grid1;
  if (wide) {
    p1.g[0].n_tiles = p1.g[0].N / 128;
    grid1w = dim3(static_cast<unsigned>(gemm_grid(tiles_max(bm, a.cap_rows, a.E_loc, dense, p1.g[0].n_tiles, 0, 0, 0))));
  }
  if (a.t0 && hipEventRecord(a.t0, s) != hipSuccess) return MOE_ERR_HIP;
  if (fp8_launch)
    launch_mfma<MODE_GATEUP, true>(bm, grid1w, s, p1, full_tiles, wide);
  else
    launch_mfma<MODE_GATEUP, false>(bm, grid1, s, p1);
  DBOMOE_CHECK_LAUNCH();
  if (a.t1 && hipEventRecord(a.t1, s) != hipSuccess) return MOE_ERR_HIP;
  if (fp8_launch)
    launch_mfma<MODE_DOWN, true>(bm, grid2, s, p2, full_tiles);
  else
    launch_mfma<MODE_DOWN, false>(bm, grid2, s, p2);
  DBOMOE_CHECK_LAUNCH();
  if (a.t2 && hipEventRecord(a.t2, s) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status check_ffn_shapes(moe_dtype act, moe_dtype wdt, int32_t H, int32_t I, int32_t E_loc,
                            const float* s13, const float* s2) {
  if (H <= 0 || I <= 0 || E_loc < 1) return MOE_ERR_INVALID_ARG;
  if (E_loc > 256) return MOE_ERR_UNSUPPORTED;
  if (act == MOE_F32) {
    if (wdt != MOE_F32) return MOE_ERR_UNSUPPORTED;
  } else if (act == MOE_BF16) {
    if (wdt != MOE_BF16 && wdt != MOE_FP8_E4M3FN) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  if (H % 128 || I % 64) return MOE_ERR_UNSUPPORTED;
  if (wdt == MOE_FP8_E4M3FN) {
    if (I % 128) return MOE_ERR_UNSUPPORTED;
    if (H > 128 * 128 || I > 128 * 128) return MOE_ERR_UNSUPPORTED;   // scale rows held in registers
    if (!s13 || !s2) return MOE_ERR_INVALID_ARG;
  } else if (s13 || s2) {
    return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

size_t ffn_ws_bytes(int64_t cap_rows, int32_t I, moe_dtype act) {
  return align_up(static_cast<size_t>(cap_rows) * I * dtype_size(act), 256);
}

}  // namespace dbomoe

using namespace dbomoe;

extern "C" int32_t moe_ffn_auto_tile(moe_dtype act, moe_dtype wdt, int32_t H, int32_t I, int64_t rows_per_expert,
                                     int64_t rows1, int32_t I1) {
  if (check_ffn_shapes(act, wdt, H, I, 1, wdt == MOE_FP8_E4M3FN ? reinterpret_cast<const float*>(16) : nullptr,
                       wdt == MOE_FP8_E4M3FN ? reinterpret_cast<const float*>(16) : nullptr) != MOE_OK ||
      rows_per_expert < 0 || rows1 < 0 || (rows1 > 0 && I1 <= 0))
    return 0;
  if (act == MOE_F32) return 32;
  return choose_tile_m(rows_per_expert);
}

extern "C" size_t moe_ffn_workspace_size(int64_t cap_rows, int32_t I, moe_dtype act) {
  if (cap_rows < 0 || I <= 0 || (act != MOE_F32 && act != MOE_BF16)) return 0;
  return ffn_ws_bytes(cap_rows, I, act);
}

extern "C" size_t moe_ffn_fp8_workspace_size(int64_t cap_rows, int32_t I) {
  if (cap_rows < 0 || I <= 0 || I % kQGroup) return 0;
  return ffn_fp8_ws_bytes(cap_rows, I);
}

extern "C" moe_status moe_grouped_ffn_fp8(const uint8_t* xq_perm, const uint8_t* xq_scale, int32_t H, int32_t I,
                                          const int32_t* offsets, int32_t E_loc, int64_t cap_rows,
                                          const uint8_t* w13, const uint8_t* w2, const float* w13_scale,
                                          const float* w2_scale, void* y_perm, int32_t tile_m, void* ws,
                                          size_t ws_bytes, void* stream) {
  moe_status st = check_ffn_fp8_shapes(H, I, E_loc, w13_scale, w2_scale);
  if (st != MOE_OK) return st;
  if (cap_rows < 0) return MOE_ERR_INVALID_ARG;
  if (!offsets && E_loc != 1) return MOE_ERR_INVALID_ARG;
  if (tile_m != 0 && tile_m != 64 && tile_m != 128) return MOE_ERR_UNSUPPORTED;
  if (cap_rows == 0) return MOE_OK;
  if (cap_rows > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (!xq_perm || !xq_scale || !w13 || !w2 || !y_perm || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned16(xq_perm) || !aligned16(xq_scale) || !aligned16(w13) || !aligned16(w2) || !aligned16(y_perm) ||
      (offsets && !aligned16(offsets)) || !aligned16(w13_scale) || !aligned16(w2_scale) || !aligned256(ws))
    return MOE_ERR_MISALIGNED;
  if (ws_bytes < ffn_fp8_ws_bytes(cap_rows, I)) return MOE_ERR_WORKSPACE;
  FfnArgs a{};
  a.x = xq_perm;
  a.xs = xq_scale;
  a.act = MOE_BF16;
  a.H = H;
  a.I = I;
  a.offsets = offsets;
  a.E_loc = E_loc;
  a.cap_rows = cap_rows;
  a.rows_hint = offsets ? cap_rows / E_loc : cap_rows;
  a.w13 = w13;
  a.w2 = w2;
  a.wdt = MOE_FP8_E4M3FN;
  a.s13 = w13_scale;
  a.s2 = w2_scale;
  a.y = y_perm;
  a.tile_m = tile_m;
  a.h = ws;
  return launch_ffn(a, as_stream(stream));
}

extern "C" moe_status moe_grouped_ffn(const void* x_perm, moe_dtype act, int32_t H, int32_t I,
                                      const int32_t* offsets, int32_t E_loc, int64_t cap_rows,
                                      const void* w13, const void* w2, moe_dtype wdt,
                                      const float* w13_scale, const float* w2_scale,
                                      void* y_perm, int32_t tile_m, void* ws, size_t ws_bytes,
                                      void* stream) {
  moe_status st = check_ffn_shapes(act, wdt, H, I, E_loc, w13_scale, w2_scale);
  if (st != MOE_OK) return st;
  if (cap_rows < 0) return MOE_ERR_INVALID_ARG;
  if (!offsets && E_loc != 1) return MOE_ERR_INVALID_ARG;
  if (tile_m != 0 && tile_m != 32 && tile_m != 64 && tile_m != 128) return MOE_ERR_INVALID_ARG;
  if (cap_rows == 0) return MOE_OK;
  if (cap_rows > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (!x_perm || !w13 || !w2 || !y_perm || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w13) || !aligned16(w2) || !aligned16(y_perm) ||
      (offsets && !aligned16(offsets)) || (w13_scale && !aligned16(w13_scale)) ||
      (w2_scale && !aligned16(w2_scale)) || !aligned256(ws))
    return MOE_ERR_MISALIGNED;
  if (ws_bytes < ffn_ws_bytes(cap_rows, I, act)) return MOE_ERR_WORKSPACE;
  FfnArgs a{};
  a.x = x_perm;
  a.act = act;
  a.H = H;
  a.I = I;
  a.offsets = offsets;
  a.E_loc = E_loc;
  a.cap_rows = cap_rows;
  a.rows_hint = offsets ? cap_rows / E_loc : cap_rows;
  a.w13 = w13;
  a.w2 = w2;
  a.wdt = wdt;
  a.s13 = w13_scale;
  a.s2 = w2_scale;
  a.y = y_perm;
  a.tile_m = tile_m;
  a.h = ws;
  return launch_ffn(a, as_stream(stream));
}
