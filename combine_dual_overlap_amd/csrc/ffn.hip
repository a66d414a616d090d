// Grouped SwiGLU expert FFN for gfx950: gate/up GEMM with SiLU-mul fused into
// its epilogue, then the down GEMM, each over all local experts in one launch.
//
// The expert compute of "[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to
// VLLM" (performance discussion: batched MoE GEMM + act-and-mul).  Reading:
// W13 = [gate rows 0..I) ; up rows I..2I)], h = silu(gate) * up rounded to the
// activation dtype, y = h W2^T.
#include "gemm_mfma.h"

namespace dbomoe {

static int choose_tile_m(int64_t rows_hint) {
  if (rows_hint <= 40) return 32;
  if (rows_hint <= 96) return 64;
  return 128;
}

template <int MODE, bool FP8>
static void launch_mfma(int bm, dim3 grid, hipStream_t s, const GemmParams& g) {
  if (bm == 32)
    hipLaunchKernelGGL((k_gemm_nt<32, 1, 4, MODE, FP8>), grid, dim3(256), 0, s, g);
  else if (bm == 64)
    hipLaunchKernelGGL((k_gemm_nt<64, 2, 2, MODE, FP8>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((k_gemm_nt<128, 2, 2, MODE, FP8>), grid, dim3(256), 0, s, g);
}

moe_status launch_ffn(const FfnArgs& a, hipStream_t s) {
  if (a.cap_rows == 0) return MOE_OK;
  const bool f32 = a.act == MOE_F32;
  const bool fp8 = a.wdt == MOE_FP8_E4M3FN;
  const bool dense = a.offsets == nullptr;
  const int bm = f32 ? 32 : (a.tile_m > 0 ? a.tile_m : choose_tile_m(a.rows_hint));

  GemmParams g1{};
  g1.A = static_cast<const bf16_t*>(a.x);
  g1.lda = a.H;
  g1.B = a.w13;
  g1.ldb = a.H;
  g1.bscale = a.s13;
  g1.K = a.H;
  g1.N = a.I;
  g1.b_rows = 2 * a.I;
  g1.offsets = a.offsets;
  g1.E_loc = a.E_loc;
  g1.dense_rows = a.cap_rows;
  g1.C = a.h;
  g1.ldc = a.I;
  g1.n_tiles = a.I / (kBN / 2);
  const int64_t row_tiles = max_row_tiles(a.cap_rows, a.E_loc, bm, dense);
  const dim3 grid1(static_cast<unsigned>(gemm_grid(row_tiles, g1.n_tiles)));

  GemmParams g2 = g1;
  g2.A = static_cast<const bf16_t*>(a.h);
  g2.lda = a.I;
  g2.B = a.w2;
  g2.ldb = a.I;
  g2.bscale = a.s2;
  g2.K = a.I;
  g2.N = a.H;
  g2.b_rows = a.H;
  g2.C = a.y;
  g2.ldc = a.H;
  g2.n_tiles = a.H / kBN;
  const dim3 grid2(static_cast<unsigned>(gemm_grid(row_tiles, g2.n_tiles)));

  if (a.t0 && hipEventRecord(a.t0, s) != hipSuccess) return MOE_ERR_HIP;
  if (f32)
    hipLaunchKernelGGL(k_gemm_nt_f32<MODE_GATEUP>, grid1, dim3(256), 0, s, g1);
  else if (fp8)
    launch_mfma<MODE_GATEUP, true>(bm, grid1, s, g1);
  else
    launch_mfma<MODE_GATEUP, false>(bm, grid1, s, g1);
  DBOMOE_CHECK_LAUNCH();
  if (a.t1 && hipEventRecord(a.t1, s) != hipSuccess) return MOE_ERR_HIP;
  if (f32)
    hipLaunchKernelGGL(k_gemm_nt_f32<MODE_DOWN>, grid2, dim3(256), 0, s, g2);
  else if (fp8)
    launch_mfma<MODE_DOWN, true>(bm, grid2, s, g2);
  else
    launch_mfma<MODE_DOWN, false>(bm, grid2, s, g2);
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

extern "C" size_t moe_ffn_workspace_size(int64_t cap_rows, int32_t I, moe_dtype act) {
  if (cap_rows < 0 || I <= 0 || (act != MOE_F32 && act != MOE_BF16)) return 0;
  return ffn_ws_bytes(cap_rows, I, act);
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
  FfnArgs a{x_perm, act, H, I, offsets, E_loc, cap_rows, offsets ? cap_rows / E_loc : cap_rows,
            w13, w2, wdt, w13_scale, w2_scale, y_perm, tile_m, ws, nullptr, nullptr, nullptr};
  return launch_ffn(a, as_stream(stream));
}
