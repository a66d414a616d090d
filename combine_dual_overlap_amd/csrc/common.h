// Internal helpers shared by the HIP kernels of the DBO MoE layer (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "dbomoe.h"

namespace dbomoe {

typedef uint16_t bf16_t;                                        // raw bf16 bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));   // MFMA operand
typedef float f32x4_t __attribute__((ext_vector_type(4)));      // 16x16 MFMA accumulator
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // 16-byte vector

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Two floats -> packed bf16x2 (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sum across a 64-lane wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
  return v;
}

// Mask of lanes below the calling lane.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

inline size_t dtype_size(moe_dtype d) {
  switch (d) {
    case MOE_F32: return 4;
    case MOE_BF16: return 2;
    case MOE_FP8_E4M3FN: return 1;
  }
  return 0;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }


#define DBOMOE_CHECK_LAUNCH()                                  \
  do {                                                         \
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;   \
  } while (0)

// ---- internal launchers (no argument validation; callers validate) --------

struct RouteArgs {
  const void* x; moe_dtype act; int64_t T; int32_t H;
  const void* w_router; const float* bias; const int32_t* forced;
  moe_route_params p; float* logits; int32_t* ids; float* w; float* part;
};
int route_splits(int64_t T, int32_t H, int32_t E);
size_t route_ws_bytes(int64_t T, int32_t H, int32_t E);
moe_status launch_route(const RouteArgs& a, hipStream_t s);

struct DispatchArgs {
  const void* x; moe_dtype act; int64_t T; int32_t H;
  const int32_t* ids; int32_t k; int32_t E_total; int32_t e_begin; int32_t e_end; int32_t tile_m;
  int32_t* counts; int32_t* offsets; int32_t* tile_offsets; int32_t* perm; int32_t* inv;
  void* x_perm; void* ws; int32_t max_blocks;
  uint8_t* x_scale;        // non-NULL: x_perm receives fp8 codes and x_scale the E8M0 bytes [rows][H/128]
  bool beside_ffn;         // issued to run beside an FFN launch on the other stream: kernels that fit
                           // into what the GEMM's resident workgroups leave free on a CU
};
size_t dispatch_ws_bytes(int64_t T, int32_t k, int32_t E_loc);
moe_status launch_dispatch(const DispatchArgs& a, hipStream_t s);
// The two phases of launch_dispatch: send = count, scan and rank (counts,
// offsets, perm, inv); recv = the row gather (x_perm, or fp8 rows + scales).
moe_status launch_dispatch_send(const DispatchArgs& a, hipStream_t s);
moe_status launch_dispatch_recv(const DispatchArgs& a, hipStream_t s);

struct FfnArgs {
  const void* x; moe_dtype act; int32_t H; int32_t I;
  const int32_t* offsets; int32_t E_loc; int64_t cap_rows; int64_t rows_hint;
  const void* w13; const void* w2; moe_dtype wdt; const float* s13; const float* s2;
  void* y; int32_t tile_m; void* h;
  hipEvent_t t0, t1, t2;   // optional timing events around the two GEMMs
  // Optional dense expert computed in the same launches (the always-on shared
  // experts): rows1 rows of x1, intermediate size I1, weights in the activation
  // dtype, output y1 [rows1, H], intermediate h1 [rows1, I1].
  const void* x1; int64_t rows1; int32_t I1; const void* w13_1; const void* w2_1; void* y1; void* h1;
  // fp8 activations: x holds E4M3 codes and xs their E8M0 bytes [cap_rows][H/128];
  // the routed experts then run fp8 x fp8 MFMAs and h (in `h`, see
  // ffn_fp8_ws_bytes) is quantised the same way.  NULL: x is in act.
  const uint8_t* xs;
};
moe_status launch_ffn(const FfnArgs& a, hipStream_t s);
moe_status check_ffn_fp8_shapes(int32_t H, int32_t I, int32_t E_loc, const float* s13, const float* s2);
size_t ffn_fp8_ws_bytes(int64_t cap_rows, int32_t I);
moe_status check_ffn_shapes(moe_dtype act, moe_dtype wdt, int32_t H, int32_t I, int32_t E_loc,
                            const float* s13, const float* s2);
// K chunks of a dense (shared) expert's down projection run in the grouped
// launch: each chunk writes its own partial output slab [rows1, H].
int dense_down_chunks(moe_dtype act, int32_t I1, int32_t I);
size_t ffn_ws_bytes(int64_t cap_rows, int32_t I, moe_dtype act);

struct CombineArgs {
  const void* y; moe_dtype act; int64_t T; int32_t H; int32_t k;
  const int32_t* inv; const float* w; const void* shared; void* out; int32_t max_blocks;
  int32_t n_shared;        // slabs [n_shared][T, H] added with weight 1 (1 if shared is set)
  bool beside_ffn;         // as in DispatchArgs
};
moe_status launch_combine(const CombineArgs& a, hipStream_t s);

moe_status check_route_params(const moe_route_params* p);

}  // namespace dbomoe
