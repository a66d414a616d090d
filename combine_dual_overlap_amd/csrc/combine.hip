// Combine: weighted gather-reduce of each token's expert outputs, for gfx950.
//
// Single-GPU stand-in for the all-to-all combine of "[Core/DBO][1/N] Add
// Dual-Batch Overlap mechanism to VLLM", Purpose:
//   out[t] = sum_j [inv[t*k+j] >= 0] w[t, j] * y_perm[inv[t*k+j]]  (+ shared[t])
// summed in j order in fp32 and rounded once.  HBM-bound: every dispatched row
// is read once and every token row written once.  One wave per token; the k
// source rows of a chunk are all loaded before any is accumulated, so a wave has
// up to KMAX x CH 16-byte loads in flight.
#include "common.h"

namespace dbomoe {

template <bool BF16>
__device__ __forceinline__ void acc_chunk(float* acc, const u32x4_t& v, float w) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += w * __uint_as_float(v[i] << 16);
      acc[2 * i + 1] += w * __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += w * __uint_as_float(v[i]);
  }
}

template <bool BF16>
__device__ __forceinline__ u32x4_t pack_chunk(const float* acc) {
  if constexpr (BF16) {
    return u32x4_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                   pack_bf16x2(acc[6], acc[7])};
  } else {
    return u32x4_t{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                   __float_as_uint(acc[3])};
  }
}

template <bool BF16, int KMAX, int CH>
__global__ __launch_bounds__(256) void k_combine(const u32x4_t* __restrict__ y, int64_t T, int row_chunks, int k,
                                                 const int32_t* __restrict__ inv, const float* __restrict__ w,
                                                 const u32x4_t* __restrict__ shared, int n_shared,
                                                 u32x4_t* __restrict__ out) {
  constexpr int EPC = BF16 ? 8 : 4;   // elements per 16-byte chunk
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave; t < T; t += stride) {
    const int my_pos = lane < k ? inv[t * k + lane] : -1;
    const float my_w = lane < k ? w[t * k + lane] : 0.f;
    int pos[KMAX];
    float wt[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      pos[j] = __shfl(my_pos, j, kWave);
      wt[j] = __shfl(my_w, j, kWave);
    }
    for (int c0 = 0; c0 < row_chunks; c0 += 64 * CH) {
      u32x4_t v[KMAX][CH];
      // Issue every source row's loads before accumulating any of them
      // (pos[j] is uniform across the wave, so the branches do not diverge).
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (pos[j] >= 0) {
#pragma unroll
          for (int c = 0; c < CH; ++c) {
            const int ci = c0 + c * 64 + lane;
            if (ci < row_chunks) v[j][c] = y[static_cast<int64_t>(pos[j]) * row_chunks + ci];
          }
        }
      }
      float acc[CH][EPC];
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[c][e] = 0.f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (pos[j] >= 0) {
#pragma unroll
          for (int c = 0; c < CH; ++c) acc_chunk<BF16>(acc[c], v[j][c], wt[j]);
        }
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int ci = c0 + c * 64 + lane;
        if (ci < row_chunks) {
          for (int sl = 0; sl < n_shared; ++sl)
            acc_chunk<BF16>(acc[c], shared[(sl * T + t) * row_chunks + ci], 1.0f);
          out[t * row_chunks + ci] = pack_chunk<BF16>(acc[c]);
        }
      }
    }
  }
}

template <bool BF16>
static void launch_k(int kmax, dim3 g, hipStream_t s, const u32x4_t* y, int64_t T, int rc, int k,
                     const int32_t* inv, const float* w, const u32x4_t* sh, int nsh, u32x4_t* out) {
  if (kmax <= 4)
    hipLaunchKernelGGL((k_combine<BF16, 4, 4>), g, dim3(256), 0, s, y, T, rc, k, inv, w, sh, nsh, out);
  else if (kmax <= 8)
    hipLaunchKernelGGL((k_combine<BF16, 8, 2>), g, dim3(256), 0, s, y, T, rc, k, inv, w, sh, nsh, out);
  else
    hipLaunchKernelGGL((k_combine<BF16, 16, 1>), g, dim3(256), 0, s, y, T, rc, k, inv, w, sh, nsh, out);
}

moe_status launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return MOE_OK;
  const int rc = static_cast<int>(static_cast<int64_t>(a.H) * dtype_size(a.act) / 16);
  int64_t blocks = (a.T + 3) / 4;
  if (a.max_blocks > 0 && blocks > a.max_blocks) blocks = a.max_blocks;
  const dim3 g(static_cast<unsigned>(blocks));
  const auto* y = static_cast<const u32x4_t*>(a.y);
  const auto* sh = static_cast<const u32x4_t*>(a.shared);
  auto* out = static_cast<u32x4_t*>(a.out);
  const int nsh = sh ? (a.n_shared > 0 ? a.n_shared : 1) : 0;
  if (a.act == MOE_BF16)
    launch_k<true>(a.k, g, s, y, a.T, rc, a.k, a.inv, a.w, sh, nsh, out);
  else
    launch_k<false>(a.k, g, s, y, a.T, rc, a.k, a.inv, a.w, sh, nsh, out);
  DBOMOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace dbomoe

using namespace dbomoe;

extern "C" moe_status moe_combine(const void* y_perm, moe_dtype act, int64_t T, int32_t H, int32_t k,
                                  const int32_t* inv, const float* topk_w, const void* shared_out,
                                  void* out, void* stream) {
  if (T < 0 || H <= 0 || k < 1 || k > 16) return MOE_ERR_INVALID_ARG;
  if (act != MOE_F32 && act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_perm || !inv || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  if (out == y_perm || (shared_out && out == shared_out)) return MOE_ERR_INVALID_ARG;
  if ((static_cast<int64_t>(H) * dtype_size(act)) % 16) return MOE_ERR_MISALIGNED;
  if (!aligned16(y_perm) || !aligned16(inv) || !aligned16(topk_w) || !aligned16(out) ||
      (shared_out && !aligned16(shared_out)))
    return MOE_ERR_MISALIGNED;
  CombineArgs a{y_perm, act, T, H, k, inv, topk_w, shared_out, out, 0, shared_out ? 1 : 0};
  return launch_combine(a, as_stream(stream));
}
