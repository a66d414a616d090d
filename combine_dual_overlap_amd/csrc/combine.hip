// Combine: weighted gather-reduce of each token's expert outputs, for gfx950.
//
// Single-GPU stand-in for the all-to-all combine of "[Core/DBO][1/N] Add
// Dual-Batch Overlap mechanism to VLLM", Purpose:
//   out[t] = sum_j [inv[t*k+j] >= 0] w[t, j] * y_perm[inv[t*k+j]]  (+ shared[t])
// summed in j order in fp32 and rounded once.  HBM-bound: every dispatched row
// is read once and every token row written once.
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

// One wave per (token, block of 64 x CH chunks of the row): the token's k
// dispatched rows and the shared slabs are summed as RMAX source rows, all
// loads of a block issued before any is accumulated (one memory round trip),
// and small batches spread each row over several waves.
template <bool BF16, int RMAX, int CH>
__global__ __launch_bounds__(256) void k_combine(const u32x4_t* __restrict__ y, int64_t T, int row_chunks, int k,
                                                 const int32_t* __restrict__ inv, const float* __restrict__ w,
                                                 const u32x4_t* __restrict__ shared, int n_shared,
                                                 u32x4_t* __restrict__ out) {
  constexpr int EPC = BF16 ? 8 : 4;   // elements per 16-byte chunk
  constexpr int BLK = 64 * CH;        // chunks per work item
  const int lane = threadIdx.x & 63;
  const int nblk = (row_chunks + BLK - 1) / BLK;
  const int64_t items = T * nblk;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); it < items; it += nwaves) {
    const int64_t t = it / nblk;
    const int c_begin = static_cast<int>(it % nblk) * BLK;
    const int my_pos = lane < k ? inv[t * k + lane] : -1;
    const float my_w = lane < k ? w[t * k + lane] : 0.f;
    // source rows: j < k the dispatched rows (skipped if not local), then the
    // shared slabs with weight 1; wave-uniform.
    const u32x4_t* src[RMAX];
    float wt[RMAX];
#pragma unroll
    for (int j = 0; j < RMAX; ++j) {
      const int pj = __shfl(my_pos, j < k ? j : 0, kWave);
      const float wj = __shfl(my_w, j < k ? j : 0, kWave);
      if (j < k) {
        src[j] = pj >= 0 ? y + static_cast<int64_t>(pj) * row_chunks : nullptr;
        wt[j] = wj;
      } else if (j < k + n_shared) {
        src[j] = shared + (static_cast<int64_t>(j - k) * T + t) * row_chunks;
        wt[j] = 1.f;
      } else {
        src[j] = nullptr;
        wt[j] = 0.f;
      }
    }
    u32x4_t v[RMAX][CH];
#pragma unroll
    for (int j = 0; j < RMAX; ++j) {
      if (src[j]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int ci = c_begin + c * 64 + lane;
          if (ci < row_chunks) v[j][c] = src[j][ci];
        }
      }
    }
    float acc[CH][EPC];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[c][e] = 0.f;
#pragma unroll
    for (int j = 0; j < RMAX; ++j) {
      if (src[j]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) acc_chunk<BF16>(acc[c], v[j][c], wt[j]);
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = c_begin + c * 64 + lane;
      if (ci < row_chunks) out[t * row_chunks + ci] = pack_chunk<BF16>(acc[c]);
    }
  }
}

// The combine issued beside an FFN launch on the other stream.  A CU running
// the fp8-weight gate/up GEMM holds three of its workgroups (160 VGPRs per
// lane each, one wave per SIMD each), which leave 32 VGPRs per SIMD lane; the
// block-accumulator form holds two (216 VGPRs), which leave 80.  A workgroup
// of k_combine (up to 110 VGPRs) fits in neither: it waits for a GEMM
// workgroup to retire and then holds its slot.  This variant takes one
// 64-chunk block per wave and the source rows two at a time, with the row
// addresses and weights wave-uniform (scalar registers), in 31 VGPRs, so that
// its workgroups fit beside the GEMM's.  (At 64 VGPRs it fitted only beside
// two GEMM workgroups: the R1-shaped layer 0.908 -> 0.901 ms in DBO.)  The same
// products are summed in the same order as in k_combine, so the output is
// bitwise the same.
template <bool BF16>
__global__ __launch_bounds__(256) void k_combine_lean(
    const u32x4_t* __restrict__ y, int64_t T, int row_chunks, int k, const int32_t* __restrict__ inv,
    const float* __restrict__ w, const u32x4_t* __restrict__ shared, int n_shared, u32x4_t* __restrict__ out) {
  constexpr int EPC = BF16 ? 8 : 4;
  constexpr int G = 2;                // source rows loaded together
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = (row_chunks + 63) / 64;
  const int rows = k + n_shared;
  const int64_t items = T * nblk;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * 4 + wave; it < items; it += nwaves) {
    const int64_t t = it / nblk;
    const int ci = static_cast<int>(it % nblk) * 64 + lane;
    const bool in = ci < row_chunks;
    const int my_pos = lane < k ? inv[t * k + lane] : -1;
    const float my_w = lane < k ? w[t * k + lane] : 0.f;
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    for (int j0 = 0; j0 < rows; j0 += G) {
      float wt[G];
      u32x4_t v[G];
      unsigned used = 0;   // bit g: source row j0 + g exists (its load is issued)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int j = j0 + g;
        const int pj = __builtin_amdgcn_readfirstlane(__shfl(my_pos, j < k ? j : 0, kWave));
        const float wj =
            __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(__shfl(my_w, j < k ? j : 0, kWave))));
        const u32x4_t* src = nullptr;
        wt[g] = 1.f;
        if (j < k) {
          if (pj >= 0) src = y + static_cast<int64_t>(pj) * row_chunks;
          wt[g] = wj;
        } else if (j < rows) {
          src = shared + (static_cast<int64_t>(j - k) * T + t) * row_chunks;
        }
        if (src) {
          used |= 1u << g;
          if (in) v[g] = src[ci];
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (used & (1u << g)) acc_chunk<BF16>(acc, v[g], wt[g]);
    }
    if (in) out[t * row_chunks + ci] = pack_chunk<BF16>(acc);
  }
}

// Rows per token = k + shared slabs (at most 32).  Two chunks per lane when
// there are enough tokens to fill the GPU, one otherwise.
template <bool BF16>
static void launch_k(int rows, int64_t T, int rc, int64_t max_blocks, hipStream_t s, const u32x4_t* y, int k,
                     const int32_t* inv, const float* w, const u32x4_t* sh, int nsh, u32x4_t* out) {
  const bool wide = T * ((rc + 127) / 128) >= 4096;
  const int blk = wide && rows <= 8 ? 128 : 64;
  int64_t blocks = (T * ((rc + blk - 1) / blk) + 3) / 4;
  if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
  const dim3 g(static_cast<unsigned>(blocks));
  if (rows <= 8 && blk == 128)
    hipLaunchKernelGGL((k_combine<BF16, 8, 2>), g, dim3(256), 0, s, y, T, rc, k, inv, w, sh, nsh, out);
  else if (rows <= 8)
    hipLaunchKernelGGL((k_combine<BF16, 8, 1>), g, dim3(256), 0, s, y, T, rc, k, inv, w, sh, nsh, out);
  else if (rows <= 16)
    hipLaunchKernelGGL((k_combine<BF16, 16, 1>), g, dim3(256), 0, s, y, T, rc, k, inv, w, sh, nsh, out);
  else
    hipLaunchKernelGGL((k_combine<BF16, 32, 1>), g, dim3(256), 0, s, y, T, rc, k, inv, w, sh, nsh, out);
}

moe_status launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return MOE_OK;
  const int rc = static_cast<int>(static_cast<int64_t>(a.H) * dtype_size(a.act) / 16);
  const auto* y = static_cast<const u32x4_t*>(a.y);
  const auto* sh = static_cast<const u32x4_t*>(a.shared);
  auto* out = static_cast<u32x4_t*>(a.out);
  const int nsh = sh ? (a.n_shared > 0 ? a.n_shared : 1) : 0;
  if (a.k + nsh > 32) return MOE_ERR_UNSUPPORTED;
  if (a.beside_ffn) {
    int64_t blocks = (a.T * ((rc + 63) / 64) + 3) / 4;
    if (a.max_blocks > 0 && blocks > a.max_blocks) blocks = a.max_blocks;
    const dim3 g(static_cast<unsigned>(blocks));
    if (a.act == MOE_BF16)
      hipLaunchKernelGGL(k_combine_lean<true>, g, dim3(256), 0, s, y, a.T, rc, a.k, a.inv, a.w, sh, nsh, out);
    else
      hipLaunchKernelGGL(k_combine_lean<false>, g, dim3(256), 0, s, y, a.T, rc, a.k, a.inv, a.w, sh, nsh, out);
  } else if (a.act == MOE_BF16) {
    launch_k<true>(a.k + nsh, a.T, rc, a.max_blocks, s, y, a.k, a.inv, a.w, sh, nsh, out);
  } else {
    launch_k<false>(a.k + nsh, a.T, rc, a.max_blocks, s, y, a.k, a.inv, a.w, sh, nsh, out);
  }
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
