// Dispatch: stable counting sort of (token, slot) pairs by local expert and the
// row gather into contiguous per-expert rows, for gfx950.
//
// Single-GPU stand-in for the all-to-all dispatch of "[Core/DBO][1/N] Add
// Dual-Batch Overlap mechanism to VLLM", Purpose.  Per-expert counts are produced
// and kept on the device and every buffer is sized for the worst case of T*k
// rows ("DeepEP HT: full decode CUDA graphs via worst-token dispatch", bot
// review 2), so nothing waits on the host.
//
// Four kernels, each a pass over HBM-resident data.  Small batches fuse the
// first three into one workgroup (k_disp_small); mid-sized batches (up to
// 256 local experts and 64k block-histogram entries, i.e. the prefill
// microbatches) count 1024 pairs per workgroup and fold the scan into the rank
// kernel (k_disp_rank_scan: every workgroup sums the histograms of the blocks
// before it and scans the expert totals itself), so they take three launches:
//  1. count   - one workgroup per 256 pairs: LDS histogram of local experts;
//               flags ids outside [0, E).
//  2. scan    - one workgroup: per expert, exclusive prefix over the blocks
//               (stable block bases; several threads per expert, each over a
//               run of blocks), then counts -> offsets (and tile offsets).
//  3. rank    - one workgroup per 256 pairs: stable rank of every pair inside its
//               block from wave ballots (lanes holding the same expert are
//               grouped with a ballot loop; rank = popcount of lower lanes) plus
//               an LDS prefix over the 4 waves; writes perm and inv.
//  4. gather  - one wave per token: the token's k positions are read first
//               (a token with no local pair is skipped), then the row is read
//               from HBM once (16-byte vector loads, several in flight per
//               lane) and written to each of its k destination rows.  The fp8 variant quantises the row on
//               the way (groups of 128 columns, E8M0 scales; fp8_act.h) and
//               writes codes and scale bytes instead.
// A dispatch issued on its own (not beside an FFN launch) folds the rank into
// the gather: k_disp_rank_gather ranks a group of tokens' pairs and moves their
// rows, after the count kernel for mid-sized batches, alone for small ones
// (each workgroup then counts all the pairs from the ids).
#include <mutex>

#include "fp8_act.h"

namespace dbomoe {

constexpr int kPairsPerBlock = 256;
constexpr int kMaxELoc = 1024;

static inline int64_t n_pair_blocks(int64_t T, int32_t k) {
  return (T * k + kPairsPerBlock - 1) / kPairsPerBlock;
}

size_t dispatch_ws_bytes(int64_t T, int32_t k, int32_t E_loc) {
  const int64_t nb = n_pair_blocks(T, k);
  return align_up(static_cast<size_t>(nb) * E_loc * 4, 256) + align_up(static_cast<size_t>(nb) * 4, 256) + 256;
}

struct DispWs {
  int32_t* block_hist;  // [nb][E_loc]; after the scan: stable base of the block inside each expert
  int32_t* block_err;   // [nb]
  int32_t* err;         // [1]
};

// Layout: error word at offset 0 (so it can be found without the shapes),
// then the per-block error flags, then the per-block histograms.
static DispWs carve(void* ws, int64_t nb, int32_t E_loc) {
  (void)E_loc;
  char* b = static_cast<char*>(ws);
  DispWs d;
  d.err = reinterpret_cast<int32_t*>(b);
  b += 256;
  d.block_err = reinterpret_cast<int32_t*>(b);
  b += align_up(static_cast<size_t>(nb) * 4, 256);
  d.block_hist = reinterpret_cast<int32_t*>(b);
  return d;
}

// PPB pairs per workgroup of THREADS threads (PPB / THREADS pairs each).
template <int PPB, int THREADS = PPB>
__global__ __launch_bounds__(THREADS) void k_disp_count(const int32_t* __restrict__ ids, int64_t n_pairs,
                                                        int E_total, int e_begin, int E_loc,
                                                        int32_t* __restrict__ block_hist,
                                                        int32_t* __restrict__ block_err) {
  __shared__ int hist[kMaxELoc];
  for (int e = threadIdx.x; e < E_loc; e += THREADS) hist[e] = 0;
  __syncthreads();
  int bad = 0;
#pragma unroll
  for (int i = 0; i < PPB / THREADS; ++i) {
    const int64_t p = static_cast<int64_t>(blockIdx.x) * PPB + i * THREADS + threadIdx.x;
    if (p < n_pairs) {
      const int e = ids[p];
      if (e < 0 || e >= E_total) {
        bad = 1;
      } else {
        const int le = e - e_begin;
        if (le >= 0 && le < E_loc) atomicAdd(&hist[le], 1);
      }
    }
  }
  bad = __syncthreads_or(bad);
  int32_t* out = block_hist + static_cast<int64_t>(blockIdx.x) * E_loc;
  for (int e = threadIdx.x; e < E_loc; e += THREADS) out[e] = hist[e];
  if (threadIdx.x == 0) block_err[blockIdx.x] = bad;
}

// Exclusive scan of v over the first n <= 1024 threads of a 1024-thread block.
__device__ __forceinline__ int block_excl_scan_1024(int v, int* s_wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < 16 ? s_wsum[lane] : 0;
    const int wi = wave_incl_scan(w);
    if (lane < 16) s_wsum[16 + lane] = wi - w;
  }
  __syncthreads();
  const int r = s_wsum[16 + wave] + incl - v;
  __syncthreads();
  return r;
}

// TPE threads per expert (TPE * E_loc <= 1024): thread (e, part) owns a
// contiguous run of blocks of expert column e, so every load is independent
// and coalesced across experts; the per-part sums are scanned in LDS.
__global__ __launch_bounds__(1024) void k_disp_scan(int64_t nb, int E_loc, int tpe, int tile_m,
                                                    int32_t* __restrict__ block_hist,
                                                    const int32_t* __restrict__ block_err,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ tile_offsets,
                                                    int32_t* __restrict__ err) {
  __shared__ int s_wsum[32];
  __shared__ int s_part[1024];          // [part][e] sums, then their exclusive prefix
  __shared__ int s_total[kMaxELoc];
  const int tid = threadIdx.x;
  const bool active = tid < tpe * E_loc;
  const int e = tid % E_loc;
  const int part = tid / E_loc;
  const int64_t per = (nb + tpe - 1) / tpe;
  const int64_t b0 = active ? min(nb, part * per) : 0;
  const int64_t b1 = active ? min(nb, b0 + per) : 0;
  constexpr int U = 8;
  int sum = 0;
  for (int64_t b = b0; b < b1; b += U) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = b + u < b1 ? block_hist[(b + u) * E_loc + e] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) sum += v[u];
  }
  if (active) s_part[part * E_loc + e] = sum;
  __syncthreads();
  int base = 0;
  if (active)
    for (int q = 0; q < part; ++q) base += s_part[q * E_loc + e];
  if (active && part == tpe - 1) s_total[e] = base + sum;
  // rewrite the blocks with their stable base inside the expert
  for (int64_t b = b0; b < b1; b += U) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = b + u < b1 ? block_hist[(b + u) * E_loc + e] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (b + u < b1) block_hist[(b + u) * E_loc + e] = base;
      base += v[u];
    }
  }
  int any = 0;
  for (int64_t b = tid; b < nb; b += 1024) any |= block_err[b];
  any = __syncthreads_or(any);
  const int cnt = tid < E_loc ? s_total[tid] : 0;
  if (tid < E_loc) counts[tid] = cnt;
  const int off = block_excl_scan_1024(cnt, s_wsum);
  if (tid < E_loc) offsets[tid] = off;
  if (tid == E_loc - 1) offsets[E_loc] = off + cnt;
  if (tile_offsets) {
    const int tiles = (cnt + tile_m - 1) / tile_m;
    const int toff = block_excl_scan_1024(tiles, s_wsum);
    if (tid < E_loc) tile_offsets[tid] = toff;
    if (tid == E_loc - 1) tile_offsets[E_loc] = toff + tiles;
  }
  if (tid == 0) err[0] = any;
}

__global__ __launch_bounds__(256) void k_disp_rank(const int32_t* __restrict__ ids, int64_t n_pairs,
                                                   int e_begin, int E_loc,
                                                   const int32_t* __restrict__ block_base,
                                                   const int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int wave_cnt[4][kMaxELoc];
  for (int i = threadIdx.x; i < 4 * E_loc; i += 256) wave_cnt[i / E_loc][i % E_loc] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t p = static_cast<int64_t>(blockIdx.x) * kPairsPerBlock + threadIdx.x;
  int le = -1;
  if (p < n_pairs) {
    const int e = ids[p] - e_begin;
    if (e >= 0 && e < E_loc) le = e;
  }
  const bool local = le >= 0;
  // Group the lanes of this wave by expert: one ballot per distinct expert.
  uint64_t remaining = __ballot(local);
  uint64_t mine = 0;
  while (remaining) {
    const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
    const int lead_e = __shfl(le, leader, kWave);
    const uint64_t m = __ballot(local && le == lead_e);
    if (local && le == lead_e) mine = m;
    remaining &= ~m;
  }
  const uint64_t lower = mine & lanemask_lt();
  if (local && lower == 0) wave_cnt[wave][le] = __popcll(mine);
  __syncthreads();
  if (p < n_pairs) {
    int pos = -1;
    if (local) {
      pos = offsets[le] + block_base[static_cast<int64_t>(blockIdx.x) * E_loc + le] + __popcll(lower);
      for (int w = 0; w < wave; ++w) pos += wave_cnt[w][le];
      perm[pos] = static_cast<int32_t>(p);
    }
    inv[p] = pos;
  }
}

// Mid-sized batches: 1024 pairs per workgroup for both the count and this
// kernel.  Workgroup b first sums the block histograms: thread (e, part) adds
// a run of blocks of expert column e (loads coalesced across experts), split
// into the blocks before b (b's stable base inside each expert) and all blocks
// (the expert totals).  Every workgroup then scans the totals into offsets
// itself (no scan launch); workgroup 0 writes counts, offsets, tile offsets
// and the error word.  The ranks of b's 1024 pairs follow as in k_disp_small.
constexpr int kMidPairsPerBlock = 1024;
constexpr int kMidMaxELoc = 256;
constexpr int64_t kMidMaxHist = 65536;    // blocks x local experts summed by each workgroup

__global__ __launch_bounds__(1024) void k_disp_rank_scan(const int32_t* __restrict__ ids, int64_t n_pairs,
                                                         int e_begin, int E_loc, int64_t nb, int parts,
                                                         int tile_m, const int32_t* __restrict__ block_hist,
                                                         const int32_t* __restrict__ block_err,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ tile_offsets,
                                                         int32_t* __restrict__ err,
                                                         int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int s_pre[kMidMaxELoc];        // pairs of expert e in blocks before this one
  __shared__ int s_tot[kMidMaxELoc];        // pairs of expert e in all blocks, then the running position
  __shared__ int s_wcnt[16][kMidMaxELoc];   // this block's count per wave and expert
  __shared__ int s_wsum[32];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int64_t b = blockIdx.x;
  for (int e = tid; e < E_loc; e += 1024) {
    s_pre[e] = 0;
    s_tot[e] = 0;
  }
  for (int i = tid; i < 16 * E_loc; i += 1024) s_wcnt[i / E_loc][i % E_loc] = 0;
  __syncthreads();
  if (tid < parts * E_loc) {
    const int e = tid % E_loc;
    const int part = tid / E_loc;
    const int64_t per = (nb + parts - 1) / parts;
    const int64_t r0 = min(nb, part * per);
    const int64_t r1 = min(nb, r0 + per);
    constexpr int U = 16;
    int pre = 0, tot = 0;
    for (int64_t r = r0; r < r1; r += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = r + u < r1 ? block_hist[(r + u) * E_loc + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        tot += v[u];
        pre += r + u < b ? v[u] : 0;
      }
    }
    if (pre) atomicAdd(&s_pre[e], pre);
    if (tot) atomicAdd(&s_tot[e], tot);
  }
  int any = 0;
  if (b == 0)
    for (int64_t q = tid; q < nb; q += 1024) any |= block_err[q];
  any = __syncthreads_or(any);
  const int cnt = tid < E_loc ? s_tot[tid] : 0;
  const int off = block_excl_scan_1024(cnt, s_wsum);
  if (b == 0) {
    if (tid < E_loc) {
      counts[tid] = cnt;
      offsets[tid] = off;
    }
    if (tid == E_loc - 1) offsets[E_loc] = off + cnt;
    if (tid == 0) err[0] = any;
  }
  if (tile_offsets) {
    const int tiles = (cnt + tile_m - 1) / tile_m;
    const int toff = block_excl_scan_1024(tiles, s_wsum);
    if (b == 0) {
      if (tid < E_loc) tile_offsets[tid] = toff;
      if (tid == E_loc - 1) tile_offsets[E_loc] = toff + tiles;
    }
  }
  if (tid < E_loc) s_tot[tid] = off + s_pre[tid];
  // ranks of this block's pairs: ballot groups per wave, then the lower waves
  const int64_t p = b * kMidPairsPerBlock + tid;
  int le = -1;
  if (p < n_pairs) {
    const int e = ids[p] - e_begin;
    if (e >= 0 && e < E_loc) le = e;
  }
  const bool local = le >= 0;
  uint64_t remaining = __ballot(local);
  uint64_t mine = 0;
  while (remaining) {
    const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
    const int lead_e = __shfl(le, leader, kWave);
    const uint64_t m = __ballot(local && le == lead_e);
    if (local && le == lead_e) mine = m;
    remaining &= ~m;
  }
  const uint64_t lower = mine & lanemask_lt();
  if (local && lower == 0) s_wcnt[wave][le] = __popcll(mine);
  __syncthreads();
  if (p < n_pairs) {
    int pos = -1;
    if (local) {
      pos = s_tot[le] + __popcll(lower);
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w][le];
      perm[pos] = static_cast<int32_t>(p);
    }
    inv[p] = pos;
  }
}

// Exclusive scan of v over a 256-thread block.
__device__ __forceinline__ int block_excl_scan_256(int v, int* s_wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wsum[w];
  __syncthreads();
  return base + incl - v;
}

// The rank kernel of a dispatch issued beside an FFN launch on the other
// stream.  A CU running the fp8-weight gate/up GEMM holds three of its
// workgroups, which leave 32 VGPRs per SIMD lane and about 14 KB of LDS (two
// block-accumulator workgroups leave 80 VGPRs): a workgroup of
// k_disp_rank_scan (1024 threads, 92 VGPRs, 19 KB) only starts once a CU has
// drained.  This variant has 256 threads, 32 VGPRs and 6 KB of LDS, so it fits
// beside the GEMM.  Same blocks of 1024 pairs, same results: the block's pairs
// are ranked in four rounds of 256 in pair order, each round on top of the
// running per-expert position the rounds before it left.  The count kernel
// before it runs 256 threads of four pairs each (12 VGPRs) for the same
// reason, and the row gather after it k_disp_gather_lean.
constexpr int kLeanThreads = 256;

__global__ __launch_bounds__(kLeanThreads) void k_disp_rank_scan_lean(
    const int32_t* __restrict__ ids, int64_t n_pairs, int e_begin, int E_loc, int64_t nb, int parts, int tile_m,
    const int32_t* __restrict__ block_hist, const int32_t* __restrict__ block_err, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tile_offsets, int32_t* __restrict__ err,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int s_pre[kMidMaxELoc];       // pairs of expert e in blocks before this one
  __shared__ int s_run[kMidMaxELoc];       // pairs of expert e in all blocks, then the running position
  __shared__ int s_wcnt[4][kMidMaxELoc];   // this round's count per wave and expert
  __shared__ int s_wsum[4];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int64_t b = blockIdx.x;
  for (int e = tid; e < E_loc; e += kLeanThreads) {
    s_pre[e] = 0;
    s_run[e] = 0;
  }
  __syncthreads();
  if (tid < parts * E_loc) {
    const int e = tid % E_loc;
    const int part = tid / E_loc;
    const int64_t per = (nb + parts - 1) / parts;
    const int64_t r0 = min(nb, part * per);
    const int64_t r1 = min(nb, r0 + per);
    constexpr int U = 4;
    int pre = 0, tot = 0;
    for (int64_t r = r0; r < r1; r += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = r + u < r1 ? block_hist[(r + u) * E_loc + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        tot += v[u];
        pre += r + u < b ? v[u] : 0;
      }
    }
    if (pre) atomicAdd(&s_pre[e], pre);
    if (tot) atomicAdd(&s_run[e], tot);
  }
  int any = 0;
  if (b == 0)
    for (int64_t q = tid; q < nb; q += kLeanThreads) any |= block_err[q];
  any = __syncthreads_or(any);
  const int cnt = tid < E_loc ? s_run[tid] : 0;
  const int off = block_excl_scan_256(cnt, s_wsum);
  if (b == 0) {
    if (tid < E_loc) {
      counts[tid] = cnt;
      offsets[tid] = off;
    }
    if (tid == E_loc - 1) offsets[E_loc] = off + cnt;
    if (tid == 0) err[0] = any;
  }
  if (tile_offsets) {
    const int tiles = (cnt + tile_m - 1) / tile_m;
    const int toff = block_excl_scan_256(tiles, s_wsum);
    if (b == 0) {
      if (tid < E_loc) tile_offsets[tid] = toff;
      if (tid == E_loc - 1) tile_offsets[E_loc] = toff + tiles;
    }
  }
  // every read of the totals is behind the scan's closing barrier
  if (tid < E_loc) s_run[tid] = off + s_pre[tid];
  for (int round = 0; round < kMidPairsPerBlock / kLeanThreads; ++round) {
    const int64_t p0 = b * kMidPairsPerBlock + round * kLeanThreads;
    if (p0 >= n_pairs) break;
    for (int i = tid; i < 4 * E_loc; i += kLeanThreads) s_wcnt[i / E_loc][i % E_loc] = 0;
    __syncthreads();
    const int64_t p = p0 + tid;
    int le = -1;
    if (p < n_pairs) {
      const int e = ids[p] - e_begin;
      if (e >= 0 && e < E_loc) le = e;
    }
    const bool local = le >= 0;
    uint64_t remaining = __ballot(local);
    uint64_t mine = 0;
    while (remaining) {
      const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      const int lead_e = __shfl(le, leader, kWave);
      const uint64_t m = __ballot(local && le == lead_e);
      if (local && le == lead_e) mine = m;
      remaining &= ~m;
    }
    const uint64_t lower = mine & lanemask_lt();
    if (local && lower == 0) s_wcnt[wave][le] = __popcll(mine);
    __syncthreads();
    if (p < n_pairs) {
      int pos = -1;
      if (local) {
        pos = s_run[le] + __popcll(lower);
        for (int w = 0; w < wave; ++w) pos += s_wcnt[w][le];
        perm[pos] = static_cast<int32_t>(p);
      }
      inv[p] = pos;
    }
    __syncthreads();
    if (tid < E_loc) s_run[tid] += s_wcnt[0][tid] + s_wcnt[1][tid] + s_wcnt[2][tid] + s_wcnt[3][tid];
    __syncthreads();
  }
}

// Small batches (few pairs, E_loc <= 256): count, scan and rank in one
// workgroup, so the dispatch is two launches (this and the gather) instead of
// four.  Pairs are taken 1024 at a time in order; inside a chunk a pair's
// stable rank is its rank among same-expert lanes of its wave (ballot groups)
// plus the counts of the lower waves, on top of the expert's running count.
constexpr int kSmallChunk = 1024;
constexpr int kSmallMaxPairs = 2048;
constexpr int kSmallMaxELoc = 256;

__global__ __launch_bounds__(1024) void k_disp_small(const int32_t* __restrict__ ids, int64_t n_pairs,
                                                     int E_total, int e_begin, int E_loc, int tile_m,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ tile_offsets,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                     int32_t* __restrict__ err) {
  __shared__ int s_hist[kSmallMaxELoc];
  __shared__ int s_run[kSmallMaxELoc];      // offsets, then offsets + pairs ranked so far
  __shared__ int s_wcnt[16][kSmallMaxELoc]; // this chunk's count per wave and expert
  __shared__ int s_wsum[32];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E_loc; e += 1024) s_hist[e] = 0;
  __syncthreads();
  int bad = 0;
  for (int64_t p = tid; p < n_pairs; p += 1024) {
    const int e = ids[p];
    if (e < 0 || e >= E_total) {
      bad = 1;
    } else {
      const int le = e - e_begin;
      if (le >= 0 && le < E_loc) atomicAdd(&s_hist[le], 1);
    }
  }
  bad = __syncthreads_or(bad);
  const int cnt = tid < E_loc ? s_hist[tid] : 0;
  const int off = block_excl_scan_1024(cnt, s_wsum);
  if (tid < E_loc) {
    counts[tid] = cnt;
    offsets[tid] = off;
    s_run[tid] = off;
  }
  if (tid == E_loc - 1) offsets[E_loc] = off + cnt;
  if (tile_offsets) {
    const int tiles = (cnt + tile_m - 1) / tile_m;
    const int toff = block_excl_scan_1024(tiles, s_wsum);
    if (tid < E_loc) tile_offsets[tid] = toff;
    if (tid == E_loc - 1) tile_offsets[E_loc] = toff + tiles;
  }
  if (tid == 0) err[0] = bad;
  for (int64_t c0 = 0; c0 < n_pairs; c0 += kSmallChunk) {
    for (int i = tid; i < 16 * E_loc; i += 1024) s_wcnt[i / E_loc][i % E_loc] = 0;
    __syncthreads();
    const int64_t p = c0 + tid;
    int le = -1;
    if (p < n_pairs) {
      const int e = ids[p] - e_begin;
      if (e >= 0 && e < E_loc) le = e;
    }
    const bool local = le >= 0;
    uint64_t remaining = __ballot(local);
    uint64_t mine = 0;
    while (remaining) {
      const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      const int lead_e = __shfl(le, leader, kWave);
      const uint64_t m = __ballot(local && le == lead_e);
      if (local && le == lead_e) mine = m;
      remaining &= ~m;
    }
    const uint64_t lower = mine & lanemask_lt();
    if (local && lower == 0) s_wcnt[wave][le] = __popcll(mine);
    __syncthreads();
    if (p < n_pairs) {
      int pos = -1;
      if (local) {
        pos = s_run[le] + __popcll(lower);
        for (int w = 0; w < wave; ++w) pos += s_wcnt[w][le];
        perm[pos] = static_cast<int32_t>(p);
      }
      inv[p] = pos;
    }
    __syncthreads();
    for (int e = tid; e < E_loc; e += 1024) {
      int add = 0;
      for (int w = 0; w < 16; ++w) add += s_wcnt[w][e];
      s_run[e] += add;
    }
    __syncthreads();
  }
}

// One wave per token; rows are moved as 16-byte chunks, kChunks per lane in
// flight at a time.
constexpr int kChunks = 4;

// Chunks c0 + 64 i + lane (i < kChunks) of a row of row_chunks 16-byte
// chunks; zero past the end of the row.
template <int CH = kChunks>
__device__ __forceinline__ void load_row_chunks(const u32x4_t* __restrict__ src, int c0, int row_chunks, int lane,
                                                u32x4_t (&v)[CH]) {
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = c0 + i * 64 + lane;
    v[i] = c < row_chunks ? src[c] : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// The chunks of v into every destination row of the token: lane j < k of
// my_pos holds the position of pair (t, j), -1 for a pair that is not local.
template <int CH = kChunks>
__device__ __forceinline__ void store_row_chunks(u32x4_t* __restrict__ x_perm, int c0, int row_chunks, int k,
                                                 int my_pos, int lane, const u32x4_t (&v)[CH]) {
  for (int j = 0; j < k; ++j) {
    const int pos = __shfl(my_pos, j, kWave);
    if (pos < 0) continue;
    u32x4_t* dst = x_perm + static_cast<int64_t>(pos) * row_chunks;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = c0 + i * 64 + lane;
      if (c < row_chunks) dst[c] = v[i];
    }
  }
}

// fp8 rows: 8 bf16 per lane per 16-byte chunk, so a 128-column group is 16
// adjacent lanes; their amax is combined with four xor shuffles, then the
// group's E8M0 byte and the E4M3 codes of the chunk.
__device__ __forceinline__ void quant_row_chunks(const u32x4_t (&v)[kChunks], uint32_t (&q)[kChunks][2],
                                                 uint32_t (&sb)[kChunks]) {
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    float f[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[2 * w] = __uint_as_float(v[i][w] << 16);
      f[2 * w + 1] = __uint_as_float(v[i][w] & 0xffff0000u);
    }
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
    sb[i] = e8m0_for_amax(m);
    const float is = e8m0_inv_scale(sb[i]);
    q[i][0] = fp8x4_rne(f[0] * is, f[1] * is, f[2] * is, f[3] * is);
    q[i][1] = fp8x4_rne(f[4] * is, f[5] * is, f[6] * is, f[7] * is);
  }
}

// Codes and scale bytes of the quantised chunks into destination row pos.
__device__ __forceinline__ void store_q8_chunks(uint8_t* __restrict__ xq, uint8_t* __restrict__ xs, int64_t pos,
                                                int c0, int row_chunks, int lane, const uint32_t (&q)[kChunks][2],
                                                const uint32_t (&sb)[kChunks]) {
  const int64_t H = static_cast<int64_t>(row_chunks) * 8;
  const int groups = row_chunks / 16;
  uint8_t* dst = xq + pos * H;
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int c = c0 + i * 64 + lane;
    if (c < row_chunks) {
      *reinterpret_cast<uint2*>(dst + c * 8) = make_uint2(q[i][0], q[i][1]);
      if ((lane & 15) == 0) xs[pos * groups + c / 16] = static_cast<uint8_t>(sb[i]);
    }
  }
}

template <int CH>
__device__ __forceinline__ void gather_rows(const u32x4_t* __restrict__ x, int64_t T, int row_chunks, int k,
                                            const int32_t* __restrict__ inv, u32x4_t* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave; t < T; t += stride) {
    // lane j < k holds the position of pair (t, j); a token without a local
    // pair is skipped before its row is read
    const int my_pos = lane < k ? inv[t * k + lane] : -1;
    if (__ballot(my_pos >= 0) == 0) continue;
    const u32x4_t* src = x + t * row_chunks;
    for (int c0 = 0; c0 < row_chunks; c0 += 64 * CH) {
      u32x4_t v[CH];
      load_row_chunks<CH>(src, c0, row_chunks, lane, v);
      store_row_chunks<CH>(x_perm, c0, row_chunks, k, my_pos, lane, v);
    }
  }
}

__global__ __launch_bounds__(256) void k_disp_gather(const u32x4_t* __restrict__ x, int64_t T, int row_chunks,
                                                     int k, const int32_t* __restrict__ inv,
                                                     u32x4_t* __restrict__ x_perm) {
  gather_rows<kChunks>(x, T, row_chunks, k, inv, x_perm);
}

// The row gather issued beside an FFN launch: two chunks per lane in flight
// (26 VGPRs), so its workgroups fit in the 32 VGPRs per lane that the GEMM's
// resident workgroups leave free.
__global__ __launch_bounds__(256) void k_disp_gather_lean(
    const u32x4_t* __restrict__ x, int64_t T, int row_chunks, int k, const int32_t* __restrict__ inv,
    u32x4_t* __restrict__ x_perm) {
  gather_rows<2>(x, T, row_chunks, k, inv, x_perm);
}

// fp8 gather.  inv == NULL maps row t to row t (plain row quantisation, k = 1).
__global__ __launch_bounds__(256) void k_disp_gather_q8(const u32x4_t* __restrict__ x, int64_t T, int row_chunks,
                                                        int k, const int32_t* __restrict__ inv,
                                                        uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave; t < T; t += stride) {
    // as in the bf16 gather: pair positions in lanes j < k, tokens without a
    // local pair skipped (without inv, k = 1 and row t goes to row t)
    const int my_pos = lane < k ? (inv ? inv[t * k + lane] : 0) : -1;
    if (inv && __ballot(my_pos >= 0) == 0) continue;
    const u32x4_t* src = x + t * row_chunks;
    for (int c0 = 0; c0 < row_chunks; c0 += 64 * kChunks) {
      u32x4_t v[kChunks];
      load_row_chunks(src, c0, row_chunks, lane, v);
      uint32_t q[kChunks][2], sb[kChunks];
      quant_row_chunks(v, q, sb);
      for (int j = 0; j < k; ++j) {
        const int64_t pos = inv ? static_cast<int64_t>(__shfl(my_pos, j, kWave)) : t;
        if (pos < 0) continue;
        store_q8_chunks(xq, xs, pos, c0, row_chunks, lane, q, sb);
      }
    }
  }
}

// Exclusive scan of v over a workgroup of NW waves.
template <int NW>
__device__ __forceinline__ int block_excl_scan_waves(int v, int* s_wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wsum[w];
  __syncthreads();
  return base + incl - v;
}

// Mid-sized batches whose dispatch is issued on its own (not beside an FFN
// launch): the rank and the row gather in one kernel after the count kernel,
// two launches instead of three.  Workgroup g owns the TOK tokens from TOK g
// on, one per wave, and so the pairs from TOK g k on, which it ranks and
// moves:
//  1. each wave reads its token's k ids and, when one of them is local,
//     starts loading the first part of the token's row (the loads stay in
//     flight during steps 2-4: a row does not depend on its positions);
//  2. it sums the count kernel's block histograms (blocks of 1024 pairs) over
//     the blocks before the block that holds its first pair, and over all of
//     them, and counts from the ids the pairs of that block before its first
//     pair: so it knows, per expert, the pairs before its own;
//  3. it scans the expert totals into offsets (workgroup 0 writes counts,
//     offsets, tile offsets and the error word);
//  4. it ranks its pairs in pair order (ballot groups in each wave: lanes
//     holding the same expert, rank = popcount of the lower ones; then the
//     counts of the lower waves) and writes perm and inv;
//  5. each wave moves its token's row to the token's positions (bf16 rows, or
//     fp8 codes and E8M0 bytes).
// The positions are those of the stable counting sort, as in
// k_disp_rank_scan + k_disp_gather.
// TOK = 16 tokens per workgroup; 4 when that leaves fewer than 256
// workgroups (the R1-shaped share's 2048-token microbatches: 128 workgroups
// of 16 left half the CUs idle; dispatch step 22.4-23.4 -> 19.4-19.5 us)
constexpr int kFusedMaxK = 64;
constexpr int64_t kFusedMaxHist = 16384;   // blocks x local experts summed by each workgroup

template <bool Q8, int TOK, bool DIRECT>
__global__ __launch_bounds__(64 * TOK) void k_disp_rank_gather(
    const int32_t* __restrict__ ids, int64_t T, int k, int E_total, int e_begin, int E_loc, int64_t nb, int parts,
    int tile_m,
    const int32_t* __restrict__ block_hist, const int32_t* __restrict__ block_err, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tile_offsets, int32_t* __restrict__ err,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, const u32x4_t* __restrict__ x, int row_chunks,
    void* __restrict__ x_perm, uint8_t* __restrict__ xs) {
  __shared__ int s_pre[kMidMaxELoc];                // pairs of expert e before this workgroup's first pair
  __shared__ int s_run[kMidMaxELoc];                // pairs of expert e in all blocks, then the first position
  constexpr int kThreads = 64 * TOK;
  __shared__ int s_wcnt[TOK][kMidMaxELoc];  // this workgroup's count per wave (token) and expert
  __shared__ int s_wsum[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t g = blockIdx.x;
  const int64_t t = g * TOK + wave;
  const int64_t p_first = g * TOK * k;
  // 1. this wave's token
  int le = -1;
  if (t < T && lane < k) {
    const int e = ids[t * k + lane] - e_begin;
    if (e >= 0 && e < E_loc) le = e;
  }
  const bool token_local = __ballot(le >= 0) != 0;
  const u32x4_t* src = x + t * row_chunks;
  u32x4_t v[kChunks];
  if (token_local) load_row_chunks(src, 0, row_chunks, lane, v);
  for (int e = tid; e < E_loc; e += kThreads) {
    s_pre[e] = 0;
    s_run[e] = 0;
  }
  for (int i = tid; i < TOK * E_loc; i += kThreads) s_wcnt[i / E_loc][i % E_loc] = 0;
  __syncthreads();
  // 2. pairs before this workgroup's, and the totals
  int any = 0;
  if constexpr (DIRECT) {
    // few pairs: every workgroup counts them all from the ids (no count
    // kernel) and flags the ids outside [0, E)
    for (int64_t q = tid; q < T * k; q += kThreads) {
      const int id = ids[q];
      if (id < 0 || id >= E_total) {
        any = 1;
        continue;
      }
      const int e = id - e_begin;
      if (e >= 0 && e < E_loc) {
        atomicAdd(&s_run[e], 1);
        if (q < p_first) atomicAdd(&s_pre[e], 1);
      }
    }
  } else {
    const int64_t cb = p_first / kMidPairsPerBlock;
    if (tid < parts * E_loc) {
      const int e = tid % E_loc;
      const int part = tid / E_loc;
      const int64_t per = (nb + parts - 1) / parts;
      const int64_t r0 = min(nb, part * per);
      const int64_t r1 = min(nb, r0 + per);
      constexpr int U = 8;
      int pre = 0, tot = 0;
      for (int64_t r = r0; r < r1; r += U) {
        int h[U];
#pragma unroll
        for (int u = 0; u < U; ++u) h[u] = r + u < r1 ? block_hist[(r + u) * E_loc + e] : 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          tot += h[u];
          pre += r + u < cb ? h[u] : 0;
        }
      }
      if (pre) atomicAdd(&s_pre[e], pre);
      if (tot) atomicAdd(&s_run[e], tot);
    }
    for (int64_t q = cb * kMidPairsPerBlock + tid; q < p_first; q += kThreads) {   // p_first <= T k
      const int e = ids[q] - e_begin;
      if (e >= 0 && e < E_loc) atomicAdd(&s_pre[e], 1);
    }
    if (g == 0)
      for (int64_t q = tid; q < nb; q += kThreads) any |= block_err[q];
  }
  any = __syncthreads_or(any);
  // 3. offsets
  const int cnt = tid < E_loc ? s_run[tid] : 0;
  const int off = block_excl_scan_waves<TOK>(cnt, s_wsum);
  if (g == 0) {
    if (tid < E_loc) {
      counts[tid] = cnt;
      offsets[tid] = off;
    }
    if (tid == E_loc - 1) offsets[E_loc] = off + cnt;
    if (tid == 0) err[0] = any;
  }
  if (tile_offsets) {
    const int tiles = (cnt + tile_m - 1) / tile_m;
    const int toff = block_excl_scan_waves<TOK>(tiles, s_wsum);
    if (g == 0) {
      if (tid < E_loc) tile_offsets[tid] = toff;
      if (tid == E_loc - 1) tile_offsets[E_loc] = toff + tiles;
    }
  }
  // every read of the totals is behind the scan's closing barrier
  if (tid < E_loc) s_run[tid] = off + s_pre[tid];
  // 4. ranks
  const bool local = le >= 0;
  uint64_t remaining = __ballot(local);
  uint64_t mine = 0;
  while (remaining) {
    const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
    const int lead_e = __shfl(le, leader, kWave);
    const uint64_t m = __ballot(local && le == lead_e);
    if (local && le == lead_e) mine = m;
    remaining &= ~m;
  }
  const uint64_t lower = mine & lanemask_lt();
  if (local && lower == 0) s_wcnt[wave][le] = __popcll(mine);
  __syncthreads();
  int pos = -1;
  if (local) {
    pos = s_run[le] + __popcll(lower);
    for (int w = 0; w < wave; ++w) pos += s_wcnt[w][le];
    perm[pos] = static_cast<int32_t>(t * k + lane);
  }
  if (t < T && lane < k) inv[t * k + lane] = pos;
  // 5. the row (no barrier from here on)
  if (!token_local) return;
  for (int c0 = 0; c0 < row_chunks; c0 += 64 * kChunks) {
    if (c0 > 0) load_row_chunks(src, c0, row_chunks, lane, v);
    if constexpr (Q8) {
      uint32_t q[kChunks][2], sb[kChunks];
      quant_row_chunks(v, q, sb);
      for (int j = 0; j < k; ++j) {
        const int pj = __shfl(pos, j, kWave);
        if (pj >= 0) store_q8_chunks(static_cast<uint8_t*>(x_perm), xs, pj, c0, row_chunks, lane, q, sb);
      }
    } else {
      store_row_chunks(static_cast<u32x4_t*>(x_perm), c0, row_chunks, k, pos, lane, v);
    }
  }
}

static moe_status launch_gather(const DispatchArgs& a, hipStream_t s) {
  int64_t blocks = (a.T + 3) / 4;
  if (a.max_blocks > 0 && blocks > a.max_blocks) blocks = a.max_blocks;
  const int row_chunks = static_cast<int>(static_cast<int64_t>(a.H) * dtype_size(a.act) / 16);
  if (a.x_scale) {
    hipLaunchKernelGGL(k_disp_gather_q8, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const u32x4_t*>(a.x), a.T, row_chunks, a.k, a.inv,
                       static_cast<uint8_t*>(a.x_perm), a.x_scale);
  } else if (a.beside_ffn) {
    hipLaunchKernelGGL(k_disp_gather_lean, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const u32x4_t*>(a.x), a.T, row_chunks, a.k, a.inv,
                       static_cast<u32x4_t*>(a.x_perm));
  } else {
    hipLaunchKernelGGL(k_disp_gather, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const u32x4_t*>(a.x), a.T, row_chunks, a.k, a.inv,
                       static_cast<u32x4_t*>(a.x_perm));
  }
  DBOMOE_CHECK_LAUNCH();
  return MOE_OK;
}

moe_status launch_dispatch_send(const DispatchArgs& a, hipStream_t s) {
  const int E_loc = a.e_end - a.e_begin;
  const int64_t n_pairs = a.T * a.k;
  const int64_t nb = n_pair_blocks(a.T, a.k);
  DispWs w = carve(a.ws, nb, E_loc);
  if (n_pairs <= kSmallMaxPairs && E_loc <= kSmallMaxELoc) {
    hipLaunchKernelGGL(k_disp_small, dim3(1), dim3(1024), 0, s, a.ids, n_pairs, a.E_total, a.e_begin, E_loc,
                       a.tile_m > 0 ? a.tile_m : 1, a.counts, a.offsets, a.tile_m > 0 ? a.tile_offsets : nullptr,
                       a.perm, a.inv, w.err);
    DBOMOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  const int64_t nb_mid = (n_pairs + kMidPairsPerBlock - 1) / kMidPairsPerBlock;
  if (E_loc <= kMidMaxELoc && nb_mid * E_loc <= kMidMaxHist) {
    if (a.beside_ffn)
      hipLaunchKernelGGL((k_disp_count<kMidPairsPerBlock, kLeanThreads>), dim3(static_cast<unsigned>(nb_mid)),
                         dim3(kLeanThreads), 0, s, a.ids, n_pairs, a.E_total, a.e_begin, E_loc, w.block_hist,
                         w.block_err);
    else
      hipLaunchKernelGGL(k_disp_count<kMidPairsPerBlock>, dim3(static_cast<unsigned>(nb_mid)),
                         dim3(kMidPairsPerBlock), 0, s, a.ids, n_pairs, a.E_total, a.e_begin, E_loc, w.block_hist,
                         w.block_err);
    DBOMOE_CHECK_LAUNCH();
    const int nt = a.beside_ffn ? kLeanThreads : 1024;
    const int parts = static_cast<int>(std::min<int64_t>(std::max(1, nt / E_loc), nb_mid));
    if (a.beside_ffn)
      hipLaunchKernelGGL(k_disp_rank_scan_lean, dim3(static_cast<unsigned>(nb_mid)), dim3(kLeanThreads), 0, s,
                         a.ids, n_pairs, a.e_begin, E_loc, nb_mid, parts, a.tile_m > 0 ? a.tile_m : 1,
                         w.block_hist, w.block_err, a.counts, a.offsets, a.tile_m > 0 ? a.tile_offsets : nullptr,
                         w.err, a.perm, a.inv);
    else
      hipLaunchKernelGGL(k_disp_rank_scan, dim3(static_cast<unsigned>(nb_mid)), dim3(1024), 0, s, a.ids,
                         n_pairs, a.e_begin, E_loc, nb_mid, parts, a.tile_m > 0 ? a.tile_m : 1, w.block_hist,
                         w.block_err, a.counts, a.offsets, a.tile_m > 0 ? a.tile_offsets : nullptr, w.err,
                         a.perm, a.inv);
    DBOMOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  if (nb > 0) {
    hipLaunchKernelGGL(k_disp_count<kPairsPerBlock>, dim3(static_cast<unsigned>(nb)), dim3(kPairsPerBlock), 0, s,
                       a.ids, n_pairs, a.E_total, a.e_begin, E_loc, w.block_hist, w.block_err);
    DBOMOE_CHECK_LAUNCH();
  }
  int tpe = 1;
  while (tpe * 2 * E_loc <= 1024 && tpe * 2 <= nb) tpe *= 2;
  hipLaunchKernelGGL(k_disp_scan, dim3(1), dim3(1024), 0, s, nb, E_loc, tpe, a.tile_m > 0 ? a.tile_m : 1,
                     w.block_hist, w.block_err, a.counts, a.offsets,
                     a.tile_m > 0 ? a.tile_offsets : nullptr, w.err);
  DBOMOE_CHECK_LAUNCH();
  if (nb == 0) return MOE_OK;
  hipLaunchKernelGGL(k_disp_rank, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, a.ids, n_pairs, a.e_begin,
                     E_loc, w.block_hist, a.offsets, a.perm, a.inv);
  DBOMOE_CHECK_LAUNCH();
  return MOE_OK;
}

moe_status launch_dispatch_recv(const DispatchArgs& a, hipStream_t s) {
  if (a.T == 0) return MOE_OK;
  return launch_gather(a, s);
}

moe_status launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const int E_loc = a.e_end - a.e_begin;
  const int64_t n_pairs = a.T * a.k;
  const int64_t nb_mid = (n_pairs + kMidPairsPerBlock - 1) / kMidPairsPerBlock;
  const int tok = (a.T + 15) / 16 >= 256 ? 16 : 4;
  const int64_t groups = (a.T + tok - 1) / tok;
  // The mid-sized path with the rank folded into the gather (two launches);
  // beside an FFN launch the lean rank kernel and the gather run instead,
  // and a grid cap on the comm kernels keeps the three-launch form.
  // Few pairs (decode): one kernel whose workgroups each count all the pairs
  // from the ids themselves.
  const bool small = n_pairs <= kSmallMaxPairs && E_loc <= kSmallMaxELoc;
  const bool fused = !a.beside_ffn && a.T > 0 && E_loc <= kMidMaxELoc && a.k <= kFusedMaxK &&
                     (small || nb_mid * E_loc <= kFusedMaxHist) && (a.max_blocks <= 0 || groups <= a.max_blocks);
  if (!fused) {
    const moe_status st = launch_dispatch_send(a, s);
    if (st != MOE_OK) return st;
    return launch_dispatch_recv(a, s);
  }
  DispWs w = carve(a.ws, n_pair_blocks(a.T, a.k), E_loc);
  if (!small) {
    hipLaunchKernelGGL(k_disp_count<kMidPairsPerBlock>, dim3(static_cast<unsigned>(nb_mid)),
                       dim3(kMidPairsPerBlock), 0, s, a.ids, n_pairs, a.E_total, a.e_begin, E_loc, w.block_hist,
                       w.block_err);
    DBOMOE_CHECK_LAUNCH();
  }
  const int parts = static_cast<int>(std::min<int64_t>(std::max(1, 64 * tok / E_loc), nb_mid));
  const int row_chunks = static_cast<int>(static_cast<int64_t>(a.H) * dtype_size(a.act) / 16);
  const int tile_m = a.tile_m > 0 ? a.tile_m : 1;
  int32_t* tile_offsets = a.tile_m > 0 ? a.tile_offsets : nullptr;
  auto launch_fused = [&](auto q8, auto tk) {
    constexpr bool Q8 = decltype(q8)::value;
    constexpr int TOK = decltype(tk)::value;
    if (small)
      hipLaunchKernelGGL((k_disp_rank_gather<Q8, TOK, true>), dim3(static_cast<unsigned>(groups)), dim3(64 * TOK), 0,
                         s, a.ids, a.T, a.k, a.E_total, a.e_begin, E_loc, nb_mid, parts, tile_m, w.block_hist,
                         w.block_err, a.counts, a.offsets, tile_offsets, w.err, a.perm, a.inv,
                         static_cast<const u32x4_t*>(a.x), row_chunks, a.x_perm, Q8 ? a.x_scale : nullptr);
    else
      hipLaunchKernelGGL((k_disp_rank_gather<Q8, TOK, false>), dim3(static_cast<unsigned>(groups)), dim3(64 * TOK), 0,
                         s, a.ids, a.T, a.k, a.E_total, a.e_begin, E_loc, nb_mid, parts, tile_m, w.block_hist,
                         w.block_err, a.counts, a.offsets, tile_offsets, w.err, a.perm, a.inv,
                         static_cast<const u32x4_t*>(a.x), row_chunks, a.x_perm, Q8 ? a.x_scale : nullptr);
  };
  using T16 = std::integral_constant<int, 16>;
  using T4 = std::integral_constant<int, 4>;
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  if (a.x_scale) {
    if (tok == 16) launch_fused(Yes{}, T16{}); else launch_fused(Yes{}, T4{});
  } else {
    if (tok == 16) launch_fused(No{}, T16{}); else launch_fused(No{}, T4{});
  }
  DBOMOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace dbomoe

using namespace dbomoe;

extern "C" size_t moe_dispatch_workspace_size(int64_t T, int32_t k, int32_t E_loc) {
  if (T < 0 || k <= 0 || E_loc <= 0) return 0;
  return dispatch_ws_bytes(T, k, E_loc);
}

extern "C" moe_status moe_dispatch(const void* x, moe_dtype act, int64_t T, int32_t H,
                                   const int32_t* topk_ids, int32_t k, int32_t E_total,
                                   int32_t expert_begin, int32_t expert_end, int32_t tile_m,
                                   int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                                   int32_t* perm, int32_t* inv, void* x_perm,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || H <= 0 || k < 1 || k > 16 || E_total < 1) return MOE_ERR_INVALID_ARG;
  if (expert_begin < 0 || expert_end <= expert_begin || expert_end > E_total) return MOE_ERR_INVALID_ARG;
  const int E_loc = expert_end - expert_begin;
  if (E_loc > kMaxELoc) return MOE_ERR_UNSUPPORTED;
  if (act != MOE_F32 && act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (tile_offsets && tile_m <= 0) return MOE_ERR_INVALID_ARG;
  if (!counts || !offsets || !ws) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !topk_ids || !perm || !inv || !x_perm)) return MOE_ERR_INVALID_ARG;
  if ((static_cast<int64_t>(H) * dtype_size(act)) % 16) return MOE_ERR_MISALIGNED;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(counts) || !aligned16(offsets) ||
      (tile_offsets && !aligned16(tile_offsets)) || !aligned16(perm) || !aligned16(inv) ||
      !aligned16(x_perm) || !aligned256(ws))
    return MOE_ERR_MISALIGNED;
  if (T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < dispatch_ws_bytes(T, k, E_loc)) return MOE_ERR_WORKSPACE;
  DispatchArgs a{x, act, T, H, topk_ids, k, E_total, expert_begin, expert_end, tile_m,
                 counts, offsets, tile_offsets, perm, inv, x_perm, ws, 0, nullptr};
  return launch_dispatch(a, as_stream(stream));
}

// ---- dispatch without a caller workspace ---------------------------------
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid it): the dispatch workspace
// (error word, per-block error flags and histograms) lives in this
// file-scope device array instead.  Each GPU holds its own copy for the life
// of the process.  Its device address is looked up once per device, with that
// device current, on the first call there; host code uses only that address.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kNoAllocMaxDevices];

static moe_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

extern "C" size_t moe_dispatch_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

extern "C" moe_status moe_dispatch_noalloc(const void* x, moe_dtype act, int64_t T, int32_t H,
                                           const int32_t* topk_ids, int32_t k, int32_t E_total,
                                           int32_t expert_begin, int32_t expert_end, int32_t tile_m,
                                           int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                                           int32_t* perm, int32_t* inv, void* x_perm, void* stream) {
  if (T < 0 || H <= 0 || k < 1 || k > 16 || E_total < 1) return MOE_ERR_INVALID_ARG;
  if (expert_begin < 0 || expert_end <= expert_begin || expert_end > E_total) return MOE_ERR_INVALID_ARG;
  const int E_loc = expert_end - expert_begin;
  if (E_loc > kMaxELoc) return MOE_ERR_UNSUPPORTED;
  if (act != MOE_F32 && act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (tile_offsets && tile_m <= 0) return MOE_ERR_INVALID_ARG;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !topk_ids || !perm || !inv || !x_perm)) return MOE_ERR_INVALID_ARG;
  if ((static_cast<int64_t>(H) * dtype_size(act)) % 16) return MOE_ERR_MISALIGNED;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(counts) || !aligned16(offsets) ||
      (tile_offsets && !aligned16(tile_offsets)) || !aligned16(perm) || !aligned16(inv) || !aligned16(x_perm))
    return MOE_ERR_MISALIGNED;
  if (T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (dispatch_ws_bytes(T, k, E_loc) > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const moe_status st = scratch_for_current_device(&ws);
  if (st != MOE_OK) return st;
  // Every word of the workspace a call reads is written earlier in the same
  // call (block histograms and flags by the count kernel, the error word by
  // the scan), so nothing left by an earlier call needs clearing.
  DispatchArgs a{x, act, T, H, topk_ids, k, E_total, expert_begin, expert_end, tile_m,
                 counts, offsets, tile_offsets, perm, inv, x_perm, ws, 0, nullptr};
  return launch_dispatch(a, as_stream(stream));
}

extern "C" moe_status moe_dispatch_send(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E_total,
                                        int32_t expert_begin, int32_t expert_end, int32_t tile_m, int32_t* counts,
                                        int32_t* offsets, int32_t* tile_offsets, int32_t* perm, int32_t* inv,
                                        void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || k > 16 || E_total < 1) return MOE_ERR_INVALID_ARG;
  if (expert_begin < 0 || expert_end <= expert_begin || expert_end > E_total) return MOE_ERR_INVALID_ARG;
  const int E_loc = expert_end - expert_begin;
  if (E_loc > kMaxELoc) return MOE_ERR_UNSUPPORTED;
  if (tile_offsets && tile_m <= 0) return MOE_ERR_INVALID_ARG;
  if (!counts || !offsets || !ws) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !perm || !inv)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(topk_ids) || !aligned16(counts) || !aligned16(offsets) ||
      (tile_offsets && !aligned16(tile_offsets)) || !aligned16(perm) || !aligned16(inv) || !aligned256(ws))
    return MOE_ERR_MISALIGNED;
  if (T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < dispatch_ws_bytes(T, k, E_loc)) return MOE_ERR_WORKSPACE;
  DispatchArgs a{nullptr, MOE_BF16, T, 0, topk_ids, k, E_total, expert_begin, expert_end, tile_m,
                 counts, offsets, tile_offsets, perm, inv, nullptr, ws, 0, nullptr};
  return launch_dispatch_send(a, as_stream(stream));
}

extern "C" moe_status moe_dispatch_recv(const void* x, moe_dtype act, int64_t T, int32_t H, int32_t k,
                                        const int32_t* inv, void* x_perm, uint8_t* xq_scale, void* stream) {
  if (T < 0 || H <= 0 || k < 1 || k > 16) return MOE_ERR_INVALID_ARG;
  if (act != MOE_F32 && act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (xq_scale && (act != MOE_BF16 || H % kQGroup)) return MOE_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(H) * dtype_size(act)) % 16) return MOE_ERR_MISALIGNED;
  if (T == 0) return MOE_OK;
  if (!x || !inv || !x_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(inv) || !aligned16(x_perm) || (xq_scale && !aligned16(xq_scale)))
    return MOE_ERR_MISALIGNED;
  if (T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  DispatchArgs a{};
  a.x = x;
  a.act = act;
  a.T = T;
  a.H = H;
  a.k = k;
  a.inv = const_cast<int32_t*>(inv);
  a.x_perm = x_perm;
  a.x_scale = xq_scale;
  return launch_dispatch_recv(a, as_stream(stream));
}

extern "C" moe_status moe_dispatch_fp8(const void* x, int64_t T, int32_t H, const int32_t* topk_ids, int32_t k,
                                       int32_t E_total, int32_t expert_begin, int32_t expert_end, int32_t tile_m,
                                       int32_t* counts, int32_t* offsets, int32_t* tile_offsets, int32_t* perm,
                                       int32_t* inv, uint8_t* xq_perm, uint8_t* xq_scale, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (H <= 0 || H % kQGroup) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && !xq_scale) return MOE_ERR_INVALID_ARG;
  if (T > 0 && !aligned16(xq_scale)) return MOE_ERR_MISALIGNED;
  // the bf16 checks cover everything else (x_perm alignment, ranges, workspace)
  if (T < 0 || k < 1 || k > 16 || E_total < 1) return MOE_ERR_INVALID_ARG;
  if (expert_begin < 0 || expert_end <= expert_begin || expert_end > E_total) return MOE_ERR_INVALID_ARG;
  const int E_loc = expert_end - expert_begin;
  if (E_loc > kMaxELoc) return MOE_ERR_UNSUPPORTED;
  if (tile_offsets && tile_m <= 0) return MOE_ERR_INVALID_ARG;
  if (!counts || !offsets || !ws) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !topk_ids || !perm || !inv || !xq_perm)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(counts) || !aligned16(offsets) ||
      (tile_offsets && !aligned16(tile_offsets)) || !aligned16(perm) || !aligned16(inv) ||
      !aligned16(xq_perm) || !aligned256(ws))
    return MOE_ERR_MISALIGNED;
  if (T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < dispatch_ws_bytes(T, k, E_loc)) return MOE_ERR_WORKSPACE;
  DispatchArgs a{x, MOE_BF16, T, H, topk_ids, k, E_total, expert_begin, expert_end, tile_m,
                 counts, offsets, tile_offsets, perm, inv, xq_perm, ws, 0, xq_scale};
  return launch_dispatch(a, as_stream(stream));
}

extern "C" moe_status moe_quant_fp8_rows(const void* x, int64_t n, int32_t K, uint8_t* q, uint8_t* scale,
                                         void* stream) {
  if (n < 0 || K <= 0) return MOE_ERR_INVALID_ARG;
  if (K % kQGroup) return MOE_ERR_UNSUPPORTED;
  if (n == 0) return MOE_OK;
  if (!x || !q || !scale) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return MOE_ERR_MISALIGNED;
  DispatchArgs a{};
  a.x = x;
  a.act = MOE_BF16;
  a.T = n;
  a.H = K;
  a.k = 1;
  a.inv = nullptr;
  a.x_perm = q;
  a.x_scale = scale;
  return launch_gather(a, as_stream(stream));
}

extern "C" moe_status moe_get_device_error(const void* dispatch_ws, int32_t* code, void* stream) {
  if (!dispatch_ws || !code) return MOE_ERR_INVALID_ARG;
  if (!aligned256(dispatch_ws)) return MOE_ERR_MISALIGNED;
  if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return MOE_ERR_HIP;
  if (hipMemcpy(code, dispatch_ws, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}
