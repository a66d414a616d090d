// Router logits + top-k routing (one wave per token) for gfx950.
//
// The pages describe the router only as the compute that precedes dispatch in
// each microbatch ("[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM",
// Purpose); the routing rule is the stated reading in dbomoe.h.
//
// Logits: x [T, H] . W_r [E, H]^T on bf16 MFMA (fp32 SIMT for fp32 inputs) with
// split-K into S fp32 partial slabs so that a 2k-token, H = 7168 microbatch still
// fills the chip; the top-k kernel adds the S partials in a fixed order (so the
// logits are deterministic), adds the bias and writes the logits it compares.
// Selection compares logits, never rounded probabilities: softmax and sigmoid are
// monotone, so the order of experts is the order of their logits.
#include "gemm_mfma.h"

namespace dbomoe {

// Split-K factor of the router GEMM: doubled while the grid has fewer than
// 256 workgroups and each split keeps at least 128 of K (a 128-wide stage),
// at most 16 splits.
// The decode layer's 128-token microbatches take 16 splits of 128 (DBO 0.484
// -> 0.481 ms against 8 of 256); the prefill and R1-shaped shapes keep 2.
int route_splits(int64_t T, int32_t H, int32_t E) {
  const int64_t base = (T + 31) / 32 * ((E + kBN - 1) / kBN);
  int S = 1;
  while (S < 16 && base * S < 256 && H / (S * 2) >= 128 && H % (S * 2 * kBK) == 0) S *= 2;
  return S;
}

size_t route_ws_bytes(int64_t T, int32_t H, int32_t E) {
  return align_up(static_cast<size_t>(route_splits(T, H, E)) * T * E * sizeof(float), 256);
}

moe_status check_route_params(const moe_route_params* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->E < 1 || p->E > 256 || p->k < 1 || p->k > 16 || p->k > p->E) return MOE_ERR_INVALID_ARG;
  if (p->score != MOE_SCORE_SOFTMAX && p->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (p->n_groups < 1 || p->n_groups > 64 || p->E % p->n_groups) return MOE_ERR_INVALID_ARG;
  if (p->n_groups > 1) {
    const int per = p->E / p->n_groups;
    if (p->topk_groups < 1 || p->topk_groups > p->n_groups) return MOE_ERR_INVALID_ARG;
    if (p->group_topn < 1 || p->group_topn > 4 || p->group_topn > per) return MOE_ERR_INVALID_ARG;
    if (p->k > p->topk_groups * per) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

struct TopkParams {
  const float* part; int S; int64_t T; int E;
  const float* bias; const int32_t* forced; moe_route_params rp;
  float* logits; int32_t* ids; float* w;
};

// (value desc, index asc) "better than" for the wave arg-max.
__device__ __forceinline__ bool better(float v, int e, float ov, int oe) {
  return v > ov || (v == ov && e < oe);
}

__device__ __forceinline__ void wave_argmax(float& v, int& e) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) {
    const float ov = __shfl_xor(v, d, kWave);
    const int oe = __shfl_xor(e, d, kWave);
    if (better(ov, oe, v, e)) { v = ov; e = oe; }
  }
}


// Selection and weights of token t, one wave: lane l holds the logits of
// experts l, l+64, ... in v (-inf beyond E); s_score is the wave's 256-float
// LDS scratch for group scores.
__device__ __forceinline__ void topk_token(const TopkParams& p, int64_t t, const float* v, float* s_score) {
  const int lane = threadIdx.x & 63;
  const int E = p.E;
  const int k = p.rp.k;
  const float NEG = -INFINITY;

  const bool softmax = p.rp.score == MOE_SCORE_SOFTMAX;
  float lmax = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
  lmax = wave_max_f(lmax);
  float denom = 0.f;
  if (softmax) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < E) denom += expf(v[i] - lmax);
    denom = wave_sum_f(denom);
  }

  // Candidate mask: bit i of lane l <=> expert l + 64 i may be selected.
  unsigned cand = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (lane + 64 * i < E) cand |= 1u << i;

  if (!softmax && p.rp.n_groups > 1 && !p.forced) {
    // Group-limited selection: score each group by the sum of its group_topn
    // best sigmoid scores, keep the topk_groups best groups.
    const int G = p.rp.n_groups, per = E / G;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < E) s_score[lane + 64 * i] = 1.0f / (1.0f + expf(-v[i]));
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float gs = NEG;
    if (lane < G) {
      float top[4] = {NEG, NEG, NEG, NEG};
      const int n = p.rp.group_topn;
      for (int j = 0; j < per; ++j) {
        float x = s_score[lane * per + j];
        // insert into the descending list top[0..n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q < n && x > top[q]) { const float tmp = top[q]; top[q] = x; x = tmp; }
        }
      }
      gs = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < n) gs += top[q];
    }
    uint64_t kept = 0;
    float gv = gs;
    for (int r = 0; r < p.rp.topk_groups; ++r) {
      float bv = (lane < G && !((kept >> lane) & 1ull)) ? gv : NEG;
      int be = (lane < G && !((kept >> lane) & 1ull)) ? lane : 1 << 30;
      wave_argmax(bv, be);
      kept |= 1ull << be;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((kept >> (e / per)) & 1ull)) cand &= ~(1u << i);
    }
  }

  // Slot j is kept by lane j (its expert and logit).  The loops run k times
  // instead of being unrolled for the largest k: the code runs once per token,
  // so its size, not its instruction count, is what costs (each new
  // instruction-cache line is a memory round trip).
  int my_e = 0;
  float my_v = NEG;
#pragma unroll 1
  for (int j = 0; j < k; ++j) {
    int be;
    float bv;
    if (p.forced) {
      be = p.forced[t * k + j];
      bv = NEG;
      if (be >= 0 && be < E) {
        const int i = be >> 6, src = be & 63;
        const float mine = i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
        bv = __shfl(mine, src, kWave);
      }
    } else {
      bv = NEG;
      be = 1 << 30;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (((cand >> i) & 1u) && better(v[i], e, bv, be)) { bv = v[i]; be = e; }
      }
      wave_argmax(bv, be);
      if ((be & 63) == lane) cand &= ~(1u << (be >> 6));
    }
    if (lane == j) {
      my_e = be;
      my_v = bv;
    }
  }
  float my_w = 0.f;
  if (lane < k && my_e >= 0 && my_e < E)
    my_w = softmax ? expf(my_v - lmax) / denom : 1.0f / (1.0f + expf(-my_v));
  float wsum = 0.f;
#pragma unroll 1
  for (int j = 0; j < k; ++j) wsum += __shfl(my_w, j, kWave);     // in slot order
  const bool renorm = p.rp.renormalize != 0 && wsum > 0.f;
  if (lane < k) {
    const float w = renorm ? my_w / wsum : my_w;
    p.ids[t * k + lane] = my_e;
    p.w[t * k + lane] = w * p.rp.routed_scale;
  }
}

// One wave per token, 4 tokens per workgroup: adds the S split-K partials of
// the router GEMM in a fixed order, adds the bias and selects.
__global__ __launch_bounds__(256) void k_topk(TopkParams p) {
  __shared__ float s_score[4][256];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (t >= p.T) return;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    v[i] = -INFINITY;
    if (e < p.E) {
      // the S partials (S <= 16) loaded eight at a time, summed in split order
      float s = 0.f;
      for (int s0 = 0; s0 < p.S; s0 += 8) {
        float pv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          pv[u] = s0 + u < p.S ? p.part[((s0 + u) * p.T + t) * p.E + e] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < p.S) s += pv[u];
      }
      if (p.bias) s += p.bias[e];
      v[i] = s;
      if (p.logits) p.logits[t * p.E + e] = s;
    }
  }
  topk_token(p, t, v, s_score[wave]);
}

moe_status launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return MOE_OK;
  const int E = a.p.E;
  const int S = route_splits(a.T, a.H, E);
  GemmParams p{};
  GemmGroup& g = p.g[0];
  g.A = static_cast<const bf16_t*>(a.x);
  g.lda = a.H;
  g.B = a.w_router;
  g.ldb = a.H;
  g.bscale = nullptr;
  g.K = a.H / S;
  g.N = E;
  g.b_rows = E;
  g.n_tiles = (E + kBN - 1) / kBN;
  g.C = a.part;
  g.ldc = E;
  g.b_estride = static_cast<int64_t>(E) * a.H;
  p.offsets = nullptr;
  p.E_loc = 1;
  p.dense_rows = a.T;
  p.rows1 = 0;
  p.bias = nullptr;
  p.split_c = a.T * E;
  const dim3 grid(static_cast<unsigned>(gemm_grid(max_row_tiles(a.T, 1, 32, true) * g.n_tiles)), S);
  if (a.act == MOE_BF16) {
    // K stages 128 wide where the split's K allows: half the dependent load
    // round trips per tile, the same K order (the MFMA steps of a stage run
    // in sequence), so the same logits.  R1-shaped layer (K = 3584 per
    // split) 0.851 -> 0.845 ms in DBO; prefill (K = 1024) unchanged.
    if (g.K % 128 == 0)
      hipLaunchKernelGGL((k_gemm_nt<32, 1, 4, MODE_ROUTER, false, kBN, 2 * kBK>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((k_gemm_nt<32, 1, 4, MODE_ROUTER, false>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_gemm_nt_f32<MODE_ROUTER>), grid, dim3(256), 0, s, p);
  }
  DBOMOE_CHECK_LAUNCH();
  TopkParams tp{a.part, S, a.T, E, a.bias, a.forced, a.p, a.logits, a.ids, a.w};
  hipLaunchKernelGGL(k_topk, dim3(static_cast<unsigned>((a.T + 3) / 4)), dim3(256), 0, s, tp);
  DBOMOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace dbomoe

using namespace dbomoe;

extern "C" size_t moe_route_workspace_size(int64_t T, int32_t H, int32_t E) {
  if (T < 0 || H <= 0 || E <= 0) return 0;
  return route_ws_bytes(T, H, E);
}

extern "C" moe_status moe_route_topk(const void* x, moe_dtype act, int64_t T, int32_t H,
                                     const void* w_router, const float* logit_bias,
                                     const int32_t* forced_ids, const moe_route_params* params,
                                     float* logits_out, int32_t* topk_ids, float* topk_w,
                                     void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_route_params(params);
  if (st != MOE_OK) return st;
  if (T < 0 || H <= 0) return MOE_ERR_INVALID_ARG;
  if (act != MOE_F32 && act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (H % 128) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_w || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(topk_ids) || !aligned16(topk_w) ||
      (logit_bias && !aligned16(logit_bias)) || (forced_ids && !aligned16(forced_ids)) ||
      (logits_out && !aligned16(logits_out)) || !aligned256(ws))
    return MOE_ERR_MISALIGNED;
  if (ws_bytes < route_ws_bytes(T, H, params->E)) return MOE_ERR_WORKSPACE;
  RouteArgs a{x, act, T, H, w_router, logit_bias, forced_ids, *params, logits_out, topk_ids, topk_w,
              static_cast<float*>(ws)};
  return launch_route(a, as_stream(stream));
}
