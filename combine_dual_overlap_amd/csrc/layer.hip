// dbo_moe_layer: the MoE layer under Dual-Batch Overlap, issued by the
// two-stream schedule of dbo_schedule.h on the HIP backend below.
//
// Split ("[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM", Purpose;
// a request may straddle the split, "[Core/DBO][2/N] ... Prefill support",
// Purpose): microbatch A = rows [0, T0), B = rows [T0, T), T0 = ceil(T/2) unless
// given; below min_tokens_to_split, or when a half would be empty (the guard of
// "[Core/DBO][2/N]", commit log), the layer runs unsplit.
// Each microbatch owns one half of the workspace, so the two never share a
// buffer ("[Core/DBO][2/N]", commit log: same buffer used across ubatches), and
// the caller reserves the whole workspace up front ("DeepEP HT: full decode CUDA
// graphs via worst-token dispatch", file table: deterministic workspace
// reservation).  Buffers inside a half are sized for the worst case of T*k
// dispatched rows.
#include <cstring>

#include "common.h"
#include "dbo_schedule.h"

constexpr int kTimingRing = 128;   // timed calls remembered by a context

struct dbo_ctx {
  hipEvent_t ev[dbomoe::sched::kNumEvents] = {};
  hipEvent_t join = nullptr;
  // Timing events, created when timing is first enabled: [call slot][microbatch][7]
  // (FFN start / between the GEMMs / end, dispatch start / end, combine start / end)
  hipEvent_t (*tev)[2][7] = nullptr;
  bool (*timed)[2] = nullptr;
  bool timing = false;
  int64_t timed_calls = 0;
  int slot = 0;
  int64_t stats[6] = {0, 0, 0, 0, 0, 0};
};

namespace dbomoe {

namespace {

enum Buf { B_LOGITS, B_IDS, B_W, B_COUNTS, B_OFFSETS, B_TILE_OFF, B_PERM, B_INV, B_XPERM, B_YPERM,
           B_SHOUT, B_DISPWS, B_ROUTEWS, B_H, B_SHH, B_XSCALE, B_COUNT };

struct HalfLayout {
  size_t off[B_COUNT];
  size_t bytes;
};

// Route split-K slabs: S * T * E floats with S * ceil(T/32) < 512 whenever S > 1.
size_t route_ws_bound(int64_t T, int32_t E) {
  const int64_t rows = T > 16384 ? T : 16384;
  return align_up(static_cast<size_t>(rows) * E * 4, 256);
}

HalfLayout half_layout(const moe_layer_desc* d, int64_t T) {
  const int E = d->route.E, k = d->route.k;
  const int E_loc = d->expert_end - d->expert_begin;
  const size_t as = dtype_size(d->act);
  const int64_t cap = T * k;
  size_t sz[B_COUNT];
  sz[B_LOGITS] = static_cast<size_t>(T) * E * 4;
  sz[B_IDS] = static_cast<size_t>(cap) * 4;
  sz[B_W] = static_cast<size_t>(cap) * 4;
  sz[B_COUNTS] = static_cast<size_t>(E_loc) * 4;
  sz[B_OFFSETS] = static_cast<size_t>(E_loc + 1) * 4;
  sz[B_TILE_OFF] = static_cast<size_t>(E_loc + 1) * 4;
  sz[B_PERM] = static_cast<size_t>(cap) * 4;
  sz[B_INV] = static_cast<size_t>(cap) * 4;
  const bool f8 = d->fp8_act != 0;
  sz[B_XPERM] = static_cast<size_t>(cap) * d->H * (f8 ? 1 : as);
  sz[B_XSCALE] = f8 ? static_cast<size_t>(cap) * (d->H / 128) : 0;
  sz[B_YPERM] = static_cast<size_t>(cap) * d->H * as;
  sz[B_SHOUT] = d->shared_I > 0
                    ? static_cast<size_t>(dense_down_chunks(d->act, d->shared_I, d->I)) * T * d->H * as
                    : 0;
  sz[B_DISPWS] = dispatch_ws_bytes(T, k, E_loc);
  sz[B_ROUTEWS] = route_ws_bound(T, E);
  sz[B_H] = f8 ? ffn_fp8_ws_bytes(cap, d->I) : ffn_ws_bytes(cap, d->I, d->act);
  sz[B_SHH] = d->shared_I > 0 ? ffn_ws_bytes(T, d->shared_I, d->act) : 0;
  HalfLayout L;
  size_t o = 0;
  for (int i = 0; i < B_COUNT; ++i) {
    L.off[i] = o;
    o += align_up(sz[i], 256);
  }
  L.bytes = o;
  return L;
}

moe_status check_desc(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  moe_status st = check_route_params(&d->route);
  if (st != MOE_OK) return st;
  if (d->expert_begin < 0 || d->expert_end <= d->expert_begin || d->expert_end > d->route.E)
    return MOE_ERR_INVALID_ARG;
  const int E_loc = d->expert_end - d->expert_begin;
  st = check_ffn_shapes(d->act, d->wdt, d->H, d->I, E_loc, d->w13_scale, d->w2_scale);
  if (st != MOE_OK) return st;
  if (d->fp8_act != 0 && d->fp8_act != 1) return MOE_ERR_INVALID_ARG;
  if (d->fp8_act) {
    if (d->act != MOE_BF16 || d->wdt != MOE_FP8_E4M3FN) return MOE_ERR_UNSUPPORTED;
    st = check_ffn_fp8_shapes(d->H, d->I, E_loc, d->w13_scale, d->w2_scale);
    if (st != MOE_OK) return st;
  }
  if (!d->w_router || !d->w13 || !d->w2) return MOE_ERR_INVALID_ARG;
  if (!aligned16(d->w_router) || !aligned16(d->w13) || !aligned16(d->w2) ||
      (d->w13_scale && !aligned16(d->w13_scale)) || (d->w2_scale && !aligned16(d->w2_scale)))
    return MOE_ERR_MISALIGNED;
  if (d->shared_I < 0) return MOE_ERR_INVALID_ARG;
  if (d->shared_I > 0) {
    st = check_ffn_shapes(d->act, d->act, d->H, d->shared_I, 1, nullptr, nullptr);
    if (st != MOE_OK) return st;
    if (!d->shared_w13 || !d->shared_w2) return MOE_ERR_INVALID_ARG;
    if (!aligned16(d->shared_w13) || !aligned16(d->shared_w2)) return MOE_ERR_MISALIGNED;
    // the combine sums k routed rows and the shared down projection's slabs
    if (d->route.k + dense_down_chunks(d->act, d->shared_I, d->I) > 32) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// Launches the kernels of one stage of one microbatch on the HIP streams.
struct HipBackend {
  dbo_ctx* ctx;
  const moe_layer_desc* d;
  const dbo_opts* o;
  hipStream_t streams[2];
  char* ws;
  HalfLayout L;
  const char* x;
  char* out;
  const int32_t* forced;
  const float* bias;
  int64_t row0[2];
  int64_t rows[2];
  int n_mb;
  int schedule;   // the schedule run (after the split rule)

  template <class T>
  T* buf(int mb, Buf b) const {
    return reinterpret_cast<T*>(ws + static_cast<size_t>(mb) * L.bytes + L.off[b]);
  }

  int launch(int stream, int mb, int stage) {
    hipStream_t s = streams[stream];
    const size_t as = dtype_size(d->act);
    const int64_t T = rows[mb];
    const char* xm = x + row0[mb] * d->H * as;
    const int k = d->route.k;
    const int E_loc = d->expert_end - d->expert_begin;
    // The comm-stream stages that can run beside the other microbatch's FFN
    // launch take the kernels that fit beside the GEMM: the second
    // microbatch's dispatch, and the first one's combine unless the FFN event
    // it waits for is the late one (recorded after the second FFN is queued,
    // so nothing runs beside it).
    const bool dispatch_stage =
        stage == sched::kDispatch || stage == sched::kDispatchSend || stage == sched::kDispatchRecv;
    const bool beside_ffn = stream == sched::kComm && n_mb == 2 &&
                            ((dispatch_stage && mb == 1) ||
                             (stage == sched::kCombine && mb == 0 && schedule != DBO_SCHED_DBO_LATE_EVENT));
    moe_status st = MOE_OK;
    switch (stage) {
      case sched::kRoute: {
        RouteArgs a{xm, d->act, T, d->H, d->w_router, bias, forced ? forced + row0[mb] * k : nullptr,
                    d->route, buf<float>(mb, B_LOGITS), buf<int32_t>(mb, B_IDS), buf<float>(mb, B_W),
                    buf<float>(mb, B_ROUTEWS)};
        st = launch_route(a, s);
        break;
      }
      case sched::kDispatch:
      case sched::kDispatchSend:
      case sched::kDispatchRecv: {
        DispatchArgs a{xm, d->act, T, d->H, buf<int32_t>(mb, B_IDS), k, d->route.E, d->expert_begin,
                       d->expert_end, 0, buf<int32_t>(mb, B_COUNTS), buf<int32_t>(mb, B_OFFSETS),
                       nullptr, buf<int32_t>(mb, B_PERM), buf<int32_t>(mb, B_INV),
                       buf<void>(mb, B_XPERM), buf<void>(mb, B_DISPWS), o->comm_cu_budget,
                       d->fp8_act ? buf<uint8_t>(mb, B_XSCALE) : nullptr, beside_ffn};
        // timing: from the first dispatch kernel to the last (send start .. recv end)
        if (stage != sched::kDispatchRecv && ctx->timing &&
            hipEventRecord(ctx->tev[ctx->slot][mb][3], s) != hipSuccess)
          return MOE_ERR_HIP;
        st = stage == sched::kDispatch       ? launch_dispatch(a, s)
             : stage == sched::kDispatchSend ? launch_dispatch_send(a, s)
                                             : launch_dispatch_recv(a, s);
        if (st == MOE_OK && stage != sched::kDispatchSend && ctx->timing &&
            hipEventRecord(ctx->tev[ctx->slot][mb][4], s) != hipSuccess)
          return MOE_ERR_HIP;
        break;
      }
      case sched::kFfn: {
        // Routed experts on the dispatched rows plus the shared experts on the
        // microbatch's own rows, in the same two launches.
        const int64_t hint = (T * k + d->route.E - 1) / d->route.E;
        FfnArgs a{};
        a.x = buf<void>(mb, B_XPERM);
        a.xs = d->fp8_act ? buf<uint8_t>(mb, B_XSCALE) : nullptr;
        a.act = d->act;
        a.H = d->H;
        a.I = d->I;
        a.offsets = buf<int32_t>(mb, B_OFFSETS);
        a.E_loc = E_loc;
        a.cap_rows = T * k;
        a.rows_hint = hint;
        a.w13 = d->w13;
        a.w2 = d->w2;
        a.wdt = d->wdt;
        a.s13 = d->w13_scale;
        a.s2 = d->w2_scale;
        a.y = buf<void>(mb, B_YPERM);
        a.tile_m = o->ffn_tile_m;
        a.h = buf<void>(mb, B_H);
        if (d->shared_I > 0) {
          a.x1 = xm;
          a.rows1 = T;
          a.I1 = d->shared_I;
          a.w13_1 = d->shared_w13;
          a.w2_1 = d->shared_w2;
          a.y1 = buf<void>(mb, B_SHOUT);
          a.h1 = buf<void>(mb, B_SHH);
        }
        if (ctx->timing) {
          a.t0 = ctx->tev[ctx->slot][mb][0];
          a.t1 = ctx->tev[ctx->slot][mb][1];
          a.t2 = ctx->tev[ctx->slot][mb][2];
          ctx->timed[ctx->slot][mb] = true;
        }
        st = launch_ffn(a, s);
        break;
      }
      case sched::kCombine: {
        CombineArgs a{buf<void>(mb, B_YPERM), d->act, T, d->H, k, buf<int32_t>(mb, B_INV), buf<float>(mb, B_W),
                      d->shared_I > 0 ? buf<void>(mb, B_SHOUT) : nullptr, out + row0[mb] * d->H * as,
                      o->comm_cu_budget, d->shared_I > 0 ? dense_down_chunks(d->act, d->shared_I, d->I) : 0,
                      beside_ffn};
        if (ctx->timing && hipEventRecord(ctx->tev[ctx->slot][mb][5], s) != hipSuccess) return MOE_ERR_HIP;
        st = launch_combine(a, s);
        if (st == MOE_OK && ctx->timing && hipEventRecord(ctx->tev[ctx->slot][mb][6], s) != hipSuccess)
          return MOE_ERR_HIP;
        break;
      }
      default:
        st = MOE_ERR_INVALID_ARG;
    }
    return st;
  }
  int record(int stream, int ev) { return hipEventRecord(ctx->ev[ev], streams[stream]) == hipSuccess ? 0 : MOE_ERR_HIP; }
  int wait(int stream, int ev) {
    return hipStreamWaitEvent(streams[stream], ctx->ev[ev], 0) == hipSuccess ? 0 : MOE_ERR_HIP;
  }
  int join() {
    if (hipEventRecord(ctx->join, streams[sched::kComm]) != hipSuccess) return MOE_ERR_HIP;
    return hipStreamWaitEvent(streams[sched::kCompute], ctx->join, 0) == hipSuccess ? 0 : MOE_ERR_HIP;
  }
};

}  // namespace
}  // namespace dbomoe

using namespace dbomoe;

extern "C" const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid size, range, pointer or combination";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: dtype combination or shape multiple not supported";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED: pointer or row pitch not 16-byte (workspace 256-byte) aligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than the size query";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP runtime call or kernel launch failed";
  }
  return "unknown moe_status";
}

extern "C" moe_status dbo_ctx_create(dbo_ctx** ctx) {
  if (!ctx) return MOE_ERR_INVALID_ARG;
  dbo_ctx* c = new dbo_ctx();
  bool ok = true;
  // The schedule's events only order two streams of one device: no host wait
  // ever synchronises on them, so they skip the system-scope fence.
  const unsigned flags = hipEventDisableTiming | hipEventDisableSystemFence;
  for (int i = 0; i < sched::kNumEvents; ++i)
    ok = ok && hipEventCreateWithFlags(&c->ev[i], flags) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&c->join, flags) == hipSuccess;
  if (!ok) {
    dbo_ctx_destroy(c);
    return MOE_ERR_HIP;
  }
  *ctx = c;
  return MOE_OK;
}

extern "C" void dbo_ctx_destroy(dbo_ctx* c) {
  if (!c) return;
  for (int i = 0; i < sched::kNumEvents; ++i)
    if (c->ev[i]) (void)hipEventDestroy(c->ev[i]);
  if (c->join) (void)hipEventDestroy(c->join);
  if (c->tev) {
    for (int r = 0; r < kTimingRing; ++r)
      for (int m = 0; m < 2; ++m)
        for (int j = 0; j < 7; ++j)
          if (c->tev[r][m][j]) (void)hipEventDestroy(c->tev[r][m][j]);
    delete[] c->tev;
    delete[] c->timed;
  }
  delete c;
}

extern "C" moe_status dbo_ctx_set_timing(dbo_ctx* c, int32_t enable) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (enable && !c->tev) {
    c->tev = new hipEvent_t[kTimingRing][2][7]();
    c->timed = new bool[kTimingRing][2]();
    for (int r = 0; r < kTimingRing; ++r)
      for (int m = 0; m < 2; ++m)
        for (int j = 0; j < 7; ++j)
          if (hipEventCreate(&c->tev[r][m][j]) != hipSuccess) return MOE_ERR_HIP;
  }
  c->timing = enable != 0;
  return MOE_OK;
}

extern "C" moe_status dbo_ctx_ffn_times(dbo_ctx* c, int32_t back, float* ms4) {
  if (!c || !ms4 || back < 0) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i) ms4[i] = 0.f;
  if (!c->tev || back >= kTimingRing || back >= c->timed_calls) return MOE_OK;
  const int r = static_cast<int>(((c->timed_calls - 1 - back) % kTimingRing + kTimingRing) % kTimingRing);
  for (int m = 0; m < 2; ++m) {
    if (!c->timed[r][m]) continue;
    if (hipEventSynchronize(c->tev[r][m][2]) != hipSuccess) return MOE_ERR_HIP;
    if (hipEventElapsedTime(&ms4[2 * m], c->tev[r][m][0], c->tev[r][m][1]) != hipSuccess) return MOE_ERR_HIP;
    if (hipEventElapsedTime(&ms4[2 * m + 1], c->tev[r][m][1], c->tev[r][m][2]) != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

extern "C" moe_status dbo_ctx_comm_times(dbo_ctx* c, int32_t back, float* ms4) {
  if (!c || !ms4 || back < 0) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i) ms4[i] = 0.f;
  if (!c->tev || back >= kTimingRing || back >= c->timed_calls) return MOE_OK;
  const int r = static_cast<int>(((c->timed_calls - 1 - back) % kTimingRing + kTimingRing) % kTimingRing);
  for (int m = 0; m < 2; ++m) {
    if (!c->timed[r][m]) continue;
    if (hipEventSynchronize(c->tev[r][m][6]) != hipSuccess) return MOE_ERR_HIP;
    if (hipEventElapsedTime(&ms4[m], c->tev[r][m][3], c->tev[r][m][4]) != hipSuccess) return MOE_ERR_HIP;
    if (hipEventElapsedTime(&ms4[2 + m], c->tev[r][m][5], c->tev[r][m][6]) != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

extern "C" moe_status dbo_ctx_last_stats(dbo_ctx* c, int64_t* stats6) {
  if (!c || !stats6) return MOE_ERR_INVALID_ARG;
  std::memcpy(stats6, c->stats, sizeof(c->stats));
  return MOE_OK;
}

extern "C" size_t moe_layer_workspace_size(const moe_layer_desc* d, int64_t T_max) {
  if (check_desc(d) != MOE_OK || T_max < 0) return 0;
  return 2 * half_layout(d, T_max).bytes;
}

extern "C" moe_status moe_layer_workspace_layout(const moe_layer_desc* d, int64_t T_max, int32_t mb, int64_t* off12) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (T_max < 0 || mb < 0 || mb > 1 || !off12) return MOE_ERR_INVALID_ARG;
  const HalfLayout L = half_layout(d, T_max);
  const Buf order[12] = {B_LOGITS, B_IDS, B_W, B_COUNTS, B_OFFSETS, B_TILE_OFF, B_PERM, B_INV, B_XPERM, B_YPERM,
                         B_SHOUT, B_DISPWS};
  for (int i = 0; i < 12; ++i) off12[i] = static_cast<int64_t>(mb * L.bytes + L.off[order[i]]);
  return MOE_OK;
}

extern "C" moe_status dbo_moe_layer(dbo_ctx* ctx, const moe_layer_desc* d, const void* x, int64_t T,
                                    const int32_t* forced_ids, const float* logit_bias, void* out,
                                    const dbo_opts* o, void* ws, size_t ws_bytes,
                                    void* compute_stream, void* comm_stream) {
  if (!ctx || !o) return MOE_ERR_INVALID_ARG;
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (o->schedule < DBO_SCHED_UNSPLIT || o->schedule > DBO_SCHED_DBO_RECV_HOOK) return MOE_ERR_INVALID_ARG;
  if (o->min_tokens_to_split < 0 || o->comm_cu_budget < 0) return MOE_ERR_INVALID_ARG;
  if (o->ffn_tile_m != 0 && o->ffn_tile_m != 32 && o->ffn_tile_m != 64 && o->ffn_tile_m != 128)
    return MOE_ERR_INVALID_ARG;
  if (d->fp8_act && o->ffn_tile_m != 0 && o->ffn_tile_m != 64 && o->ffn_tile_m != 128) return MOE_ERR_UNSUPPORTED;
  if (o->split_at != -1 && (o->split_at < 1 || o->split_at >= T)) return MOE_ERR_INVALID_ARG;
  for (auto& v : ctx->stats) v = 0;
  if (T == 0) return MOE_OK;
  if (!x || !out || !ws) return MOE_ERR_INVALID_ARG;
  if (x == out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out) || !aligned256(ws) || (forced_ids && !aligned16(forced_ids)) ||
      (logit_bias && !aligned16(logit_bias)))
    return MOE_ERR_MISALIGNED;
  if (T * d->route.k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  const HalfLayout L = half_layout(d, T);
  if (ws_bytes < 2 * L.bytes) return MOE_ERR_WORKSPACE;

  // Split rule.
  int schedule = o->schedule;
  const int min_split = o->min_tokens_to_split < 2 ? 2 : o->min_tokens_to_split;
  int64_t T0 = o->split_at > 0 ? o->split_at : (T + 1) / 2;
  if (schedule != DBO_SCHED_UNSPLIT && (T < min_split || T0 <= 0 || T0 >= T)) schedule = DBO_SCHED_UNSPLIT;

  HipBackend be;
  be.ctx = ctx;
  be.d = d;
  be.o = o;
  be.streams[sched::kCompute] = as_stream(compute_stream);
  be.streams[sched::kComm] = as_stream(comm_stream);
  be.ws = static_cast<char*>(ws);
  be.L = L;
  be.x = static_cast<const char*>(x);
  be.out = static_cast<char*>(out);
  be.forced = forced_ids;
  be.bias = logit_bias;
  be.schedule = schedule;
  if (schedule == DBO_SCHED_UNSPLIT) {
    be.row0[0] = 0;
    be.rows[0] = T;
    be.n_mb = 1;
  } else {
    be.row0[0] = 0;
    be.rows[0] = T0;
    be.row0[1] = T0;
    be.rows[1] = T - T0;
    be.n_mb = 2;
  }
  if (ctx->timing) {
    ctx->slot = static_cast<int>(ctx->timed_calls % kTimingRing);
    ctx->timed[ctx->slot][0] = ctx->timed[ctx->slot][1] = false;
    ctx->timed_calls++;
  }
  const sched::Plan plan = sched::build_plan(schedule);
  sched::RunStats rs;
  const int r = sched::run_plan(plan, be, &rs);
  ctx->stats[0] = schedule;
  ctx->stats[1] = schedule == DBO_SCHED_UNSPLIT ? T : T0;
  ctx->stats[2] = rs.yields[0];
  ctx->stats[3] = rs.yields[1];
  ctx->stats[4] = rs.launches;
  ctx->stats[5] = rs.records;
  return static_cast<moe_status>(r);
}
