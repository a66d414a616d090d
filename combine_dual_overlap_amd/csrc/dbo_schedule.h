// Two-stream Dual-Batch-Overlap schedule: plain C++, no HIP, so the same code
// runs under the HIP backend of the library and under a recording backend in
// the host-side schedule tests.
//
// What it follows ("[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM",
// Purpose): the batch is split into two microbatches; one stream carries
// compute, the other dispatch/combine; a microbatch hands over ("yields") at
// each switch between the two, only one microbatch issues at a time, and both
// issue the same number of yields.  Cross-stream order comes from per-
// microbatch events.  "[Perf] Fix DBO overlap: capture DeepEP event before
// yield", Purpose: the event a microbatch's dispatch/combine waits on must be
// recorded on the compute stream BEFORE the yield, so it covers only that
// microbatch's own compute tail and not work the other microbatch enqueued
// after it.  The late-event schedule keeps the old behaviour as a diagnostic.
//
// One host thread issues everything in the order two cooperating microbatch
// threads would: A.p0, B.p0, A.p1, B.p1, ... with the phases
//   p0 compute: route, record route-event                       yield
//   p1 comm:    wait route-event, dispatch, record dispatch-event   yield
//   p2 compute: wait dispatch-event, expert FFN (routed + shared), record ffn-event   yield
//   p3 comm:    wait ffn-event, combine, record combine-event
// and finally the compute stream waits both combine events (comm work joined
// back before anything that follows the layer on the compute stream).
//
// Receive-hook variant (the low-latency dispatch structure of "[Core/DBO][2/N]
// Dual-Batch Overlap add DeepEP High Throughput support and Prefill support",
// review of modular_kernel.py: the dispatch returns a receive hook, which
// under DBO is registered with the microbatch and run after one more yield):
// p1 becomes two phases on the comm stream,
//   p1  comm: wait route-event, dispatch send (count, scan, rank), register hook   yield
//   p1r comm: run the hook: dispatch receive (row gather), record recv-event       yield
// and p2 waits for the recv-event.  Each microbatch yields four times, and the
// comm stream carries A.send, B.send, A.recv, B.recv.
#pragma once

#include <cstdint>
#include <vector>

namespace dbomoe {
namespace sched {

enum StreamId { kCompute = 0, kComm = 1 };
// kDispatch is the whole dispatch; kDispatchSend + kDispatchRecv are its two
// phases in the receive-hook schedule.
enum Stage { kRoute = 0, kDispatch = 1, kFfn = 2, kCombine = 3, kDispatchSend = 4, kDispatchRecv = 5,
             kNumStages = 6 };
enum Schedule { kUnsplit = 0, kSerial = 1, kDbo = 2, kDboLate = 3, kDboRecvHook = 4 };

struct Op {
  enum Kind { LAUNCH = 0, RECORD = 1, WAIT = 2, YIELD = 3 } kind;
  int stream;  // LAUNCH / RECORD / WAIT
  int mb;      // microbatch of the launch, of the yield, or owning the event
  int stage;   // launched stage, or the stage whose event is recorded / awaited
};

inline int event_id(int mb, int stage) { return mb * kNumStages + stage; }
constexpr int kNumEvents = 2 * kNumStages;

struct Plan {
  std::vector<Op> ops;
  int n_mb = 0;
  int yields[2] = {0, 0};
};

inline Op launch(int s, int mb, int st) { return Op{Op::LAUNCH, s, mb, st}; }
inline Op record(int s, int mb, int st) { return Op{Op::RECORD, s, mb, st}; }
inline Op wait(int s, int mb, int st) { return Op{Op::WAIT, s, mb, st}; }
inline Op yield(int mb) { return Op{Op::YIELD, -1, mb, -1}; }

// One microbatch, everything in order on the compute stream.
inline void append_sequential(Plan& p, int mb) {
  p.ops.push_back(launch(kCompute, mb, kRoute));
  p.ops.push_back(launch(kCompute, mb, kDispatch));
  p.ops.push_back(launch(kCompute, mb, kFfn));
  p.ops.push_back(launch(kCompute, mb, kCombine));
}

// Phase `ph` of microbatch `mb` of the two-stream schedule.  `late`: the
// compute-stream events that the comm stream waits on are recorded when the
// microbatch resumes after its yield instead of before it.  `hook`: the
// receive-hook variant, whose phases are 0, 1, 4 (the hook), 2, 3.
inline void append_phase(Plan& p, int mb, int ph, bool late, bool hook) {
  const int ready = hook ? kDispatchRecv : kDispatch;   // the event the FFN waits for
  switch (ph) {
    case 0:
      p.ops.push_back(launch(kCompute, mb, kRoute));
      if (!late) p.ops.push_back(record(kCompute, mb, kRoute));
      break;
    case 1:
      if (late) p.ops.push_back(record(kCompute, mb, kRoute));
      p.ops.push_back(wait(kComm, mb, kRoute));
      if (hook) {
        p.ops.push_back(launch(kComm, mb, kDispatchSend));   // the receive hook is registered here
      } else {
        p.ops.push_back(launch(kComm, mb, kDispatch));
        p.ops.push_back(record(kComm, mb, kDispatch));
      }
      break;
    case 4:   // the microbatch resumes and runs its receive hook
      p.ops.push_back(launch(kComm, mb, kDispatchRecv));
      p.ops.push_back(record(kComm, mb, kDispatchRecv));
      break;
    case 2:
      p.ops.push_back(wait(kCompute, mb, ready));
      p.ops.push_back(launch(kCompute, mb, kFfn));
      if (!late) p.ops.push_back(record(kCompute, mb, kFfn));
      break;
    case 3:
      if (late) p.ops.push_back(record(kCompute, mb, kFfn));
      p.ops.push_back(wait(kComm, mb, kFfn));
      p.ops.push_back(launch(kComm, mb, kCombine));
      p.ops.push_back(record(kComm, mb, kCombine));
      break;
  }
  if (ph != 3) {
    p.ops.push_back(yield(mb));
    p.yields[mb]++;
  }
}

inline Plan build_plan(int schedule) {
  Plan p;
  if (schedule == kUnsplit) {
    p.n_mb = 1;
    append_sequential(p, 0);
    return p;
  }
  p.n_mb = 2;
  if (schedule == kSerial) {
    append_sequential(p, 0);
    append_sequential(p, 1);
    return p;
  }
  const bool late = schedule == kDboLate;
  const bool hook = schedule == kDboRecvHook;
  const int order_plain[4] = {0, 1, 2, 3};
  const int order_hook[5] = {0, 1, 4, 2, 3};
  const int* order = hook ? order_hook : order_plain;
  const int n_ph = hook ? 5 : 4;
  for (int i = 0; i < n_ph; ++i)
    for (int mb = 0; mb < 2; ++mb) append_phase(p, mb, order[i], late, hook);
  p.ops.push_back(wait(kCompute, 0, kCombine));
  p.ops.push_back(wait(kCompute, 1, kCombine));
  return p;
}

struct RunStats {
  int yields[2] = {0, 0};
  int launches = 0;
  int records = 0;
  int waits = 0;
  bool joined = false;
};

// Issues a plan on a backend with
//   int launch(int stream, int mb, int stage);
//   int record(int stream, int event);
//   int wait(int stream, int event);
//   int join();          // order everything issued on comm before later compute work
// each returning 0 on success.  Stops at the first failure; if anything was
// issued on the comm stream it is then joined into the compute stream, so no
// issued wait can target an unrecorded event and no comm work is left
// unordered with what the caller does next.  Returns the first failure (or -1
// for an inconsistent plan), 0 on success.
template <class Backend>
int run_plan(const Plan& plan, Backend& be, RunStats* st) {
  if (plan.n_mb == 2 && plan.yields[0] != plan.yields[1]) return -1;   // equal-yield invariant
  bool recorded[kNumEvents] = {};
  bool comm_used = false;
  int status = 0;
  for (const Op& op : plan.ops) {
    switch (op.kind) {
      case Op::LAUNCH:
        status = be.launch(op.stream, op.mb, op.stage);
        if (op.stream == kComm) comm_used = true;
        if (status == 0) st->launches++;
        break;
      case Op::RECORD:
        status = be.record(op.stream, event_id(op.mb, op.stage));
        if (op.stream == kComm) comm_used = true;
        if (status == 0) {
          recorded[event_id(op.mb, op.stage)] = true;
          st->records++;
        }
        break;
      case Op::WAIT:
        if (!recorded[event_id(op.mb, op.stage)]) {
          status = -1;
        } else {
          status = be.wait(op.stream, event_id(op.mb, op.stage));
          if (status == 0) st->waits++;
        }
        break;
      case Op::YIELD:
        st->yields[op.mb]++;
        break;
    }
    if (status != 0) break;
  }
  if (status != 0 && comm_used) {
    be.join();
    st->joined = true;
  }
  return status;
}

}  // namespace sched
}  // namespace dbomoe
