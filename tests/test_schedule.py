"""Host-side checks of the two-stream DBO schedule (combine_dual_overlap_amd/
csrc/dbo_schedule.h), run through a recording backend built with g++: no GPU.

From the operation log the test rebuilds the happens-before graph (stream
order + event record -> wait edges) and checks:
  1. both microbatches yield equally often, 3 times each under DBO
     ("[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM", Purpose);
  2. every wait targets an event recorded earlier in issue order;
  3. each microbatch's dispatch/combine depends on its own compute only: no
     path from B's route to A's dispatch, or from B's FFN to A's combine, under
     DBO; the late-event diagnostic has both paths ("[Perf] Fix DBO overlap:
     capture DeepEP event before yield", Purpose);
  4. no two launches the graph leaves unordered touch a common buffer with a
     write (a host-level race detector; a planted shared-buffer layout fails);
  5. an injected failure at any operation stops issuing, returns an error,
     leaves no wait on an unrecorded event and joins issued comm work back;
  6. both combines are ordered before the end of the compute stream.
The receive-hook schedule (dispatch in a send phase and a receive hook run
after one more yield, "[Core/DBO][2/N] Dual-Batch Overlap add DeepEP High
Throughput support and Prefill support", review of modular_kernel.py) is
checked the same way, with four yields per microbatch.
"""
import itertools
import os
import subprocess

import pytest

from conftest import ROOT

SCHED = {"unsplit": 0, "serial": 1, "dbo": 2, "late": 3, "hook": 4}
ROUTE, DISPATCH, FFN, COMBINE, SEND, RECV = range(6)
COMPUTE, COMM = 0, 1
NAMES = ["route", "dispatch", "ffn", "combine", "dispatch_send", "dispatch_recv"]


def stages_of(schedule):
    return [ROUTE, SEND, RECV, FFN, COMBINE] if schedule == "hook" else [ROUTE, DISPATCH, FFN, COMBINE]


@pytest.fixture(scope="module")
def sched_bin(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("sched") / "sched_log")
    src = os.path.join(ROOT, "tests", "sched_log.cpp")
    inc = os.path.join(ROOT, "combine_dual_overlap_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", f"-I{inc}", src, "-o", out], check=True)
    return out


def run_log(binary, schedule, fail_at=-1):
    r = subprocess.run([binary, str(SCHED[schedule]), str(fail_at)], capture_output=True, text=True, check=True)
    ops = []
    status = yields = None
    for line in r.stdout.splitlines():
        f = line.split()
        if f[0] == "STATUS":
            status = int(f[1])
        elif f[0] == "YIELDS":
            yields = (int(f[1]), int(f[2]))
        elif f[0] == "JOIN":
            ops.append(("JOIN",))
        else:
            ops.append((f[0],) + tuple(int(v) for v in f[1:]))
    return ops, status, yields


class Graph:
    """Happens-before graph of an op log.  Nodes are op indices plus 'END'
    (the point after the last op issued on the compute stream)."""

    def __init__(self, ops):
        self.ops = ops
        self.succ = {i: set() for i in range(len(ops))}
        self.succ["END"] = set()
        last = {COMPUTE: None, COMM: None}
        last_record = {}
        self.launch = {}
        self.wait_ok = True
        for i, op in enumerate(ops):
            kind = op[0]
            if kind == "JOIN":            # record on comm + wait on compute
                if last[COMM] is not None:
                    self.succ[last[COMM]].add(i)
                if last[COMPUTE] is not None:
                    self.succ[last[COMPUTE]].add(i)
                last[COMPUTE] = i
                continue
            s = op[1]
            if last[s] is not None:
                self.succ[last[s]].add(i)
            last[s] = i
            if kind == "LAUNCH":
                self.launch[(op[2], op[3])] = i
            elif kind == "RECORD":
                last_record[op[2]] = i
            elif kind == "WAIT":
                if op[2] not in last_record:
                    self.wait_ok = False
                else:
                    self.succ[last_record[op[2]]].add(i)
        if last[COMPUTE] is not None:
            self.succ[last[COMPUTE]].add("END")
        self._reach = {}

    def reach(self, a):
        if a not in self._reach:
            seen, stack = set(), [a]
            while stack:
                n = stack.pop()
                for m in self.succ[n]:
                    if m not in seen:
                        seen.add(m)
                        stack.append(m)
            self._reach[a] = seen
        return self._reach[a]

    def before(self, a, b):
        return b in self.reach(a)

    def node(self, mb, stage):
        return self.launch[(mb, stage)]


def accesses(mb, stage, half):
    """Buffers one stage's kernels read and write (half = workspace half).
    The FFN stage also runs the shared experts on the microbatch's rows."""
    h = f"ws{half}"
    table = {
        ROUTE: ({f"x{mb}", "w_router"}, {f"{h}.logits", f"{h}.ids", f"{h}.w", f"{h}.route_ws"}),
        DISPATCH: ({f"x{mb}", f"{h}.ids"}, {f"{h}.counts", f"{h}.offsets", f"{h}.perm", f"{h}.inv",
                                           f"{h}.x_perm", f"{h}.disp_ws"}),
        SEND: ({f"{h}.ids"}, {f"{h}.counts", f"{h}.offsets", f"{h}.perm", f"{h}.inv", f"{h}.disp_ws"}),
        RECV: ({f"x{mb}", f"{h}.inv"}, {f"{h}.x_perm"}),
        FFN: ({f"{h}.x_perm", f"{h}.offsets", "w13", "w2", f"x{mb}", "w_shared"},
              {f"{h}.h", f"{h}.y", f"{h}.shared_h", f"{h}.shared_out"}),
        COMBINE: ({f"{h}.y", f"{h}.inv", f"{h}.w", f"{h}.shared_out"}, {f"out{mb}"}),
    }
    return table[stage]


def races(g, halves=(0, 1)):
    found = []
    items = [(mb, st, i) for (mb, st), i in g.launch.items()]
    for (m1, s1, i1), (m2, s2, i2) in itertools.combinations(items, 2):
        if g.before(i1, i2) or g.before(i2, i1):
            continue
        r1, w1 = accesses(m1, s1, halves[m1])
        r2, w2 = accesses(m2, s2, halves[m2])
        clash = (w1 & (r2 | w2)) | (w2 & r1)
        if clash:
            found.append((m1, NAMES[s1], m2, NAMES[s2], sorted(clash)))
    return found


@pytest.mark.parametrize("schedule", ["dbo", "late", "hook", "serial", "unsplit"])
def test_schedule_invariants(sched_bin, schedule):
    ops, status, yields = run_log(sched_bin, schedule)
    assert status == 0
    g = Graph(ops)
    assert g.wait_ok
    n_mb = 1 if schedule == "unsplit" else 2
    stages = stages_of(schedule)
    assert sorted(g.launch) == sorted((mb, st) for mb in range(n_mb) for st in stages)
    if schedule in ("dbo", "late"):
        assert yields == (3, 3)
    if schedule == "hook":
        assert yields == (4, 4)
    # each microbatch's own chain is ordered, and the layer ends after both combines
    for mb in range(n_mb):
        chain = [g.node(mb, st) for st in stages]
        for a, b in zip(chain, chain[1:]):
            assert g.before(a, b), (schedule, mb)
        assert g.before(g.node(mb, COMBINE), "END")
    assert races(g) == []


def test_event_before_yield_removes_cross_microbatch_waits(sched_bin):
    g = Graph(run_log(sched_bin, "dbo")[0])
    A, B = 0, 1
    # A's comm waits only on A's compute tail
    assert not g.before(g.node(B, ROUTE), g.node(A, DISPATCH))
    assert not g.before(g.node(B, FFN), g.node(A, COMBINE))
    # so the overlaps DBO is for are allowed
    assert not g.before(g.node(A, DISPATCH), g.node(B, ROUTE))
    assert not g.before(g.node(A, COMBINE), g.node(B, FFN))
    assert not g.before(g.node(B, DISPATCH), g.node(A, FFN)) and not g.before(g.node(A, FFN), g.node(B, DISPATCH))


def test_recv_hook_schedule_orders_and_overlaps(sched_bin):
    ops, _, _ = run_log(sched_bin, "hook")
    g = Graph(ops)
    A, B = 0, 1
    # the comm stream carries A.send, B.send, A.recv, B.recv, then the combines
    comm = [(o[2], o[3]) for o in ops if o[0] == "LAUNCH" and o[1] == COMM]
    assert comm == [(A, SEND), (B, SEND), (A, RECV), (B, RECV), (A, COMBINE), (B, COMBINE)]
    # each microbatch's FFN waits for its own receive, not only its send
    for mb in (A, B):
        assert g.before(g.node(mb, RECV), g.node(mb, FFN))
    # events before yields: A's send and combine do not wait for B's compute
    # (A's receive runs behind B's send on the comm stream, by stream order)
    assert not g.before(g.node(B, ROUTE), g.node(A, SEND))
    assert g.before(g.node(B, SEND), g.node(A, RECV))
    assert not g.before(g.node(B, FFN), g.node(A, COMBINE))
    # and the overlaps DBO is for remain possible
    assert not g.before(g.node(A, RECV), g.node(B, ROUTE))
    assert not g.before(g.node(B, RECV), g.node(A, FFN)) and not g.before(g.node(A, FFN), g.node(B, RECV))


def test_late_event_reproduces_over_serialisation(sched_bin):
    g = Graph(run_log(sched_bin, "late")[0])
    A, B = 0, 1
    assert g.before(g.node(B, ROUTE), g.node(A, DISPATCH))
    assert g.before(g.node(B, FFN), g.node(A, COMBINE))


def test_race_detector_catches_shared_workspace(sched_bin):
    g = Graph(run_log(sched_bin, "dbo")[0])
    found = races(g, halves=(0, 0))         # both microbatches on one workspace half
    assert found, "a shared workspace must show up as a race"
    assert any("ws0.ids" in c[4] or "ws0.w" in c[4] for c in found)


@pytest.mark.parametrize("schedule", ["dbo", "late", "hook", "serial"])
def test_failure_injection(sched_bin, schedule):
    full, _, _ = run_log(sched_bin, schedule)
    n_issued = sum(1 for o in full if o[0] in ("LAUNCH", "RECORD", "WAIT"))
    for fail_at in range(n_issued):
        ops, status, _ = run_log(sched_bin, schedule, fail_at)
        assert status == -5
        issued = [o for o in ops if o[0] in ("LAUNCH", "RECORD", "WAIT")]
        assert len(issued) == fail_at                     # nothing after the failure
        g = Graph(ops)
        assert g.wait_ok                                  # no wait on an unrecorded event
        comm_used = any(o[0] != "JOIN" and o[1] == COMM for o in issued)
        assert (("JOIN",) in ops) == comm_used
        # everything issued on the comm stream is ordered before the end of compute
        for i, o in enumerate(ops):
            if o[0] == "LAUNCH" and o[1] == COMM:
                assert g.before(i, "END")
