"""Throughput of the DBO expert-parallel MoE layer on one MI355X.

One step = one dbo_moe_layer call over one batch of synthetic input (routing,
dispatch, grouped SwiGLU FFN and combine of both microbatches, both streams
joined).  Default workload: the Qwen3-30B-A3B-shaped prefill layer (T=8192
tokens split 4096/4096, H=2048, 128 experts top-8 with uniform-random expert
ids, I=768, fp8 e4m3 expert weights with 128x128 block scales, bf16
activations), the stand-in for the 8192-token prefill benchmark of "[Perf]
Fix DBO overlap: capture DeepEP event before yield" (Test Plan / Test Result).

Prints one JSON line: `value` is the DBO step captured once in a HIP graph and
replayed K times (after W warm-up replays, bracketed by device syncs).  Before
it, the schedules DBO, SERIAL, DBO_LATE_EVENT (the event recorded after the
yield, the over-serialisation the page fixes) and UNSPLIT are timed as
interleaved repeated trials, graph-replayed and eager, with median and p10/p90
per schedule and per-round paired ratios (the trials also bring the chip to
its clocks under load before the headline's timed replays); the roofline of the dominant kernel
(the gate/up expert GEMM) against the per-expert roof; the dispatch and
combine HBM fractions; the CPU oracle on a bounded sample; and the
DeepSeek-V2-Lite-shaped decode layer as a secondary record.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
F8_DMA_MAX_K = 4096  # longest K the fp8 x fp8 GEMM stages by LDS DMA (kF8DmaMaxK)
KERNEL_SOURCES = ["combine_dual_overlap_amd/csrc/gemm_mfma.h", "combine_dual_overlap_amd/csrc/gemm_fp8.h",
                  "combine_dual_overlap_amd/csrc/gemm_fp8w.h", "combine_dual_overlap_amd/csrc/fp8_act.h",
                  "combine_dual_overlap_amd/csrc/ffn.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per gate/up launch from the committed rocprofv3 --pmc summary,
    or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"ffn_gate_up_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def gateup_work(cfg, counts_per_mb, rows_per_mb, fp8_act=False):
    """Algorithmic bytes and flops of one gate/up GEMM step per microbatch:
    weights of every routed expert that received rows and of the shared
    experts (each read once), the dispatched rows and the microbatch's rows for
    the shared experts (read once), the SwiGLU outputs h (written once).  With
    fp8 activations the routed rows and h are one byte per element plus one
    scale byte per 128."""
    w_s = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.wdt]
    a_s = 4 if cfg.act == "f32" else 2
    r_s = 1 + 1 / 128 if fp8_act else a_s
    I_sh = cfg.n_shared * cfg.shared_I
    out = []
    for counts, T_mb in zip(counts_per_mb, rows_per_mb):
        hit = int((counts > 0).sum())
        M = int(counts.sum())
        wbytes = hit * 2 * cfg.I * cfg.H * w_s
        if cfg.wdt == "fp8":
            wbytes += hit * (2 * cfg.I // 128) * (cfg.H // 128) * 4
        nbytes = wbytes + M * cfg.H * r_s + M * cfg.I * r_s
        flops = 2.0 * M * cfg.H * 2 * cfg.I
        if I_sh:
            nbytes += 2 * I_sh * cfg.H * a_s + T_mb * cfg.H * a_s + T_mb * I_sh * a_s
            flops += 2.0 * T_mb * cfg.H * 2 * I_sh
        out.append((nbytes, flops))
    return out


def ffn_expert_roof(cfg, counts, T_mb, gemm, fp8_act=False, bf16_peak=True):
    """The per-expert roof of one grouped GEMM launch: the sum over experts
    with rows of max(flops_e / P_MFMA, bytes_e / B_HBM) (and the shared
    experts as one dense expert), where bytes_e are the expert's weights (and
    block scales) read once plus its rows read and its outputs written once.
    gemm: "gate_up" or "down".  Returns (roof seconds, flops, bytes, seconds
    of the experts the MFMA bounds, seconds of those HBM bounds)."""
    w_s = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.wdt]
    a_s = 4 if cfg.act == "f32" else 2
    r_s = 1 + 1 / 128 if fp8_act else a_s
    P = (MFMA_PEAK_TFLOPS["f32" if cfg.act == "f32" else "fp8" if fp8_act else "bf16"]) * 1e12
    B = HBM_PEAK_GBS * 1e9
    H, I = cfg.H, cfg.I
    experts = [(int(n), cfg.wdt, r_s, I) for n in counts if n > 0]
    I_sh = cfg.n_shared * cfg.shared_I
    if I_sh:
        experts.append((T_mb, cfg.act, a_s, I_sh))
    t_mfma = t_hbm = fl_tot = by_tot = 0.0
    for n, wdt, rs, Ie in experts:
        ws = {"f32": 4, "bf16": 2, "fp8": 1}[wdt]
        if gemm == "gate_up":
            flops = 4.0 * n * H * Ie
            nbytes = 2 * Ie * H * ws + n * H * rs + n * Ie * rs
            if wdt == "fp8":
                nbytes += (2 * Ie // 128) * (H // 128) * 4
        else:
            flops = 2.0 * n * H * Ie
            out_s = a_s
            nbytes = H * Ie * ws + n * Ie * rs + n * H * out_s
            if wdt == "fp8":
                nbytes += (H // 128) * (Ie // 128) * 4
        tm, tb = flops / P, nbytes / B
        if tm >= tb:
            t_mfma += tm
        else:
            t_hbm += tb
        fl_tot += flops
        by_tot += nbytes
    return t_mfma + t_hbm, fl_tot, by_tot, t_mfma, t_hbm


def shared_slabs(cfg) -> int:
    """Slabs the shared experts' down projection writes (the library cuts it
    into K chunks of at most about I, each a multiple of 64)."""
    I1 = cfg.n_shared * cfg.shared_I
    if not I1 or cfg.act == "f32":
        return 1 if I1 else 0
    for d in range(-(-I1 // cfg.I), 1, -1):
        if I1 % (d * 64) == 0:
            return d
    return 1


def comm_work(cfg, L, halves, comm_ms, fp8_act=False):
    """Achieved HBM bandwidth of the dispatch step (count, scan, rank, gather)
    and of the combine, from their algorithmic bytes per microbatch: dispatch
    reads every token row with a local expert once and writes its dispatched
    rows (plus ids, perm and inv); combine reads the dispatched rows, the
    shared slabs, ids and weights, and writes every token row."""
    import torch
    s = 4 if cfg.act == "f32" else 2
    s_out = 1 + 1 / 128 if fp8_act else s         # dispatched row: codes + scale bytes
    d_bytes, c_bytes = [], []
    for mb, (a, b) in enumerate(halves):
        n = b - a
        inv = L.view(mb, "inv", torch.int32, (n * cfg.k,), T=cfg.T).cpu().numpy().reshape(n, cfg.k)
        M = int((inv >= 0).sum())
        t_hit = int((inv >= 0).any(axis=1).sum())
        d_bytes.append(t_hit * cfg.H * s + M * cfg.H * s_out + 4 * n * cfg.k + 4 * M + 4 * n * cfg.k)
        c_bytes.append(M * cfg.H * s + 8 * n * cfg.k + n * cfg.H * s + shared_slabs(cfg) * n * cfg.H * s)
    out = {"schedule": "serial"}
    for name, cols, byts in (("dispatch", [0, 1], d_bytes), ("combine", [2, 3], c_bytes)):
        ms = comm_ms[:, cols[:len(halves)]]
        avg_s = float(ms[ms > 0].mean()) / 1e3
        gbs = float(np.mean(byts)) / avg_s / 1e9
        out[name] = {"avg_us": round(avg_s * 1e6, 2), "algorithmic_bytes": int(np.mean(byts)),
                     "achieved_GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    if not fp8_act:
        out["dispatch"]["row_gather_kernel"], out["combine"]["kernel_without_shared"] = \
            comm_kernels_alone(cfg, L, halves[0])
    return out


def comm_kernels_alone(cfg, L, half, reps=20, reps_cold=10):
    """The data-moving kernels of the comm steps timed alone on microbatch 0's
    routing: the row gather of the dispatch (moe_dispatch_recv; its count and
    rank kernels excluded) and the combine without the shared-expert slabs.
    Warm: HIP events around `reps` back-to-back calls on the current stream
    (inputs may sit in the 256 MB MALL).  Cold: each call alone between two
    events, after a read of a 512 MiB scratch buffer has displaced the MALL."""
    import torch
    from combine_dual_overlap_amd import binding as B
    a, b = half
    n = b - a
    s = 4 if cfg.act == "f32" else 2
    x = L.x[a:b]
    inv = L.view(0, "inv", torch.int32, (n * cfg.k,), T=cfg.T)
    w = L.view(0, "topk_w", torch.float32, (n, cfg.k), T=cfg.T)
    inv_np = inv.cpu().numpy().reshape(n, cfg.k)
    M = int((inv_np >= 0).sum())
    t_hit = int((inv_np >= 0).any(axis=1).sum())
    rows = torch.empty(max(n * cfg.k, 1), cfg.H, dtype=x.dtype, device=x.device)
    scratch = torch.ones(128 << 20, dtype=torch.float32, device=x.device)     # 512 MiB
    out = torch.empty(n, cfg.H, dtype=x.dtype, device=x.device)
    calls = {"gather": lambda: B.moe_dispatch_recv(x, cfg.k, inv, rows),
             "combine": lambda: B.moe_combine(rows, n, cfg.k, inv, w, out)}
    byts = {"gather": t_hit * cfg.H * s + M * cfg.H * s + 4 * n * cfg.k,
            "combine": M * cfg.H * s + 8 * n * cfg.k + n * cfg.H * s}
    rec = []
    for name in ("gather", "combine"):
        for _ in range(3):
            calls[name]()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            calls[name]()
        t1.record()
        torch.cuda.synchronize()
        avg_s = t0.elapsed_time(t1) / reps / 1e3
        gbs = byts[name] / avg_s / 1e9
        cold = []
        for _ in range(reps_cold):
            scratch.sum()
            t0.record()
            calls[name]()
            t1.record()
            torch.cuda.synchronize()
            cold.append(t0.elapsed_time(t1) / 1e3)
        cold_s = float(np.median(cold))
        cold_gbs = byts[name] / cold_s / 1e9
        rec.append({"avg_us": round(avg_s * 1e6, 2), "algorithmic_bytes": int(byts[name]),
                    "achieved_GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                    "cold_median_us": round(cold_s * 1e6, 2), "cold_achieved_GBps": round(cold_gbs, 1),
                    "cold_frac_of_hbm_peak": round(cold_gbs / HBM_PEAK_GBS, 4)})
    return rec


def cpu_baseline(inp, cfg, budget_s: float, fp8_act=False, threads: int = 8):
    """The oracle (as it stands) on a bounded sample of the same workload: its
    first n tokens, float64 numpy with `threads` BLAS threads (the build
    host's 8 cores); one warm-up run, then the median of three.  n is the
    largest of 512, 256, 128, ... tokens whose warm-up run fits a quarter of
    the budget (a fixed cost, decoding every hit expert's weights, dominates
    small samples of the fp8-weight layers)."""
    import oracle as O
    import workloads as W
    from threadpoolctl import threadpool_limits
    ov = dict(W.oracle_view(inp), fp8_act=fp8_act)
    n = min(cfg.T, 512)
    with threadpool_limits(limits=threads):
        while True:
            sub = O.slice_view(ov, 0, n)
            t0 = time.perf_counter()
            O.moe_layer_expert(sub)
            warm = time.perf_counter() - t0
            if warm <= budget_s / 4 or n <= 16:
                break
            n //= 2
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            O.moe_layer_expert(sub)
            runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} tokens of {cfg.name} (T={cfg.T}), oracle.moe_layer_expert in float64 "
                      f"numpy/OpenBLAS on {threads} threads; warm-up {warm:.2f} s, then median of 3 runs "
                      f"{', '.join(f'{r:.2f}' for r in runs)} s"}


def _stats(v):
    v = np.asarray(v, np.float64)
    return {"median": round(float(np.median(v)), 5), "p10": round(float(np.percentile(v, 10)), 5),
            "p90": round(float(np.percentile(v, 90)), 5), "n": int(v.size)}


def schedule_trials(L, run, schedules, rounds, steps, warmup):
    """Interleaved repeated trials: each round times `steps` steps of every
    schedule, graph-replayed and eager, in a rotated order, with HIP events on
    the current (compute) stream around each trial.  Returns per schedule and
    mode the ms per step of every round."""
    import torch
    graphs = {}
    for sched in schedules:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run(sched)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(sched)
        graphs[sched] = g
    modes = {"graph": lambda sc: graphs[sc].replay(), "eager": lambda sc: run(sc)}
    for sched in schedules:
        for m in modes.values():
            for _ in range(warmup):
                m(sched)
    torch.cuda.synchronize()
    res = {m: {sc: [] for sc in schedules} for m in modes}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for r in range(rounds):
        order = schedules[r % len(schedules):] + schedules[:r % len(schedules)]
        for sched in order:
            for mname, m in modes.items():
                torch.cuda.synchronize()
                e0.record()
                for _ in range(steps):
                    m(sched)
                e1.record()
                torch.cuda.synchronize()
                res[mname][sched].append(e0.elapsed_time(e1) / steps)
    for g in graphs.values():
        del g
    return res


def summarize_trials(res, T):
    """Median and p10/p90 of ms per step and tokens/s per schedule, and the
    per-round paired ratios (time of the other schedule / time of DBO)."""
    out = {}
    for mode, per in res.items():
        o = {"ms_per_step": {sc: _stats(v) for sc, v in per.items()},
             "tokens_per_s": {sc: _stats([T / (x / 1e3) for x in v]) for sc, v in per.items()}}
        if "dbo" in per:
            d = np.asarray(per["dbo"])
            o["speedup_of_dbo_over"] = {sc: _stats(np.asarray(v) / d) for sc, v in per.items() if sc != "dbo"}
        out[mode] = o
    return out


COMM_KERNELS = ("k_disp_", "k_combine")


def overlap_from_trace(db_path: str, gap_us: float = 300.0):
    """Per-step overlap of a rocprofv3 kernel trace (rocpd SQLite database)
    of `bench.py --trace-steps`: the library's kernels are cut into steps at
    idle gaps longer than gap_us (the trace mode synchronises and pauses
    between steps) and into schedules at the longer pauses between them.  Per
    step: the wall time from the first kernel start to the last kernel end,
    the union of comm-kernel intervals (dispatch and combine), the union of
    compute-kernel intervals (router, top-k, expert GEMMs), and their
    intersection.  overlap % = intersection / step time; hidden comm % =
    intersection / comm union; exposed comm = step time - compute union."""
    import sqlite3
    con = sqlite3.connect(db_path)
    rows = [(n, s, e) for n, s, e in con.execute("select name, start, end from kernels order by start")
            if "dbomoe::" in n]
    if not rows:
        raise SystemExit(f"no library kernels in {db_path}")

    def union(iv):
        iv = sorted(iv)
        out = []
        for a, b in iv:
            if out and a <= out[-1][1]:
                out[-1][1] = max(out[-1][1], b)
            else:
                out.append([a, b])
        return out

    def length(u):
        return sum(b - a for a, b in u)

    def inter(u, v):
        i = j = 0
        tot = 0
        while i < len(u) and j < len(v):
            a, b = max(u[i][0], v[j][0]), min(u[i][1], v[j][1])
            if b > a:
                tot += b - a
            if u[i][1] < v[j][1]:
                i += 1
            else:
                j += 1
        return tot

    steps, cur, last_end = [], [], None
    for n, s0, e0 in rows:
        if last_end is not None and s0 - last_end > gap_us * 1e3:
            steps.append(cur)
            cur = []
        cur.append((n, s0, e0))
        last_end = e0 if last_end is None else max(last_end, e0)
    steps.append(cur)
    recs = []
    for st in steps:
        comm = union([[s0, e0] for n, s0, e0 in st if any(k in n for k in COMM_KERNELS)])
        comp = union([[s0, e0] for n, s0, e0 in st if not any(k in n for k in COMM_KERNELS)])
        wall = max(e0 for _, _, e0 in st) - min(s0 for _, s0, _ in st)
        recs.append({"start": min(s0 for _, s0, _ in st), "kernels": len(st), "wall_us": wall / 1e3,
                     "comm_us": length(comm) / 1e3, "compute_us": length(comp) / 1e3,
                     "overlap_us": inter(comm, comp) / 1e3})
    return recs


def trace_steps(L, run, schedules, n, torch):
    """Trace mode: n steps of every schedule, each step alone (synchronised,
    then a 1 ms pause), 5 ms between schedules, for a kernel trace."""
    for sched in schedules:
        for _ in range(3):
            run(sched)
        torch.cuda.synchronize()
        time.sleep(0.005)
        for _ in range(n):
            run(sched)
            torch.cuda.synchronize()
            time.sleep(0.001)
        time.sleep(0.005)
        log(f"bench: traced {n} separated steps of {sched}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed graph-replayed DBO steps (200 steps of the prefill layer: about 0.2 s, long enough to average the few-percent drift of the chip's speed over sub-second windows)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="layer configuration 1..5 (default 3)")
    ap.add_argument("--rounds", type=int, default=10, help="interleaved trial rounds per schedule")
    ap.add_argument("--trial-steps", type=int, default=20, help="steps per trial")
    ap.add_argument("--comm-cu-budget", type=int, default=0)
    ap.add_argument("--ffn-tile-m", type=int, default=0,
                    help="expert FFN row tile: 0 automatic, else 32, 64 or 128 rows")
    ap.add_argument("--fp8-act", action="store_true",
                    help="routed experts with fp8 activations (fp8-weight configurations 3 and 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=24.0)
    ap.add_argument("--secondary", type=int, default=2,
                    help="configuration timed as a secondary record after the headline (0: none)")
    ap.add_argument("--trace-steps", type=int, default=0,
                    help="trace mode: run this many separated steps of DBO, SERIAL and DBO_LATE_EVENT (eager) "
                         "for a rocprofv3 kernel trace, then exit")
    ap.add_argument("--overlap-from", default=None,
                    help="print the per-step overlap summary of a rocprofv3 kernel-trace database written "
                         "in trace mode (no GPU needed), then exit")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain elementwise copy of this many MiB three times, the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes")
    args = ap.parse_args()

    if args.overlap_from:
        print_overlap(args.overlap_from, ["dbo", "serial", "dbo_late_event"])
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the layer is one GPU's share of the expert-parallel work "
              f"and no multi-GPU path is built (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from combine_dual_overlap_amd import DeviceLayer
    from combine_dual_overlap_amd import binding as B

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)       # reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        del src, dst
        log(f"bench: copy calibration, 3 x {args.calibrate_copy_mib} MiB read + write")
    cfg = W.get_config(args.config)
    log(f"bench: generating {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I}")
    inp = W.make_inputs(cfg)
    if args.fp8_act and cfg.wdt != "fp8":
        print("--fp8-act needs fp8 weights (configurations 3 and 4)", file=sys.stderr)
        sys.exit(2)
    L = DeviceLayer(inp, device="cuda:0", fp8_act=args.fp8_act)
    K, Wm = args.steps, args.warmup
    T = cfg.T

    def run(sched):
        L.run(sched, comm_cu_budget=args.comm_cu_budget, ffn_tile_m=args.ffn_tile_m)

    if args.trace_steps:
        trace_steps(L, run, ["dbo", "serial", "dbo_late_event"], args.trace_steps, torch)
        return

    # The schedule comparison first: interleaved trials of every schedule,
    # graph-replayed and eager.  They also bring the chip to the clocks it
    # holds under this load, which a few warm-up steps from idle do not.
    schedules = ["dbo", "serial", "dbo_late_event", "unsplit"]
    log(f"bench: {args.rounds} interleaved rounds x {args.trial_steps} steps of {schedules}, graph and eager")
    trials = summarize_trials(schedule_trials(L, run, schedules, args.rounds, args.trial_steps, 3), T)

    # The headline: the DBO step captured once in a HIP graph (the whole step,
    # both streams and their events, one launch), W warm-up replays, then
    # exactly K timed replays bracketed by device syncs.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run("dbo")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run("dbo")
    log(f"bench: warmup {Wm}, timing {K} graph-replayed DBO steps")
    for _ in range(Wm):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        g.replay()
    torch.cuda.synchronize()
    dt_graph = time.perf_counter() - t0
    del g

    # Kernel timing: events around each microbatch's gate/up and down GEMMs on
    # the compute stream (the stream they are launched on), over more steps of
    # the DBO schedule.
    n_t = min(K, 128)
    L.ctx.set_timing(True)
    for _ in range(n_t):
        run("dbo")
    torch.cuda.synchronize()
    times = np.array([L.ctx.ffn_times(b) for b in range(n_t)])     # [n, 4] ms
    L.ctx.set_timing(False)
    gu_ms = times[:, [0, 2]]
    gu_ms = gu_ms[gu_ms > 0]
    dn_ms = times[:, [1, 3]]
    dn_ms = dn_ms[dn_ms > 0]

    # Dispatch and combine timed in the SERIAL schedule (nothing runs beside
    # them there), against their algorithmic bytes.
    L.ctx.set_timing(True)
    for _ in range(n_t):
        run("serial")
    torch.cuda.synchronize()
    comm = np.array([L.ctx.comm_times(b) for b in range(n_t)])     # [n, 4] ms
    L.ctx.set_timing(False)

    T0 = L.ctx.last_stats()["T0"]
    halves = [(0, T0), (T0, T)] if T0 < T else [(0, T)]
    counts = [L.view(mb, "counts", torch.int32, (cfg.E_loc,), T=T).cpu().numpy() for mb in range(len(halves))]
    rows = [b - a for a, b in halves]
    work = gateup_work(cfg, counts, rows, args.fp8_act)
    bytes_launch = float(np.mean([w[0] for w in work]))
    flops_launch = float(np.mean([w[1] for w in work]))
    avg_s = float(np.mean(gu_ms)) / 1e3
    mfma_peak = MFMA_PEAK_TFLOPS["f32" if cfg.act == "f32" else "fp8" if args.fp8_act else "bf16"]
    roofs = {gm: [ffn_expert_roof(cfg, c, n, gm, args.fp8_act) for c, n in zip(counts, rows)]
             for gm in ("gate_up", "down")}
    gu_roof = float(np.mean([r[0] for r in roofs["gate_up"]]))
    dn_roof = float(np.mean([r[0] for r in roofs["down"]]))
    mfma_part = float(np.mean([r[3] for r in roofs["gate_up"]]))
    hbm_bound = mfma_part < gu_roof / 2        # the bound that holds most of the per-expert roof
    traffic = read_traffic(cfg.name + ("_fp8act" if args.fp8_act else ""))
    ach_gbs = bytes_launch / avg_s / 1e9
    ach_tf = flops_launch / avg_s / 1e12
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(ach_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(ach_tf, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(ach_tf / mfma_peak, 4)}
    roof["traffic"] = traffic
    T_mb0 = halves[0][1] - halves[0][0]
    I_sh = cfg.n_shared * cfg.shared_I
    tile = args.ffn_tile_m or B.moe_ffn_auto_tile(B.dtype_code(L.x), B.dtype_code(L.w13), cfg.H, cfg.I,
                                                  -(-T_mb0 * cfg.k // cfg.E), T_mb0 if I_sh else 0, I_sh)
    if args.fp8_act:
        m = -(-T_mb0 * cfg.k // cfg.E)
        tile = (128 if args.ffn_tile_m >= 128 else 64) if args.ffn_tile_m else \
            (64 if m + 3 * m ** 0.5 + 1 <= 64 else 128)
    kname = ("k_gemm_nt_f32 (fp32 SIMT)" if cfg.act == "f32" else
             (f"k_gemm_f8d ({tile}-row tiles staged by LDS DMA, fp8 x fp8)" if cfg.H <= F8_DMA_MAX_K else
              f"k_gemm_f8 ({tile}-row LDS tiles, fp8 x fp8)") if args.fp8_act else
             "k_gemm_dma (128-row tiles staged by LDS DMA)" if (tile == 128 and cfg.wdt == "bf16" and not I_sh) else
             f"k_gemm_fp8w ({tile}-row tiles, fp8 codes staged by LDS DMA)" if (tile in (64, 128) and cfg.wdt == "fp8"
                                                                              and not I_sh) else
             f"k_gemm_nt ({tile}-row LDS tiles)")
    roof["kernel"] = f"gate/up expert GEMM + SwiGLU, routed and shared experts: {kname}, MODE_GATEUP"
    roof["avg_launch_us"] = round(avg_s * 1e6, 2)
    roof["algorithmic_bytes_per_launch"] = int(bytes_launch)
    roof["algorithmic_flops_per_launch"] = int(flops_launch)
    roof["mfma_frac"] = round(ach_tf / mfma_peak, 4)
    roof["hbm_frac"] = round(ach_gbs / HBM_PEAK_GBS, 4)
    roof["per_expert_roof_us"] = round(gu_roof * 1e6, 2)
    roof["frac_of_per_expert_roof"] = round(gu_roof / avg_s, 4)
    down = {"avg_launch_us": round(float(np.mean(dn_ms)) * 1e3, 2), "per_expert_roof_us": round(dn_roof * 1e6, 2),
            "frac_of_per_expert_roof": round(dn_roof / (float(np.mean(dn_ms)) / 1e3), 4)}

    comm_rec = comm_work(cfg, L, halves, comm, args.fp8_act)

    base = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        base = cpu_baseline(inp, cfg, args.cpu_budget_s, args.fp8_act)

    secondary = None
    if args.secondary and args.secondary != args.config:
        del L
        torch.cuda.empty_cache()
        secondary = secondary_record(args.secondary, args, W, DeviceLayer, torch)

    value = T * K / dt_graph
    dtype = "fp8" if args.fp8_act else {"f32": "f32", "bf16": "bf16"}[cfg.act]
    g_tr = trials["graph"]
    rec = {
        "metric": "MoE-layer tokens/sec (DBO vs serial) + MFMA util % and HBM GB/s % of peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(dt_graph / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded random activations and weights of the layer's shape)",
        "config": {"workload": cfg.name, "T": T, "split": [T0, T - T0] if T0 < T else [T], "H": cfg.H,
                   "E": cfg.E, "E_local": cfg.E_loc, "k": cfg.k, "I": cfg.I, "shared_experts": cfg.n_shared,
                   "weights": cfg.wdt, "expert_activations": "fp8" if args.fp8_act else cfg.act,
                   "schedule": "dbo", "comm_cu_budget": args.comm_cu_budget,
                   "execution": "HIP graph replay of one dbo_moe_layer call per step"},
        "dbo_speedup_vs_serial": g_tr["speedup_of_dbo_over"]["serial"]["median"],
        "dbo_speedup_vs_late_event": g_tr["speedup_of_dbo_over"]["dbo_late_event"]["median"],
        "schedule_trials": {"rounds": args.rounds, "steps_per_trial": args.trial_steps,
                            "order": "interleaved, rotated each round", **trials},
        "comm_steps": comm_rec,
        "kernel_ms": {"gate_up_avg": round(float(np.mean(gu_ms)), 4), "down_avg": round(float(np.mean(dn_ms)), 4)},
        "down_gemm": down,
        "roofline": roof,
        "cpu_baseline": base,
        "secondary": secondary,
    }
    print(json.dumps(rec), flush=True)


def print_overlap(db_path: str, schedules):
    """Markdown summary of overlap_from_trace: steps are grouped by schedule
    in the order trace mode runs them (each schedule's separated steps)."""
    recs = overlap_from_trace(db_path)
    # schedules are separated by the 5 ms pauses: cut where the gap to the previous step exceeds 3 ms
    groups, cur = [], [recs[0]]
    for a, b in zip(recs, recs[1:]):
        if b["start"] - (a["start"] + a["wall_us"] * 1e3) > 3e6:
            groups.append(cur)
            cur = []
        cur.append(b)
    groups.append(cur)
    groups = [g for g in groups if len(g) > 3]        # drop the warm-up clusters
    print("| schedule | steps | step us (median) | compute us | comm us | overlap us | overlap % of step | "
          "comm hidden % | exposed comm us |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|")
    for name, g in zip(schedules, groups[-len(schedules):]):
        med = lambda key: float(np.median([r[key] for r in g]))
        wall, comp, comm, ov = med("wall_us"), med("compute_us"), med("comm_us"), med("overlap_us")
        print(f"| {name} | {len(g)} | {wall:.1f} | {comp:.1f} | {comm:.1f} | {ov:.1f} | {100 * ov / wall:.1f} | "
              f"{100 * ov / comm:.1f} | {wall - comp:.1f} |")


def secondary_record(cid, args, W, DeviceLayer, torch):
    """A smaller record of another configuration: DBO, SERIAL and
    DBO_LATE_EVENT in interleaved graph-replayed trials, and the gate/up
    kernel against its per-expert roof."""
    cfg = W.get_config(cid)
    log(f"bench: secondary record {cfg.name}")
    L = DeviceLayer(W.make_inputs(cfg), device="cuda:0")
    run = lambda sched: L.run(sched)
    res = schedule_trials(L, run, ["dbo", "serial", "dbo_late_event"], max(3, args.rounds // 2),
                          args.trial_steps, 3)
    res.pop("eager")
    tr = summarize_trials(res, cfg.T)["graph"]
    L.ctx.set_timing(True)
    for _ in range(32):
        run("dbo")
    torch.cuda.synchronize()
    times = np.array([L.ctx.ffn_times(b) for b in range(32)])
    L.ctx.set_timing(False)
    gu = times[:, [0, 2]]
    gu_s = float(np.mean(gu[gu > 0])) / 1e3
    T0 = L.ctx.last_stats()["T0"]
    halves = [(0, T0), (T0, cfg.T)]
    counts = [L.view(mb, "counts", torch.int32, (cfg.E_loc,), T=cfg.T).cpu().numpy() for mb in range(2)]
    work = gateup_work(cfg, counts, [b - a for a, b in halves])
    nbytes = float(np.mean([w[0] for w in work]))
    roof = float(np.mean([ffn_expert_roof(cfg, c, b - a, "gate_up")[0] for c, (a, b) in zip(counts, halves)]))
    return {"workload": cfg.name, "T": cfg.T, "tokens_per_s_graph": tr["tokens_per_s"],
            "speedup_of_dbo_over": tr["speedup_of_dbo_over"],
            "gate_up": {"avg_launch_us": round(gu_s * 1e6, 2), "hbm_GBps": round(nbytes / gu_s / 1e9, 1),
                        "hbm_frac": round(nbytes / gu_s / 1e9 / HBM_PEAK_GBS, 4),
                        "frac_of_per_expert_roof": round(roof / gu_s, 4)}}


if __name__ == "__main__":
    main()
