"""Whole-layer GPU parity (dbo_moe_layer) against the CPU oracle: every
schedule on reduced shapes, the five full-size configurations on sampled
tokens, split edge cases, DBO == SERIAL bitwise, repeat determinism."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import assert_close, check_routing, inputs, rms_tol_for, to_f64, tol_for

pytestmark = pytest.mark.gpu

SCHEDULES = ["unsplit", "serial", "dbo", "dbo_late_event", "dbo_recv_hook"]


def _layer(inp, **kw):
    import combine_dual_overlap_amd as C
    C.binding.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return C.DeviceLayer(inp, **kw)


def _gpu_routing(L, cfg, ov, T0):
    """Checks each microbatch's ids (oracle selection on the GPU's own logits;
    near-ties only against the oracle's float64 logits) and returns the GPU
    ids of the whole batch."""
    halves = [(0, cfg.T)] if T0 is None else [(0, T0), (T0, cfg.T)]
    oracle_logits = O.moe_layer_expert(ov, tokens=np.arange(0))["logits"]
    all_ids = []
    for mb, (a, b) in enumerate(halves):
        n = b - a
        logits = to_f64(L.view(mb, "logits", torch.float32, (n, cfg.E)))
        ids = L.view(mb, "topk_ids", torch.int32, (n, cfg.k)).cpu().numpy()
        forced = None if ov["forced_ids"] is None else ov["forced_ids"][a:b]
        check_routing(ids, logits, oracle_logits[a:b], cfg, forced, f"mb{mb} ids")
        all_ids.append(ids)
    return np.vstack(all_ids)


def _reference(ov, gpu_ids, tokens=None):
    """The oracle layer taking the GPU's (checked) routing choices, so that a
    float near-tie cannot make the two pick different experts downstream."""
    return O.moe_layer_expert(dict(ov, forced_ids=gpu_ids.astype(np.int32)), tokens=tokens)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_layer_small(cid, schedule):
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    L = _layer(inp)
    print(f"layer cfg={cfg.name} schedule={schedule}", flush=True)
    out = L.run(schedule)
    torch.cuda.synchronize()
    st = L.ctx.last_stats()
    T0 = None if schedule == "unsplit" else (cfg.T + 1) // 2
    assert st["T0"] == (cfg.T if T0 is None else T0)
    if schedule.startswith("dbo"):
        assert st["yields_a"] == st["yields_b"] == (4 if schedule == "dbo_recv_hook" else 3)
    ids = _gpu_routing(L, cfg, ov, T0)
    ref = _reference(ov, ids)
    assert_close(to_f64(out), ref["out"], tol_for(cfg), f"out {cfg.name} {schedule}", ref["scale"])


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_dbo_equals_serial_bitwise_and_repeatable(cid):
    inp, _ = inputs(cid, True)
    L = _layer(inp)
    base = L.run("serial").clone()
    for sched in ["dbo", "dbo_late_event", "dbo_recv_hook"] + ["dbo"] * 17:
        out = L.run(sched)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           base.view(torch.int16) if base.dtype == torch.bfloat16 else base), sched


@pytest.mark.parametrize("cid,small,fp8_act", [(3, True, False), (3, False, False), (4, False, False),
                                                (5, False, False), (3, False, True)])
def test_dispatch_and_combine_beside_ffn(cid, small, fp8_act):
    """In the two-stream schedules the second microbatch's dispatch and the
    first one's combine take the kernels sized to fit beside the GEMM (the
    256-thread rank kernel over blocks of 1024 pairs, the 64-VGPR combine).
    The second microbatch's counts, offsets, perm and inv equal the oracle's
    dispatch of its ids bit for bit (ragged last block at the skewed shape),
    its bf16 rows are the token rows they name, and the layer output equals
    SERIAL's (the standard kernels) bitwise."""
    inp, _ = inputs(cid, small)
    cfg = inp["cfg"]
    L = _layer(inp, fp8_act=fp8_act)
    print(f"beside-ffn cfg={cfg.name} fp8_act={fp8_act}", flush=True)
    base = L.run("serial").clone()
    T0 = (cfg.T + 1) // 2
    n1 = cfg.T - T0
    for sched in ["dbo", "dbo_recv_hook", "dbo_late_event"]:
        out = L.run(sched)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), base.view(torch.int16)), sched
        ids = L.view(1, "topk_ids", torch.int32, (n1, cfg.k)).cpu().numpy()
        ref = O.dispatch_ref(ids, cfg.expert_begin, cfg.expert_end)
        M = int(ref["M"])
        E_loc = cfg.E_loc
        assert np.array_equal(L.view(1, "counts", torch.int32, (E_loc,)).cpu().numpy(), ref["counts"]), sched
        assert np.array_equal(L.view(1, "offsets", torch.int32, (E_loc + 1,)).cpu().numpy(), ref["offsets"]), sched
        assert np.array_equal(L.view(1, "perm", torch.int32, (M,)).cpu().numpy(), ref["perm"]), sched
        assert np.array_equal(L.view(1, "inv", torch.int32, (n1 * cfg.k,)).cpu().numpy(), ref["inv"]), sched
        if not fp8_act:
            rows = inp["x"][T0 + torch.from_numpy(ref["perm"] // cfg.k).long()]
            xp = L.view(1, "x_perm", torch.bfloat16, (M, cfg.H)).cpu()
            assert torch.equal(xp.view(torch.int16), rows.view(torch.int16)), sched


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_layer_full_size_sampled(cid):
    inp, ov = inputs(cid, False)
    cfg = inp["cfg"]
    L = _layer(inp)
    print(f"full layer cfg={cfg.name} T={cfg.T}", flush=True)
    out = L.run("dbo")
    torch.cuda.synchronize()
    T0 = (cfg.T + 1) // 2
    ids = _gpu_routing(L, cfg, ov, T0)
    rng = np.random.default_rng(cid)
    sample = np.unique(np.concatenate([[0, 1, T0 - 1, T0, T0 + 1, cfg.T - 1], rng.integers(0, cfg.T, 26)]))
    ref = _reference(ov, ids, tokens=sample)
    assert_close(to_f64(out[torch.from_numpy(sample).cuda()]), ref["out"], tol_for(cfg), f"out {cfg.name}",
                 ref["scale"])
    # properties that hold at any size: every dispatched row count adds up
    for mb, (a, b) in enumerate([(0, T0), (T0, cfg.T)]):
        E_loc = cfg.E_loc
        offs = L.view(mb, "offsets", torch.int32, (E_loc + 1,)).cpu().numpy()
        ids = L.view(mb, "topk_ids", torch.int32, (b - a, cfg.k)).cpu().numpy()
        local = ((ids >= cfg.expert_begin) & (ids < cfg.expert_end)).sum()
        assert offs[0] == 0 and offs[-1] == local and (np.diff(offs) >= 0).all()


@pytest.mark.parametrize("T", [1, 2, 3, 5, 33])
def test_split_edge_cases(T):
    cfg = W.get_config(2, small=True).replace(T=T)
    inp = W.make_inputs(cfg)
    ov = W.oracle_view(inp)
    L = _layer(inp)
    for sched in SCHEDULES:
        out = L.run(sched, min_tokens_to_split=4)
        torch.cuda.synchronize()
        st = L.ctx.last_stats()
        if sched != "unsplit" and T < 4:
            assert st["schedule"] == 0, "below min_tokens_to_split the layer runs unsplit"
        T0 = None if st["schedule"] == 0 else st["T0"]
        ref = _reference(ov, _gpu_routing(L, cfg, ov, T0))
        assert_close(to_f64(out), ref["out"], 1e-2, f"T={T} {sched}", ref["scale"])


def test_custom_split_point():
    inp, ov = inputs(5, True)
    cfg = inp["cfg"]
    L = _layer(inp)
    for split_at in [1, 7, cfg.T - 1]:
        out = L.run("dbo", split_at=split_at)
        torch.cuda.synchronize()
        assert L.ctx.last_stats()["T0"] == split_at
        ref = _reference(ov, _gpu_routing(L, cfg, ov, split_at))
        assert_close(to_f64(out), ref["out"], 1e-2, f"split_at={split_at}", ref["scale"])


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_comm_cu_budget_and_tile_overrides(cid):
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    L = _layer(inp)
    base = L.run("serial").clone()
    for budget in [1, 8, 64]:
        out = L.run("dbo", comm_cu_budget=budget)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), base.view(torch.int16))
    ref = O.moe_layer_expert(ov)
    for tm in [32, 64, 128]:
        out = L.run("dbo", ffn_tile_m=tm).clone()
        torch.cuda.synchronize()
        assert_close(to_f64(out), ref["out"], tol_for(cfg), f"tile_m={tm}", ref["scale"])
        again = L.run("serial", ffn_tile_m=tm).clone()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), again.view(torch.int16))


def test_layer_workspace_too_small_is_rejected():
    import combine_dual_overlap_amd as C
    inp, _ = inputs(1, True)
    L = _layer(inp)
    small = L.ws[: L.ws.numel() // 2]
    opts = C.binding.dbo_opts(C.binding.DBO_SCHED_DBO, 2, -1, 0, 0)
    with pytest.raises(C.binding.MoEError) as e:
        C.binding.dbo_moe_layer(L.ctx, L.desc, L.x, L.out, opts, small, torch.cuda.current_stream(), L.comm)
    assert e.value.status == C.binding.MOE_ERR_WORKSPACE


def test_timing_events_report_ffn_times():
    inp, _ = inputs(2, True)
    L = _layer(inp)
    L.ctx.set_timing(True)
    L.run("dbo")
    t = L.ctx.ffn_times()
    assert all(v > 0 for v in t), t
    c = L.ctx.comm_times()
    assert all(v > 0 for v in c), c
    L.run("unsplit")
    t2 = L.ctx.ffn_times()
    assert t2[0] > 0 and t2[1] > 0 and t2[2:] == [0.0, 0.0]
    c2 = L.ctx.comm_times()
    assert c2[0] > 0 and c2[2] > 0 and c2[1] == 0.0 and c2[3] == 0.0
    assert L.ctx.ffn_times(1)[2] > 0          # the earlier DBO call is still remembered
    L.ctx.set_timing(False)
    L.run("dbo")
    assert L.ctx.ffn_times() == t2            # untimed calls leave the record alone


@pytest.mark.parametrize("cid,fp8_act", [(2, False), (3, False), (5, False), (3, True), (4, True)])
@pytest.mark.parametrize("schedule", ["dbo", "serial", "dbo_recv_hook"])
def test_layer_captured_in_a_graph_replays_exactly(cid, fp8_act, schedule):
    """dbo_moe_layer under stream capture (the comm stream joins the capture
    through the layer's events; device-side counts, no host sync): every
    replay, with eager layer calls in between, equals the eager output bit for
    bit, and the eager output is within tolerance of the oracle (bf16 and fp8
    activations, every two-microbatch schedule)."""
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    L = _layer(inp, fp8_act=fp8_act)
    eager = L.run(schedule).clone()
    torch.cuda.synchronize()
    ids = _gpu_routing(L, cfg, ov, (cfg.T + 1) // 2)
    ref = _reference(dict(ov, fp8_act=fp8_act), ids)
    print(f"graph cfg={cfg.name} fp8_act={fp8_act} schedule={schedule}", flush=True)
    assert_close(to_f64(eager), ref["out"], tol_for(cfg, fp8_act), "eager", ref["scale"],
                 rms_tol=rms_tol_for(cfg, fp8_act))
    out = torch.empty_like(L.out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.run(schedule, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.run(schedule, out=out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        other = L.run("unsplit" if rep % 2 else schedule).clone()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(other.float()).all()
    del g
