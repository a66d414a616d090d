"""Pins of the CPU oracle against things other than itself: hand-derived
golden values (tests/golden/), closed forms, brute force on tiny inputs,
library routines for special cases, and invariants.  No GPU."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle.routing import route_cfg
import workloads as W
from conftest import read_golden

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- numerics

def test_fp8_golden_points():
    import os
    from conftest import GOLDEN
    with open(os.path.join(GOLDEN, "fp8_e4m3fn_points.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) >= 10
    for code_s, val_s, *_ in rows:
        code, want = int(code_s, 16), float(val_s)
        got = O.fp8_e4m3fn_value(code)
        if math.isnan(want):
            assert math.isnan(got), code_s
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code_s


def test_fp8_table_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = O.FP8_E4M3FN_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(tab))
    assert np.array_equal(ref[~nan], tab[~nan])
    assert nan.sum() == 2            # only 0x7F and 0xFF


def test_bf16_decode_matches_torch():
    u = RNG.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    u = u[(u & 0x7F80) != 0x7F80]    # drop inf/nan patterns
    ref = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.decode(u, "bf16"), ref)


def test_dequant_blocks_brute_force_ragged():
    R, C = 200, 300                  # not multiples of 128
    codes = RNG.integers(0, 256, size=(R, C), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    scales = RNG.uniform(0.5, 2.0, size=(2, 3)).astype(np.float32)
    got = O.dequant_fp8_blocks(codes, scales)
    for r in range(0, R, 7):
        for c in range(0, C, 11):
            want = O.fp8_e4m3fn_value(codes[r, c]) * float(scales[r // 128, c // 128])
            assert got[r, c] == want


def test_workload_fp8_quantisation_roundtrips_within_half_ulp():
    w = torch.randn(256, 384, generator=torch.Generator().manual_seed(3)) * 0.02
    codes, scales = W.quantize_fp8_blocks(w)
    deq = O.dequant_fp8_blocks(codes.numpy(), scales.numpy())
    rel = np.abs(deq - w.double().numpy()) / (np.abs(w.double().numpy()) + 1e-30)
    big = np.abs(w.numpy()) > 1e-3
    assert rel[big].max() <= 2.0 ** -4 + 1e-9   # 3 mantissa bits -> half ulp 2^-4


# ---------------------------------------------------------------- routing

def test_router_logits_brute_force():
    x = RNG.normal(size=(5, 7))
    wr = RNG.normal(size=(4, 7))
    b = RNG.normal(size=4)
    got = O.router_logits(x, wr, b)
    for t in range(5):
        for e in range(4):
            want = sum(x[t, h] * wr[e, h] for h in range(7)) + b[e]
            assert abs(got[t, e] - want) < 1e-12


def test_softmax_matches_scipy_and_sums_to_one():
    from scipy.special import softmax
    l = RNG.normal(size=(9, 13)) * 3
    p = O.softmax_rows(l)
    assert np.allclose(p, softmax(l, axis=1), rtol=0, atol=1e-15)
    assert np.allclose(p.sum(1), 1.0, atol=1e-15)


def test_sigmoid_closed_forms():
    v = O.sigmoid(np.array([[0.0, math.log(3.0), -math.log(3.0), 50.0]]))
    assert v[0, 0] == 0.5
    assert abs(v[0, 1] - 0.75) < 1e-15 and abs(v[0, 2] - 0.25) < 1e-15
    assert abs(v[0, 3] - 1.0) < 1e-15


def _brute_topk(row, k):
    return [e for _, e in sorted(((-v, e) for e, v in enumerate(row)))][:k]


@pytest.mark.parametrize("E,k", [(4, 1), (6, 3), (8, 8), (9, 4)])
def test_select_topk_brute_force_with_ties(E, k):
    vals = RNG.integers(-3, 3, size=(50, E)).astype(np.float64)   # many ties
    got = O.select_topk(vals, k)
    for t in range(50):
        assert list(got[t]) == _brute_topk(vals[t], k)
        sel = set(got[t])
        lo = min(vals[t, list(sel)])
        assert all(vals[t, e] <= lo for e in range(E) if e not in sel)


def test_select_topk_k_equals_E_is_a_permutation():
    vals = RNG.normal(size=(20, 16))
    got = O.select_topk(vals, 16)
    assert all(sorted(r) == list(range(16)) for r in got)


def _brute_grouped(s, k, G, keep, topn):
    E = len(s)
    per = E // G
    gs = [sum(sorted(s[q * per:(q + 1) * per])[-topn:]) for q in range(G)]
    best, best_set = -1, None
    for subset in itertools.combinations(range(G), keep):
        tot = sum(gs[q] for q in subset)
        if tot > best:
            best, best_set = tot, subset
    cand = [e for e in range(E) if e // per in best_set]
    return [e for _, e in sorted((-s[e], e) for e in cand)][:k]


@pytest.mark.parametrize("E,G,keep,k", [(8, 4, 2, 3), (32, 8, 4, 8), (24, 6, 3, 5), (16, 4, 1, 2)])
def test_select_grouped_brute_force(E, G, keep, k):
    s = O.sigmoid(RNG.normal(size=(40, E)) * 2)
    got = O.select_grouped(s, k, G, keep, 2)
    for t in range(40):
        assert list(got[t]) == _brute_grouped(list(s[t]), k, G, keep, 2)


def test_grouped_with_one_group_is_plain_topk():
    s = O.sigmoid(RNG.normal(size=(30, 12)))
    assert np.array_equal(O.select_grouped(s, 4, 1, 1, 2), O.select_topk(s, 4))


def test_grouped_routing_golden():
    g = read_golden("grouped_routing_handcalc.txt")
    logits = np.array([[float(v) for v in g["logits"]]])
    ids, w = O.route(logits, "sigmoid", int(g["k"][0]), renormalize=True,
                     n_groups=int(g["n_groups"][0]), topk_groups=int(g["topk_groups"][0]))
    assert list(ids[0]) == [int(v) for v in g["ids"]]
    assert np.allclose(w[0], [float(v) for v in g["weights"]], rtol=0, atol=1e-15)


def test_route_weights_softmax_and_renorm():
    l = RNG.normal(size=(25, 10))
    ids, w = O.route(l, "softmax", 3)
    p = O.softmax_rows(l)
    assert np.array_equal(w, np.take_along_axis(p, ids.astype(np.int64), 1))
    assert (w.sum(1) <= 1 + 1e-15).all()
    ids2, w2 = O.route(l, "softmax", 3, renormalize=True)
    assert np.array_equal(ids, ids2)
    assert np.allclose(w2.sum(1), 1.0, atol=1e-15)
    _, w3 = O.route(l, "softmax", 3, routed_scale=2.5)
    assert np.allclose(w3, 2.5 * w, rtol=1e-15, atol=0)


def test_route_forced_ids():
    l = RNG.normal(size=(6, 8))
    forced = np.array([[3, 1], [0, 7], [5, 2], [2, 5], [6, 4], [1, 0]], np.int32)
    ids, w = O.route(l, "softmax", 2, renormalize=True, forced_ids=forced)
    assert np.array_equal(ids, forced)
    p = O.softmax_rows(l)
    for t in range(6):
        a, b = p[t, forced[t, 0]], p[t, forced[t, 1]]
        assert np.allclose(w[t], [a / (a + b), b / (a + b)], rtol=1e-15)


def test_softmax_selection_on_logits_equals_selection_on_probabilities():
    l = RNG.normal(size=(40, 64))
    assert np.array_equal(O.select_topk(l, 6), O.select_topk(O.softmax_rows(l), 6))


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("case", ["A", "B"])
def test_dispatch_golden(case):
    g = read_golden("dispatch_handcalc.txt")
    T, k = int(g["T"][0]), int(g["k"][0])
    ids = np.array([int(v) for v in g["ids"]]).reshape(T, k)
    lo, hi = (int(v) for v in g[f"{case}.range"])
    d = O.dispatch_ref(ids, lo, hi, tile_m=int(g[f"{case}.tile_m"][0]))
    for key in ["counts", "offsets", "perm", "inv", "tile_offsets"]:
        assert list(d[key]) == [int(v) for v in g[f"{case}.{key}"]], key


def _brute_dispatch(ids, lo, hi):
    T, k = ids.shape
    buckets = [[] for _ in range(hi - lo)]
    for p in range(T * k):                     # visiting p in order keeps it stable
        e = ids[p // k, p % k]
        if lo <= e < hi:
            buckets[e - lo].append(p)
    perm = [p for b in buckets for p in b]
    inv = [-1] * (T * k)
    for pos, p in enumerate(perm):
        inv[p] = pos
    return [len(b) for b in buckets], perm, inv


@pytest.mark.parametrize("T,k,E,lo,hi", [(37, 3, 9, 0, 9), (50, 4, 16, 4, 12), (1, 2, 4, 0, 4),
                                         (64, 8, 256, 0, 32), (20, 1, 3, 2, 3)])
def test_dispatch_brute_force_and_invariants(T, k, E, lo, hi):
    ids = np.stack([RNG.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    d = O.dispatch_ref(ids, lo, hi, tile_m=16)
    counts, perm, inv = _brute_dispatch(ids, lo, hi)
    assert list(d["counts"]) == counts
    assert list(d["perm"]) == perm
    assert list(d["inv"]) == inv
    M = d["M"]
    assert d["offsets"][0] == 0 and d["offsets"][-1] == M == sum(counts)
    assert (np.diff(d["offsets"]) >= 0).all()
    assert np.array_equal(d["inv"][d["perm"]], np.arange(M))          # inv o perm = id
    local = (ids.reshape(-1) >= lo) & (ids.reshape(-1) < hi)
    assert ((d["inv"] >= 0) == local).all()
    if lo == 0 and hi == E:
        assert M == T * k
        assert np.array_equal(np.bincount(d["perm"] // k, minlength=T), np.full(T, k))
    assert list(d["tile_offsets"][1:] - d["tile_offsets"][:-1]) == [-(-c // 16) for c in counts]


def test_dispatch_empty():
    d = O.dispatch_ref(np.zeros((0, 4), np.int32), 0, 8, tile_m=8)
    assert d["M"] == 0 and list(d["offsets"]) == [0] * 9


# ---------------------------------------------------------------- FFN

def test_silu_closed_forms():
    g = np.array([0.0, math.log(3.0), -60.0, 60.0])
    s = O.silu(g)
    assert s[0] == 0.0
    assert abs(s[1] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(s[2]) < 1e-20 and abs(s[3] - 60.0) < 1e-12


def test_swiglu_matches_torch_dense_mlp():
    H, I, n = 24, 40, 7
    x = RNG.normal(size=(n, H))
    w13 = RNG.normal(size=(2 * I, H))
    w2 = RNG.normal(size=(H, I))
    tx, t13, t2 = (torch.from_numpy(a) for a in (x, w13, w2))
    ref = (torch.nn.functional.silu(tx @ t13[:I].T) * (tx @ t13[I:].T)) @ t2.T
    assert np.allclose(O.swiglu_expert(x, w13, w2), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_zero_w2_gives_zero():
    x = RNG.normal(size=(3, 8))
    assert not O.swiglu_expert(x, RNG.normal(size=(10, 8)), np.zeros((8, 5))).any()


def test_grouped_ffn_ref_rows():
    H, I = 8, 6
    ws = [(RNG.normal(size=(2 * I, H)), RNG.normal(size=(H, I))) for _ in range(3)]
    offsets = np.array([0, 2, 2, 5])
    x = RNG.normal(size=(5, H))
    y = O.grouped_ffn_ref(x, offsets, lambda e: ws[e])
    assert np.allclose(y[0:2], O.swiglu_expert(x[0:2], *ws[0]))
    assert np.allclose(y[2:5], O.swiglu_expert(x[2:5], *ws[2]))


# ---------------------------------------------------------------- layer

def _tiny_view(cfg, x, wr, w13, w2, bias=None, forced=None, shared=((), ())):
    return dict(cfg=cfg, x=np.asarray(x, np.float32), act="f32", w_router=np.asarray(wr, np.float32),
                logit_bias=bias, forced_ids=forced, w13=np.asarray(w13, np.float32),
                w2=np.asarray(w2, np.float32), wdt="f32", w13_scale=None, w2_scale=None,
                shared_w13=list(shared[0]), shared_w2=list(shared[1]), shared_wdt="f32")


def test_tiny_layer_golden():
    g = read_golden("tiny_layer_handcalc.txt")
    cfg = W.LayerConfig("golden", T=2, H=2, E=3, k=2, I=1, act="f32", wdt="f32")
    f = lambda key: np.array([float(v) for v in g[key]])
    ov = _tiny_view(cfg, f("x").reshape(2, 2), f("w_router").reshape(3, 2),
                    f("w13").reshape(3, 2, 2), f("w2").reshape(3, 2, 1))
    for layer in (O.moe_layer_token, O.moe_layer_expert):
        r = layer(ov)
        assert r["ids"].reshape(-1).tolist() == [int(v) for v in g["ids"]]
        assert np.allclose(r["out"].reshape(-1), f("out"), rtol=0, atol=1e-15)


def test_identical_experts_scale_dense_mlp():
    cfg = W.LayerConfig("same", T=20, H=16, E=6, k=3, I=12, act="f32", wdt="f32")
    x = RNG.normal(size=(20, 16)).astype(np.float32)
    wr = RNG.normal(size=(6, 16)).astype(np.float32)
    a = RNG.normal(size=(24, 16)).astype(np.float32)
    b = RNG.normal(size=(16, 12)).astype(np.float32)
    ov = _tiny_view(cfg, x, wr, np.stack([a] * 6), np.stack([b] * 6))
    r = O.moe_layer_expert(ov)
    mlp = O.swiglu_expert(x.astype(np.float64), a.astype(np.float64), b.astype(np.float64))
    assert np.allclose(r["out"], r["w"].sum(1)[:, None] * mlp, rtol=1e-12, atol=1e-12)


def test_k1_renormalised_is_pure_unpermute():
    cfg = W.LayerConfig("k1", T=15, H=8, E=4, k=1, I=6, act="f32", wdt="f32", renormalize=True)
    x = RNG.normal(size=(15, 8)).astype(np.float32)
    wr = RNG.normal(size=(4, 8)).astype(np.float32)
    w13 = RNG.normal(size=(4, 12, 8)).astype(np.float32)
    w2 = RNG.normal(size=(4, 8, 6)).astype(np.float32)
    r = O.moe_layer_expert(_tiny_view(cfg, x, wr, w13, w2))
    assert np.allclose(r["w"], 1.0, rtol=0, atol=1e-15)
    for t in range(15):
        e = r["ids"][t, 0]
        want = O.swiglu_expert(x[t:t + 1].astype(np.float64), w13[e].astype(np.float64),
                               w2[e].astype(np.float64))[0]
        assert np.allclose(r["out"][t], want, rtol=1e-12, atol=1e-12)


def test_two_shared_experts_equal_one_concatenated():
    H, I = 10, 7
    s13 = [RNG.normal(size=(2 * I, H)) for _ in range(2)]
    s2 = [RNG.normal(size=(H, I)) for _ in range(2)]
    x = RNG.normal(size=(5, H))
    two = sum(O.swiglu_expert(x, a, b) for a, b in zip(s13, s2))
    cat13 = np.vstack([s13[0][:I], s13[1][:I], s13[0][I:], s13[1][I:]])
    cat2 = np.hstack(s2)
    assert np.allclose(O.swiglu_expert(x, cat13, cat2), two, rtol=1e-12, atol=1e-12)


def test_nonlocal_tokens_get_zero():
    cfg = W.LayerConfig("loc", T=30, H=8, E=8, k=2, I=4, act="f32", wdt="f32",
                        expert_begin=2, expert_end=4)
    x = RNG.normal(size=(30, 8)).astype(np.float32)
    wr = RNG.normal(size=(8, 8)).astype(np.float32)
    w13 = RNG.normal(size=(2, 8, 8)).astype(np.float32)
    w2 = RNG.normal(size=(2, 8, 4)).astype(np.float32)
    ov = _tiny_view(cfg, x, wr, w13, w2)
    r = O.moe_layer_expert(ov)
    rt = O.moe_layer_token(ov)
    none_local = ~((r["ids"] >= 2) & (r["ids"] < 4)).any(1)
    assert none_local.any()
    assert not r["out"][none_local].any()
    assert np.allclose(r["out"], rt["out"], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_small_configs_token_equals_expert_and_split_equals_unsplit(cid):
    cfg = W.get_config(cid, small=True)
    ov = W.oracle_view(W.make_inputs(cfg))
    sample = np.unique(np.concatenate([np.arange(8), np.arange(cfg.T - 8, cfg.T),
                                       RNG.integers(0, cfg.T, 8)]))
    re = O.moe_layer_expert(ov)
    rt = O.moe_layer_token(ov, tokens=sample)
    assert np.allclose(rt["out"], re["out"][sample], rtol=1e-11, atol=1e-13)
    rs = O.moe_layer_microbatched(ov)
    assert rs["T0"] == (cfg.T + 1) // 2
    assert np.array_equal(rs["ids"], re["ids"])
    assert np.allclose(rs["out"], re["out"], rtol=1e-12, atol=1e-14)
    # per-token literal layer: split output is bitwise the unsplit output
    T0 = rs["T0"]
    half = O.moe_layer_token(O.slice_view(ov, T0, cfg.T), tokens=sample[sample >= T0] - T0)
    assert np.array_equal(half["out"], rt["out"][sample >= T0])


@pytest.mark.parametrize("cid", [2, 3, 5])
def test_dispatch_ffn_combine_reproduces_layer(cid):
    cfg = W.get_config(cid, small=True)
    ov = W.oracle_view(W.make_inputs(cfg))
    r = O.moe_layer_expert(ov)
    x = O.decode(ov["x"], ov["act"])
    d = O.dispatch_ref(r["ids"], cfg.expert_begin, cfg.expert_end)
    x_perm = x[d["perm"] // cfg.k]
    y = O.grouped_ffn_ref(x_perm, d["offsets"], lambda e: O.expert_weights(ov, e))
    shared = None
    if cfg.n_shared:
        shared = sum(O.swiglu_expert(x, a, b) for a, b in O.shared_weights(ov))
    out = O.combine_ref(y, d["inv"], r["w"], shared)
    assert np.allclose(out, r["out"], rtol=1e-11, atol=1e-13)


def test_split_rule():
    assert O.split_point(64) == 32 and O.split_point(6001) == 3001
    assert O.split_point(1) is None
    assert O.split_point(3, min_tokens_to_split=4) is None
    assert O.split_point(4, min_tokens_to_split=4) == 2
    assert O.split_point(10, split_at=10) is None and O.split_point(10, split_at=0) is None
    assert O.split_point(10, split_at=3) == 3


def test_c5_workload_has_empty_experts_in_each_half():
    cfg = W.get_config(5, small=True)
    ov = W.oracle_view(W.make_inputs(cfg))
    r = O.moe_layer_expert(ov, tokens=np.arange(2))
    T0 = O.split_point(cfg.T)
    for a, b in [(0, T0), (T0, cfg.T)]:
        d = O.dispatch_ref(r["ids"][a:b], 0, cfg.E)
        assert (d["counts"] == 0).sum() >= 1
    assert sum(cfg.seq_lens) == cfg.T
    # one request crosses the split
    ends = np.cumsum(cfg.seq_lens)
    starts = ends - np.array(cfg.seq_lens)
    assert ((starts < T0) & (ends > T0)).any()


def test_forced_uniform_ids_distinct_and_in_range():
    cfg = W.get_config(3, small=True)
    inp = W.make_inputs(cfg)
    f = inp["forced_ids"].numpy()
    assert f.shape == (cfg.T, cfg.k) and f.min() >= 0 and f.max() < cfg.E
    assert all(len(set(r)) == cfg.k for r in f)


def test_error_scale_bounds_output_and_is_tight_for_nonnegative_terms():
    cfg = W.LayerConfig("pos", T=12, H=8, E=4, k=2, I=6, act="f32", wdt="f32")
    x = RNG.uniform(0.1, 1.0, size=(12, 8)).astype(np.float32)
    wr = RNG.normal(size=(4, 8)).astype(np.float32)
    w13 = RNG.uniform(0.1, 1.0, size=(4, 12, 8)).astype(np.float32)
    w2 = RNG.uniform(0.1, 1.0, size=(4, 8, 6)).astype(np.float32)
    r = O.moe_layer_expert(_tiny_view(cfg, x, wr, w13, w2))
    assert (r["out"] > 0).all()
    assert np.allclose(r["scale"], r["out"], rtol=1e-13, atol=0)   # all terms >= 0: |sum| = sum |.|
    w2n = RNG.normal(size=(4, 8, 6)).astype(np.float32)
    r2 = O.moe_layer_expert(_tiny_view(cfg, x, wr, w13, w2n))
    assert (np.abs(r2["out"]) <= r2["scale"] * (1 + 1e-12)).all()
    assert (np.abs(r2["out"]) < r2["scale"]).any()


def test_combine_scale():
    y = np.array([[1.0, -2.0], [3.0, 4.0]])
    out, s = O.combine_ref(y, np.array([0, 1]), np.array([[0.5, -1.0]]), with_scale=True)
    assert np.allclose(out, [[0.5 - 3.0, -1.0 - 4.0]]) and np.allclose(s, [[0.5 + 3.0, 1.0 + 4.0]])
