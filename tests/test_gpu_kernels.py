"""Per-entry-point GPU parity against the CPU oracle (moe_route_topk,
moe_dispatch, moe_grouped_ffn, moe_combine), on reduced shapes of the five
layer configurations and on edge cases."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import assert_close, check_ids, check_routing, inputs, routing_inputs, to_f64, tol_for

pytestmark = pytest.mark.gpu

CIDS = [1, 2, 3, 4, 5]


def _gpu():
    import combine_dual_overlap_amd as C
    C.binding.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return C


def _route(C, cfg, x, w_router, bias=None, forced=None):
    B = C.binding
    T = x.shape[0]
    p = B.route_params(cfg.E, cfg.k, cfg.score, cfg.renormalize, cfg.n_groups, cfg.topk_groups,
                       cfg.group_topn, cfg.routed_scale)
    ids = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
    logits = torch.empty(T, cfg.E, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(B.moe_route_workspace_size(T, cfg.H, cfg.E), 256), dtype=torch.uint8, device="cuda")
    B.moe_route_topk(x, w_router, p, ids, w, ws, logits_out=logits, logit_bias=bias, forced_ids=forced)
    torch.cuda.synchronize()
    return ids, w, logits


@pytest.mark.parametrize("cid", CIDS)
def test_route_topk(cid):
    C = _gpu()
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    dev = lambda t: None if t is None else t.cuda()
    ids, w, logits = _route(C, cfg, dev(inp["x"]), dev(inp["w_router"]), dev(inp["logit_bias"]),
                            dev(inp["forced_ids"]))
    print(f"route cfg={cfg.name} T={cfg.T}", flush=True)
    ref = O.moe_layer_expert(ov, tokens=np.arange(1))       # routing covers every token
    gl = to_f64(logits)
    check_routing(ids.cpu().numpy(), gl, ref["logits"], cfg, ov["forced_ids"])
    ref_ids, ref_w, diff = check_ids(ids.cpu().numpy(), gl, cfg, ov["forced_ids"])
    ok = ~diff
    assert np.abs(w.cpu().double().numpy()[ok] - ref_w[ok]).max() < 1e-5


# Edge shapes of the selection: one expert; k = E; the largest k (16) with 64
# and 256 experts (one and four experts per lane); experts not a multiple of
# 64; group-limited routing with k = 16 and with uneven groups; forced ids.
@pytest.mark.parametrize("E,k,score,renorm,G,TG,forced", [
    (1, 1, "softmax", False, 1, 1, False), (5, 5, "softmax", True, 1, 1, False),
    (64, 16, "softmax", False, 1, 1, False), (256, 16, "softmax", True, 1, 1, False),
    (200, 7, "sigmoid", False, 1, 1, False), (256, 16, "sigmoid", True, 8, 4, False),
    (96, 3, "sigmoid", True, 4, 2, False), (128, 8, "softmax", True, 1, 1, True)])
def test_route_edge_shapes(E, k, score, renorm, G, TG, forced):
    C = _gpu()
    T, H = 300, 256
    cfg = W.LayerConfig("edge", T=T, H=H, E=E, k=k, I=64, act="bf16", wdt="bf16", score=score,
                        renormalize=renorm, n_groups=G, topk_groups=TG)
    g = torch.Generator().manual_seed(E * 100 + k)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    wr = (torch.randn(E, H, generator=g) * 0.1).to(torch.bfloat16)
    fids = None
    if forced:
        fids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    ids, w, logits = _route(C, cfg, x.cuda(), wr.cuda(), forced=None if fids is None else fids.cuda())
    print(f"route edge E={E} k={k} {score} groups={G}/{TG} forced={forced}", flush=True)
    ol = O.router_logits(O.decode(W.bits(x), "bf16"), O.decode(W.bits(wr), "bf16"))
    gl = to_f64(logits)
    assert (np.abs(gl - ol) <= 1e-4 + 1e-6 * np.abs(ol)).all()
    fnp = None if fids is None else fids.numpy()
    ref_ids, ref_w, diff = check_ids(ids.cpu().numpy(), gl, cfg, fnp)
    ok = ~diff
    assert np.abs(w.cpu().double().numpy()[ok] - ref_w[ok]).max() < 1e-5
    if forced:
        assert np.array_equal(ids.cpu().numpy(), fnp)


def test_route_ties_pick_lower_index():
    C = _gpu()
    cfg = W.LayerConfig("ties", T=8, H=128, E=64, k=4, I=64, act="bf16", wdt="bf16")
    x = torch.zeros(8, 128, dtype=torch.bfloat16)
    x[:, 0] = 1.0
    wr = torch.zeros(64, 128, dtype=torch.bfloat16)
    wr[[5, 9, 40, 63], 0] = 2.0         # four experts tie at the top
    wr[[1, 2], 0] = 1.0
    ids, w, logits = _route(C, cfg, x.cuda(), wr.cuda())
    assert ids.cpu().tolist() == [[5, 9, 40, 63]] * 8
    assert torch.allclose(w.cpu(), w.cpu()[:, :1].expand(8, 4))


def _dispatch(C, cfg, x, ids, tile_m=16, two_phase=False):
    B = C.binding
    T = x.shape[0]
    E_loc = cfg.expert_end - cfg.expert_begin
    cap = max(T * cfg.k, 1)
    counts = torch.full((E_loc,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E_loc + 1,), -7, dtype=torch.int32, device="cuda")
    toff = torch.full((E_loc + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    x_perm = torch.zeros(cap, cfg.H, dtype=x.dtype, device="cuda")
    ws = torch.empty(B.moe_dispatch_workspace_size(T, cfg.k, E_loc), dtype=torch.uint8, device="cuda")
    if two_phase:       # send (count, scan, rank), then the receive hook (row gather)
        B.moe_dispatch_send(ids, cfg.E, cfg.expert_begin, cfg.expert_end, counts, offsets, perm, inv, ws,
                            tile_m=tile_m, tile_offsets=toff)
        B.moe_dispatch_recv(x, cfg.k, inv, x_perm)
    else:
        B.moe_dispatch(x, ids, cfg.E, cfg.expert_begin, cfg.expert_end, counts, offsets, perm, inv, x_perm, ws,
                       tile_m=tile_m, tile_offsets=toff)
    torch.cuda.synchronize()
    return dict(counts=counts, offsets=offsets, tile_offsets=toff, perm=perm, inv=inv, x_perm=x_perm, ws=ws)


def _check_dispatch(cfg, x_cpu, ids_np, g, tile_m=16):
    ref = O.dispatch_ref(ids_np, cfg.expert_begin, cfg.expert_end, tile_m=tile_m)
    M = ref["M"]
    assert np.array_equal(g["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(g["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(g["tile_offsets"].cpu().numpy(), ref["tile_offsets"])
    assert np.array_equal(g["perm"].cpu().numpy()[:M], ref["perm"])
    assert np.array_equal(g["inv"].cpu().numpy()[:ids_np.size], ref["inv"])
    xp = g["x_perm"].cpu()[:M]
    want = x_cpu[torch.from_numpy(ref["perm"] // cfg.k).long()]
    assert torch.equal(xp.view(torch.int16) if xp.dtype == torch.bfloat16 else xp.view(torch.int32),
                       want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32))
    return ref


@pytest.mark.parametrize("cid", CIDS)
@pytest.mark.parametrize("small", [True, False])
def test_dispatch(cid, small):
    C = _gpu()
    inp, ov = routing_inputs(cid, small)         # dispatch needs x and the ids, not the expert weights
    cfg = inp["cfg"]
    T0 = O.split_point(cfg.T)
    ids_all = O.moe_layer_expert(ov, tokens=np.arange(0))["ids"]
    print(f"dispatch cfg={cfg.name} T={cfg.T}", flush=True)
    for a, b in [(0, T0), (T0, cfg.T)]:
        x = inp["x"][a:b]
        ids = ids_all[a:b]
        g = _dispatch(C, cfg, x.cuda(), torch.from_numpy(ids).cuda())
        _check_dispatch(cfg, x, ids, g)
        assert C.binding.moe_get_device_error(g["ws"]) == 0


# Dispatch paths: up to 2048 pairs and 256 local experts one workgroup
# counts, scans and ranks (pairs taken 1024 at a time); up to 256 local experts
# and 65536 entries of 1024-pair block histograms, a count kernel and a rank
# kernel that scans for itself; beyond, count, scan and rank kernels over
# 256-pair blocks.  A one-call dispatch on the middle path with at most 16384
# histogram entries folds the rank into the gather (groups of 16
# tokens; with k = 6 a group's pairs straddle the 1024-pair count blocks).
# The shapes below cover each path, partial last blocks and groups, one local
# expert, non-local pairs and the boundaries between the paths.
@pytest.mark.parametrize("T,k,E,lo,hi", [(1, 1, 1, 0, 1), (3, 2, 5, 1, 4), (257, 6, 64, 0, 64),
                                         (64, 16, 300, 100, 300), (256, 8, 64, 0, 64),
                                         (2049, 1, 8, 0, 8), (300, 8, 256, 0, 32), (5000, 1, 1, 0, 1),
                                         (1024, 8, 64, 0, 64), (1025, 8, 64, 0, 64),
                                         (2048, 4, 256, 0, 256), (3000, 8, 256, 32, 64),
                                         (3001, 6, 64, 0, 64), (200, 16, 64, 0, 64),
                                         (9000, 8, 256, 0, 256),
                                         (8193, 8, 64, 0, 64), (1000, 3, 300, 0, 257),
                                         (33000, 8, 256, 0, 256)])
@pytest.mark.parametrize("two_phase", [False, True])
def test_dispatch_shapes(T, k, E, lo, hi, two_phase):
    C = _gpu()
    rng = np.random.default_rng(T * 31 + k)
    cfg = W.LayerConfig("d", T=T, H=128, E=E, k=k, I=64, act="bf16", wdt="bf16", expert_begin=lo, expert_end=hi)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = torch.randn(T, 128).to(torch.bfloat16)
    g = _dispatch(C, cfg, x.cuda(), torch.from_numpy(ids).cuda(), two_phase=two_phase)
    _check_dispatch(cfg, x, ids, g)


def test_dispatch_all_to_one_expert_and_repeats():
    C = _gpu()
    T, k = 700, 4
    cfg = W.LayerConfig("one", T=T, H=256, E=8, k=k, I=64, act="f32", wdt="f32")
    ids = np.full((T, k), 3, np.int32)          # repeated ids inside a token are dispatched too
    x = torch.randn(T, 256)
    g = _dispatch(C, cfg, x.cuda(), torch.from_numpy(ids).cuda())
    _check_dispatch(cfg, x, ids, g)


@pytest.mark.parametrize("T,E", [(10, 8), (1500, 8), (4000, 300)])     # each dispatch path
def test_dispatch_flags_bad_ids(T, E):
    C = _gpu()
    cfg = W.LayerConfig("bad", T=T, H=128, E=E, k=2, I=64, act="bf16", wdt="bf16")
    ids = np.tile(np.array([[1, 2]], np.int32), (T, 1))
    bad = [(4, 1, E), (7, 0, -1), (T - 1, 1, 1 << 20)]
    for t, j, v in bad:
        ids[t, j] = v
    x = torch.randn(T, 128).to(torch.bfloat16)
    g = _dispatch(C, cfg, x.cuda(), torch.from_numpy(ids).cuda())
    assert C.binding.moe_get_device_error(g["ws"]) == 1
    inv = g["inv"].cpu().numpy()
    assert all(inv[t * 2 + j] == -1 for t, j, _ in bad)
    assert g["offsets"].cpu().numpy()[-1] == 2 * T - len(bad)
    good = ids.copy()
    for t, j, _ in bad:
        good[t, j] = 0          # a valid id that the check below leaves out
    ref = O.dispatch_ref(good, 0, E)
    keep = np.ones(2 * T, bool)
    keep[[t * 2 + j for t, j, _ in bad]] = False
    # the valid pairs keep their order: perm lists them by (expert, pair index)
    want = ref["perm"][keep[ref["perm"]]]
    assert np.array_equal(g["perm"].cpu().numpy()[:2 * T - len(bad)], want)


def test_dispatch_empty_batch():
    C = _gpu()
    cfg = W.LayerConfig("empty", T=0, H=128, E=8, k=2, I=64, act="bf16", wdt="bf16")
    x = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    g = _dispatch(C, cfg, x, torch.empty(0, 2, dtype=torch.int32, device="cuda"))
    assert g["counts"].cpu().tolist() == [0] * 8 and g["offsets"].cpu().tolist() == [0] * 9


def _ffn(C, x_perm, I, offsets, E_loc, w13, w2, s13=None, s2=None, tile_m=0):
    B = C.binding
    cap = x_perm.shape[0]
    y = torch.full_like(x_perm, float("nan"))
    ws = torch.empty(max(B.moe_ffn_workspace_size(cap, I, B.dtype_code(x_perm)), 256), dtype=torch.uint8,
                     device="cuda")
    B.moe_grouped_ffn(x_perm, I, offsets, E_loc, w13, w2, y, ws, s13, s2, tile_m=tile_m)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("cid", CIDS)
@pytest.mark.parametrize("tile_m", [0, 32, 64, 128])
def test_grouped_ffn(cid, tile_m):
    C = _gpu()
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    if cfg.act == "f32" and tile_m not in (0, 32):
        pytest.skip("fp32 path has one tile shape")
    ids = O.moe_layer_expert(ov, tokens=np.arange(1))["ids"]
    ref = O.dispatch_ref(ids, cfg.expert_begin, cfg.expert_end)
    M = ref["M"]
    x_perm = inp["x"][torch.from_numpy(ref["perm"] // cfg.k).long()].contiguous()
    dev = lambda t: None if t is None else t.cuda()
    y = _ffn(C, x_perm.cuda(), cfg.I, torch.from_numpy(ref["offsets"]).cuda(), cfg.E_loc, dev(inp["w13"]),
             dev(inp["w2"]), dev(inp["w13_scale"]), dev(inp["w2_scale"]), tile_m)
    xp64 = O.decode(W.bits(x_perm), cfg.act)
    want, scale = O.grouped_ffn_ref(xp64, ref["offsets"], lambda e: O.expert_weights(ov, e), with_scale=True)
    print(f"ffn cfg={cfg.name} M={M} tile_m={tile_m}", flush=True)
    assert_close(to_f64(y[:M]), want, tol_for(cfg), f"y_perm {cfg.name}", scale)


def test_dense_shared_ffn():
    C = _gpu()
    inp, ov = inputs(2, True)
    from combine_dual_overlap_amd.device_layer import concat_shared
    w13, w2, shI = concat_shared(inp["shared_w13"], inp["shared_w2"])
    y = _ffn(C, inp["x"].cuda(), shI, None, 1, w13.cuda(), w2.cuda())
    x64 = O.decode(ov["x"], "bf16")
    parts = [O.swiglu_expert(x64, a, b, with_scale=True) for a, b in O.shared_weights(ov)]
    assert_close(to_f64(y), sum(p[0] for p in parts), 1e-2, "shared expert", sum(p[1] for p in parts))


# One column tile and several; an I that is not a multiple of 128.
@pytest.mark.parametrize("H,I", [(256, 128), (512, 384), (256, 192)])
def test_ffn_single_row_experts_and_gaps(H, I):
    C = _gpu()
    E = 6
    counts = np.array([1, 0, 33, 0, 129, 2])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    x = torch.randn(M, H).to(torch.bfloat16)
    w13 = (torch.randn(E, 2 * I, H) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn(E, H, I) * 0.05).to(torch.bfloat16)
    for tm in (32, 64, 128):
        y = _ffn(C, x.cuda(), I, torch.from_numpy(offsets).cuda(), E, w13.cuda(), w2.cuda(), tile_m=tm)
        want, scale = O.grouped_ffn_ref(
            O.decode(W.bits(x), "bf16"), offsets,
            lambda e: (O.decode(W.bits(w13[e]), "bf16"), O.decode(W.bits(w2[e]), "bf16")), with_scale=True)
        assert_close(to_f64(y), want, 1e-2, f"ragged experts tile_m={tm}", scale)


@pytest.mark.parametrize("cid", [2, 5])
def test_bf16_row_tiles_agree(cid):
    """bf16: the 64-row tiles (weights staged through registers) and the
    128-row tiles (weights staged by LDS DMA) add the same fp32 products in the
    same K order, so their outputs are equal bit for bit; the 32-row tiles start
    each weight tile at its own K stage, a different order, so they agree to a
    few units in the last place.  K = 1408 = 11 x 128 and a row count of 5
    exercise partial tiles."""
    C = _gpu()
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    ids = O.moe_layer_expert(ov, tokens=np.arange(1))["ids"]
    ref = O.dispatch_ref(ids, cfg.expert_begin, cfg.expert_end)
    x_perm = inp["x"][torch.from_numpy(ref["perm"] // cfg.k).long()].contiguous().cuda()
    off = torch.from_numpy(ref["offsets"]).cuda()

    def agree(ys, what):
        assert torch.equal(ys[1].view(torch.int16), ys[2].view(torch.int16)), what + ": 64 vs 128 rows"
        a, b = ys[0].float().cpu(), ys[1].float().cpu()
        scale = a.abs().max().item()
        assert torch.allclose(a, b, rtol=2.0 ** -6, atol=scale * 2.0 ** -9), what + ": 32 vs 64 rows"

    ys = [_ffn(C, x_perm, cfg.I, off, cfg.E_loc, inp["w13"].cuda(), inp["w2"].cuda(), tile_m=tm)[:ref["M"]]
          for tm in (32, 64, 128)]
    agree(ys, cfg.name)
    rng = torch.Generator().manual_seed(11)
    H, I, E = 2048, 1408, 3
    counts = np.array([5, 0, 221])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    x = torch.randn(M, H, generator=rng).to(torch.bfloat16).cuda()
    w13 = (torch.randn(E, 2 * I, H, generator=rng) * 0.02).to(torch.bfloat16).cuda()
    w2 = (torch.randn(E, H, I, generator=rng) * 0.02).to(torch.bfloat16).cuda()
    off = torch.from_numpy(offsets).cuda()
    ys = [_ffn(C, x, I, off, E, w13, w2, tile_m=tm) for tm in (32, 64, 128)]
    agree(ys, "H=2048 I=1408")


@pytest.mark.parametrize("cid", [3, 4])
def test_fp8_weight_row_tiles_agree(cid):
    """fp8 weights: the DMA-staged tiles of 64 and 128 rows of one launch
    (gate/up 2 x 2 waves; down 2 x 2 or 2 x 4 waves) and the automatic choice
    take the same arithmetic (block sums scaled with one fma each, or at
    prefill sizes one accumulator rescaled at every block) in the same K
    order, so their outputs are equal bit for bit.  (Each tile, and the register-staged 32-row tile that
    rounds the weights first, is checked against the oracle by
    test_grouped_ffn.)"""
    C = _gpu()
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    ids = O.moe_layer_expert(ov, tokens=np.arange(1))["ids"]
    ref = O.dispatch_ref(ids, cfg.expert_begin, cfg.expert_end)
    x_perm = inp["x"][torch.from_numpy(ref["perm"] // cfg.k).long()].contiguous().cuda()
    off = torch.from_numpy(ref["offsets"]).cuda()
    args = (cfg.I, off, cfg.E_loc, inp["w13"].cuda(), inp["w2"].cuda(), inp["w13_scale"].cuda(),
            inp["w2_scale"].cuda())
    y0, y64, y128 = (_ffn(C, x_perm, *args, tile_m=tm)[:ref["M"]] for tm in (0, 64, 128))
    assert torch.isfinite(y64.float()).all()
    assert torch.equal(y64.view(torch.int16), y128.view(torch.int16)), "64 vs 128 rows"
    assert torch.equal(y0.view(torch.int16), y128.view(torch.int16)), "automatic vs 128 rows"


def _fp8_experts(E, rows, cols, gen, zero_block_of=None, spread=4.0, zero_scales=False):
    """E expert matrices of block-quantised fp8 weights: N(0, 0.02) scaled by
    2^u, u ~ U(-spread, spread), per 128 x 128 block (so block scales differ),
    and one all-zero block in expert zero_block_of (the quantiser gives it
    scale 1).  zero_scales: about one block in four gets scale 0 while its
    codes stay as drawn (the block contributes nothing), and every scale of
    expert 3 is zero (row blocks with no nonzero scale at all)."""
    codes = torch.empty(E, rows, cols, dtype=torch.uint8)
    scales = torch.empty(E, rows // 128, cols // 128, dtype=torch.float32)
    for e in range(E):
        u = (torch.rand(rows // 128, cols // 128, generator=gen) * (2 * spread) - spread)
        f = torch.pow(2.0, u).repeat_interleave(128, 0).repeat_interleave(128, 1)
        w = torch.randn(rows, cols, generator=gen) * 0.02 * f
        if e == zero_block_of:
            w[:128, :128] = 0.0
        codes[e], scales[e] = W.quantize_fp8_blocks(w)
        if zero_scales:
            scales[e][torch.rand(rows // 128, cols // 128, generator=gen) < 0.25] = 0.0
            if e == 3:
                scales[e] = 0.0
    return codes, scales


def _fp8_ffn_vs_oracle(C, H, I, counts, tiles, seed, spread=4.0, zero_scales=False):
    gen = torch.Generator().manual_seed(seed)
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    x = torch.randn(M, H, generator=gen).to(torch.bfloat16)
    c13, s13 = _fp8_experts(E, 2 * I, H, gen, zero_block_of=min(2, E - 1), spread=spread, zero_scales=zero_scales)
    c2, s2 = _fp8_experts(E, H, I, gen, spread=spread, zero_scales=zero_scales)
    if zero_scales:
        assert (s13 == 0).any() and (s2 == 0).any() and (c13[s13.repeat_interleave(128, 1).repeat_interleave(
            128, 2) == 0] != 0).any()
    want, scale = O.grouped_ffn_ref(
        O.decode(W.bits(x), "bf16"), offsets,
        lambda e: (O.dequant_fp8_blocks(c13[e].numpy(), s13[e].numpy()),
                   O.dequant_fp8_blocks(c2[e].numpy(), s2[e].numpy())), with_scale=True)
    for tm in tiles:
        y = _ffn(C, x.cuda(), I, torch.from_numpy(offsets).cuda(), E, c13.cuda(), c2.cuda(), s13.cuda(), s2.cuda(),
                 tile_m=tm)
        print(f"fp8-weight ffn H={H} I={I} counts={list(counts)} tile_m={tm}", flush=True)
        assert_close(to_f64(y[:M]), want, 1e-2, f"fp8 weights H={H} I={I} tile_m={tm}", scale)


def test_fp8_weight_ffn_ragged_experts():
    """fp8 weights, bf16 activations, experts of 0, 1, 33, 64, 65, 128, 129 and
    257 rows: partial last row tiles, waves without rows, several row tiles;
    varied block scales and an all-zero weight block (scale 1)."""
    _fp8_ffn_vs_oracle(_gpu(), 256, 256, np.array([1, 0, 33, 64, 65, 128, 129, 257]), (32, 64, 128), 21)


@pytest.mark.parametrize("counts", [[1, 0, 33, 64, 65, 128, 129, 257], [0, 1, 127, 128, 129, 200, 257, 300]])
def test_fp8_weight_ffn_zero_and_wide_block_scales(counts):
    """Block scales spread over 2^-20 .. 2^20 and about a quarter of them
    zero (over nonzero codes), at about 85 rows per expert (block
    accumulator, one fma per block) and about 140 (full tiles: one
    accumulator kept in units of the current block's scale, zero-scale blocks
    masked); row tiles of 64 and 128 and the automatic choice."""
    _fp8_ffn_vs_oracle(_gpu(), 512, 256, np.array(counts), (0, 64, 128), 23, spread=20.0, zero_scales=True)


def test_fp8_weight_ffn_k_beyond_dma_scale_rows():
    """H = 8448 (66 scale blocks along K) is past the 64 K blocks the
    DMA-staged fp8 tile stages per scale row: the gate/up GEMM falls back to the
    register-staged fp8 tile, the down GEMM (K = I = 128) stays DMA-staged."""
    _fp8_ffn_vs_oracle(_gpu(), 8448, 128, np.array([3, 130]), (128,), 22)


@pytest.mark.parametrize("cid", CIDS)
def test_combine(cid):
    C = _gpu()
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    r = O.moe_layer_expert(ov, tokens=np.arange(1))
    ref = O.dispatch_ref(r["ids"], cfg.expert_begin, cfg.expert_end)
    M, T = ref["M"], cfg.T
    dt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    y = torch.randn(max(M, 1), cfg.H).to(dt)
    shared = torch.randn(T, cfg.H).to(dt) if cfg.n_shared else None
    w = torch.from_numpy(r["w"].astype(np.float32))
    out = torch.empty(T, cfg.H, dtype=dt, device="cuda")
    C.binding.moe_combine(y.cuda(), T, cfg.k, torch.from_numpy(ref["inv"]).cuda(), w.cuda(), out,
                          shared_out=None if shared is None else shared.cuda())
    torch.cuda.synchronize()
    want, scale = O.combine_ref(O.decode(W.bits(y), cfg.act), ref["inv"], w.double().numpy(),
                                None if shared is None else O.decode(W.bits(shared), cfg.act), with_scale=True)
    # only the fp32 sum and one final rounding: at most 2^-8 of |out| (bf16 has
    # an 8-bit significand), so 4e-3 leaves no room for any other error
    assert_close(to_f64(out), want, 4e-3 if cfg.act == "bf16" else 1e-6, f"combine {cfg.name}", scale)


def test_invalid_arguments_enqueue_nothing():
    C = _gpu()
    B = C.binding
    x = torch.randn(4, 128, device="cuda").to(torch.bfloat16)
    ids = torch.zeros(4, 2, dtype=torch.int32, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    t = lambda n: torch.empty(n, dtype=torch.int32, device="cuda")
    with pytest.raises(B.MoEError) as e:
        B.moe_dispatch(x, ids, 8, 0, 8, t(8), t(9), t(8), t(8), torch.empty(8, 128, device="cuda",
                       dtype=torch.bfloat16), small)
    assert e.value.status == B.MOE_ERR_WORKSPACE
    with pytest.raises(B.MoEError) as e:
        B.moe_dispatch(x, ids, 8, 3, 2, t(8), t(9), t(8), t(8), x, small)
    assert e.value.status == B.MOE_ERR_INVALID_ARG
