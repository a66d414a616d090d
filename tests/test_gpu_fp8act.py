"""GPU parity of the fp8-activation path against the CPU oracle: the row
quantisation (bit-exact codes and scale bytes), the quantising dispatch, the
fp8 x fp8 grouped FFN and the layer with fp8 activations."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from conftest import read_golden
from helpers import RMS_TOL_FP8_ACT, TOL as _TOL, assert_close, inputs, to_f64

pytestmark = pytest.mark.gpu

# fp8 weights and fp8 activations: the codes of x are exact on both sides; h
# is quantised from fp32 (GPU) and float64 (oracle) sums, so a code may land
# one step apart where h sits on a rounding boundary (each such flip moves one
# of I terms by at most 1/8 of its magnitude); y and out are rounded to bf16.
# Elementwise 5e-2 of A, output-relative 1e-2 (helpers).  The FFN test
# checks the h codes themselves and y from the GPU's own h at 1e-2.
TOL = _TOL["fp8_act"]
RTOL = RMS_TOL_FP8_ACT


def _B():
    import combine_dual_overlap_amd as C
    C.binding.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return C.binding


def _quant_gpu(B, x_bf16: torch.Tensor):
    n, K = x_bf16.shape
    q = torch.full((n, K), 0xAA, dtype=torch.uint8, device="cuda")
    s = torch.full((n, K // 128), 0xAA, dtype=torch.uint8, device="cuda")
    B.moe_quant_fp8_rows(x_bf16.cuda(), q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def _check_quant(x_bf16: torch.Tensor, q, s, what):
    codes, e = O.quant_rows_fp8(O.decode(W.bits(x_bf16), "bf16"))
    assert np.array_equal(s.astype(np.int64), e + 127), f"{what}: scale bytes"
    bad = np.nonzero(q != codes)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}: "
                              f"gpu {q[bad][0]:#x} oracle {codes[bad][0]:#x}")


def test_quant_rows_golden_bitwise():
    B = _B()
    g = read_golden("fp8_act_quant_handcalc.txt")
    x = torch.zeros(2, 256)
    for key, vals in g.items():
        if key.startswith("x."):
            _, r, c = key.split(".")
            x[int(r), int(c)] = float(vals[0])
    xb = x.to(torch.bfloat16)
    q, s = _quant_gpu(B, xb)
    _check_quant(xb, q, s, "golden rows")
    for key, vals in g.items():
        kind, r, c = key.split(".")
        if kind == "code":
            assert q[int(r), int(c)] == int(vals[0], 16), key


@pytest.mark.parametrize("n,K", [(1, 128), (37, 512), (300, 2048), (64, 7168)])
def test_quant_rows_random_bitwise(n, K):
    B = _B()
    g = torch.Generator().manual_seed(n * 7 + K)
    mag = torch.pow(2.0, torch.randint(-40, 40, (n, K // 128, 1), generator=g).float())
    x = (torch.randn(n, K // 128, 128, generator=g) * mag).reshape(n, K)
    x[0, :128] = 0.0                                      # all-zero group
    if n > 3:
        x[3, :] = torch.randn(K, generator=g) * 1e-38     # subnormal bf16 values
        x[2, :128] = 448.0 * 2.0 ** -5                    # amax exactly on a bound
    xb = x.to(torch.bfloat16)
    print(f"quant n={n} K={K}", flush=True)
    q, s = _quant_gpu(B, xb)
    _check_quant(xb, q, s, f"n={n} K={K}")


def test_quant_rows_every_tie():
    """Rows of one 128-column group each: 1.75 = 448 * 2^-8 first (fixing
    e = -8), then the midpoints between consecutive positive codes and the
    codes themselves, scaled by 2^-8, with both signs."""
    B = _B()
    pos = O.FP8_E4M3FN_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([mids, -mids, pos, -pos]) * 2.0 ** -8
    n = -(-vals.size // 127)
    rows = np.zeros((n, 128))
    rows[:, 0] = 1.75
    rows[:, 1:].flat[:vals.size] = vals
    xb = torch.from_numpy(rows).float().to(torch.bfloat16)
    assert np.array_equal(O.decode(W.bits(xb), "bf16"), rows)     # bf16 holds every one of them
    q, s = _quant_gpu(B, xb)
    assert (s == 127 - 8).all()
    _check_quant(xb, q, s, "ties")


@pytest.mark.parametrize("cid", [3, 4])
def test_dispatch_fp8_matches_oracle(cid):
    B = _B()
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    ids = O.moe_layer_expert(ov, tokens=np.arange(1))["ids"].astype(np.int32)
    ref = O.dispatch_ref(ids, cfg.expert_begin, cfg.expert_end)
    T, k, E_loc = cfg.T, cfg.k, cfg.E_loc
    x = inp["x"].cuda()
    counts = torch.empty(E_loc, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E_loc + 1, dtype=torch.int32, device="cuda")
    perm = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    xq = torch.zeros(T * k, cfg.H, dtype=torch.uint8, device="cuda")
    xs = torch.zeros(T * k, cfg.H // 128, dtype=torch.uint8, device="cuda")
    ws = torch.empty(B.moe_dispatch_workspace_size(T, k, E_loc), dtype=torch.uint8, device="cuda")
    B.moe_dispatch_fp8(x, torch.from_numpy(ids).cuda(), cfg.E, cfg.expert_begin, cfg.expert_end, counts, offsets,
                       perm, inv, xq, xs, ws)
    torch.cuda.synchronize()
    M = ref["M"]
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(inv.cpu().numpy(), ref["inv"])
    assert np.array_equal(perm.cpu().numpy()[:M], ref["perm"][:M])
    rows = O.decode(W.bits(inp["x"]), "bf16")[ref["perm"][:M] // k]
    codes, e = O.quant_rows_fp8(rows)
    assert np.array_equal(xq.cpu().numpy()[:M], codes)
    assert np.array_equal(xs.cpu().numpy()[:M].astype(np.int64), e + 127)


# The quantising gather on each dispatch path: one workgroup (small), the
# rank folded into the gather (groups of 16 tokens, the last one partial, with
# k = 6 a group's pairs straddling the 1024-pair count blocks), and the
# separate count, scan and rank kernels (more than 256 local experts).
@pytest.mark.parametrize("T,k,E,lo,hi", [(200, 6, 64, 0, 64), (1001, 6, 64, 0, 64), (3001, 8, 256, 32, 96),
                                         (700, 4, 300, 0, 257)])
def test_dispatch_fp8_shapes(T, k, E, lo, hi):
    B = _B()
    rng = np.random.default_rng(T * 7 + k)
    H = 256
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = (torch.randn(T, H) * torch.exp2(torch.randint(-6, 7, (T, 1)).float())).to(torch.bfloat16)
    ref = O.dispatch_ref(ids, lo, hi)
    E_loc, M = hi - lo, ref["M"]
    i32 = lambda n: torch.full((n,), -7, dtype=torch.int32, device="cuda")
    counts, offsets, perm, inv = i32(E_loc), i32(E_loc + 1), i32(T * k), i32(T * k)
    xq = torch.zeros(T * k, H, dtype=torch.uint8, device="cuda")
    xs = torch.zeros(T * k, H // 128, dtype=torch.uint8, device="cuda")
    ws = torch.empty(B.moe_dispatch_workspace_size(T, k, E_loc), dtype=torch.uint8, device="cuda")
    print(f"fp8 dispatch T={T} k={k} E={E} local [{lo}, {hi})", flush=True)
    B.moe_dispatch_fp8(x.cuda(), torch.from_numpy(ids).cuda(), E, lo, hi, counts, offsets, perm, inv, xq, xs, ws)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(perm.cpu().numpy()[:M], ref["perm"])
    assert np.array_equal(inv.cpu().numpy(), ref["inv"])
    codes, e = O.quant_rows_fp8(O.decode(W.bits(x), "bf16")[ref["perm"] // k])
    assert np.array_equal(xq.cpu().numpy()[:M], codes)
    assert np.array_equal(xs.cpu().numpy()[:M].astype(np.int64), e + 127)


def test_dispatch_send_recv_fp8_equals_one_call():
    B = _B()
    inp, ov = inputs(3, True)
    cfg = inp["cfg"]
    ids = torch.from_numpy(O.moe_layer_expert(ov, tokens=np.arange(1))["ids"].astype(np.int32)).cuda()
    T, k, E_loc = cfg.T, cfg.k, cfg.E_loc
    x = inp["x"].cuda()
    outs = []
    for two_phase in (False, True):
        i32 = lambda n: torch.full((n,), -7, dtype=torch.int32, device="cuda")
        counts, offsets, perm, inv = i32(E_loc), i32(E_loc + 1), i32(T * k), i32(T * k)
        xq = torch.zeros(T * k, cfg.H, dtype=torch.uint8, device="cuda")
        xs = torch.zeros(T * k, cfg.H // 128, dtype=torch.uint8, device="cuda")
        ws = torch.empty(B.moe_dispatch_workspace_size(T, k, E_loc), dtype=torch.uint8, device="cuda")
        if two_phase:
            B.moe_dispatch_send(ids, cfg.E, cfg.expert_begin, cfg.expert_end, counts, offsets, perm, inv, ws)
            B.moe_dispatch_recv(x, k, inv, xq, xq_scale=xs)
        else:
            B.moe_dispatch_fp8(x, ids, cfg.E, cfg.expert_begin, cfg.expert_end, counts, offsets, perm, inv, xq,
                               xs, ws)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (counts, offsets, perm, inv, xq, xs)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def _ffn_fp8(B, xq, xs, I, offsets, E_loc, w13, w2, s13, s2, tile_m=0, with_h=False):
    cap, H = xq.shape
    y = torch.full((cap, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(B.moe_ffn_fp8_workspace_size(cap, I), 256), dtype=torch.uint8, device="cuda")
    B.moe_grouped_ffn_fp8(xq, xs, I, offsets, E_loc, w13, w2, s13, s2, y, ws, tile_m=tile_m)
    torch.cuda.synchronize()
    if not with_h:
        return y
    # the workspace holds h: codes [cap, I], then (256-byte aligned) E8M0 bytes [cap, I/128]
    w = ws.cpu().numpy()
    hq = w[:cap * I].reshape(cap, I)
    off = -(-cap * I // 256) * 256
    hs = w[off:off + cap * (I // 128)].reshape(cap, I // 128)
    return y, hq, hs


_POS = O.FP8_E4M3FN_TABLE[:0x7F]          # magnitudes of codes 0x00..0x7E, increasing


def _check_h_decisions(hq, hs, h64, dh, what):
    """The GPU's h codes and scale bytes against the oracle's float64 h, given
    dh, a bound on |h_gpu - h| from the fp32 arithmetic: the group exponent
    may differ only where the group's amax lies within the group's largest dh
    of a bound 448 * 2^e; a code may differ from the oracle's rounding of h
    only if it is a correct rounding of some value within dh of h, i.e. its
    value lies within dh plus half a code step of h (scaled by 2^-e).
    Returns the number of codes that differ."""
    n, I = h64.shape
    codes, e = O.quant_rows_fp8(h64)
    e_gpu = hs.astype(np.int64) - 127
    amax = np.abs(h64.reshape(n, I // 128, 128)).max(axis=2)
    dmax = dh.reshape(n, I // 128, 128).max(axis=2)
    near_bound = (np.abs(amax - 448.0 * np.ldexp(1.0, e)) <= dmax) | \
                 (np.abs(amax - 448.0 * np.ldexp(1.0, e - 1)) <= dmax)
    bad_e = (e_gpu != e) & ~near_bound
    assert not bad_e.any(), f"{what}: {bad_e.sum()} h group exponents differ away from a bound"
    same_e = np.repeat(e_gpu == e, 128, axis=1)
    inv = np.ldexp(1.0, -np.repeat(e, 128, axis=1))
    a = h64 * inv                                            # the oracle's h in code units
    mag = (hq & 0x7F).astype(np.int64)
    v = np.where(hq & 0x80, -1.0, 1.0) * _POS[np.minimum(mag, 0x7E)]
    half = 0.5 * np.maximum(_POS[np.minimum(mag + 1, 0x7E)] - _POS[np.minimum(mag, 0x7E)],
                            _POS[np.minimum(mag, 0x7E)] - _POS[np.maximum(mag - 1, 0)])
    diff = (hq != codes) & same_e
    ok = ~diff | ((mag <= 0x7E) & (np.abs(v - a) <= dh * inv + half))
    if not ok.all():
        r, c = np.nonzero(~ok)
        det = "; ".join(f"({r[i]},{c[i]}) gpu {hq[r[i], c[i]]:#04x} oracle {codes[r[i], c[i]]:#04x} "
                        f"h {h64[r[i], c[i]]:.9g} scaled {a[r[i], c[i]]:.9g} "
                        f"dh {dh[r[i], c[i]] * inv[r[i], c[i]]:.3g} e {e[r[i], c[i] // 128]}"
                        for i in range(min(6, r.size)))
        raise AssertionError(f"{what}: {int((~ok).sum())} h codes are no rounding of h within its error "
                             f"bound: {det}")
    return int(diff.sum())


def _h_and_bound(xq, w13, I):
    """float64 h = silu(g) * u of the fp8 expert and a bound on the error of
    the same h computed in fp32: |dg| <= K 2^-23 sum_k |x_k w_k| (a dot
    product's rounding bound, doubled for the block-scale products), same for
    u, then dh = |silu'(g) u| dg + |silu(g)| du + 4 ulp of h."""
    K = xq.shape[1]
    g, u = xq @ w13[:I].T, xq @ w13[I:].T
    dg = K * 2.0 ** -23 * (np.abs(xq) @ np.abs(w13[:I]).T)
    du = K * 2.0 ** -23 * (np.abs(xq) @ np.abs(w13[I:]).T)
    sg = 1.0 / (1.0 + np.exp(-g))
    h = g * sg * u
    dh = np.abs(sg * (1.0 + g * (1.0 - sg)) * u) * dg + np.abs(g * sg) * du + 4 * 2.0 ** -24 * np.abs(h)
    return h, dh


@pytest.mark.parametrize("cid", [3, 4])
@pytest.mark.parametrize("tile_m", [0, 64, 128])
def test_grouped_ffn_fp8_matches_oracle(cid, tile_m):
    B = _B()
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    ids = O.moe_layer_expert(ov, tokens=np.arange(1))["ids"]
    ref = O.dispatch_ref(ids, cfg.expert_begin, cfg.expert_end)
    M = ref["M"]
    x_perm = inp["x"][torch.from_numpy(ref["perm"][:M] // cfg.k).long()].contiguous()
    xq = torch.empty(M, cfg.H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, cfg.H // 128, dtype=torch.uint8, device="cuda")
    B.moe_quant_fp8_rows(x_perm.cuda(), xq, xs)
    y, hq, hs = _ffn_fp8(B, xq, xs, cfg.I, torch.from_numpy(ref["offsets"]).cuda(), cfg.E_loc,
                         inp["w13"].cuda(), inp["w2"].cuda(), inp["w13_scale"].cuda(), inp["w2_scale"].cuda(),
                         tile_m, with_h=True)
    xp64 = O.decode(W.bits(x_perm), "bf16")
    print(f"ffn fp8 cfg={cfg.name} M={M} tile_m={tile_m}", flush=True)
    want, scale = O.grouped_ffn_fp8act_ref(xp64, ref["offsets"], lambda e: O.expert_weights(ov, e),
                                           with_scale=True)
    assert_close(to_f64(y), want, TOL, f"y_perm fp8-act {cfg.name}", scale, rms_tol=RTOL)
    # the h decisions, then y from the GPU's own h at the bf16 tolerance
    xq64 = O.fp8_roundtrip_rows(xp64)
    h64 = np.zeros((M, cfg.I))
    dh = np.zeros((M, cfg.I))
    y_h = np.zeros((M, cfg.H))
    s_h = np.zeros((M, cfg.H))
    hg = O.dequant_rows_fp8(hq[:M], hs[:M].astype(np.int64) - 127)
    offs = ref["offsets"]
    for e in range(cfg.E_loc):
        a, b = int(offs[e]), int(offs[e + 1])
        if b > a:
            w13, w2 = O.expert_weights(ov, e)
            h64[a:b], dh[a:b] = _h_and_bound(xq64[a:b], w13, cfg.I)
            y_h[a:b] = hg[a:b] @ w2.T
            s_h[a:b] = np.abs(hg[a:b]) @ np.abs(w2).T
    flips = _check_h_decisions(hq[:M], hs[:M], h64, dh, f"h fp8-act {cfg.name}")
    print(f"  h codes: {flips} of {hq[:M].size} differ from the oracle's, each within the fp32 error bound")
    assert_close(to_f64(y), y_h, _TOL["fp8"], f"y_perm from the GPU's h {cfg.name}", s_h)


def test_grouped_ffn_fp8_ragged_experts():
    """Experts of 0, 1, 63, 64, 65 and 200 rows (partial and empty row tiles)."""
    B = _B()
    g = torch.Generator().manual_seed(11)
    H, I = 512, 384
    counts = np.array([1, 0, 63, 64, 0, 65, 200, 2])
    E = counts.size
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    x = torch.randn(M, H, generator=g).to(torch.bfloat16)
    w13c, s13 = zip(*[W.quantize_fp8_blocks(torch.randn(2 * I, H, generator=g) * 0.05) for _ in range(E)])
    w2c, s2 = zip(*[W.quantize_fp8_blocks(torch.randn(H, I, generator=g) * 0.05) for _ in range(E)])
    w13c, s13, w2c, s2 = (torch.stack(t).contiguous() for t in (w13c, s13, w2c, s2))
    xq = torch.empty(M, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, H // 128, dtype=torch.uint8, device="cuda")
    B.moe_quant_fp8_rows(x.cuda(), xq, xs)
    wof = lambda e: (O.dequant_fp8_blocks(w13c[e].numpy(), s13[e].numpy()),
                     O.dequant_fp8_blocks(w2c[e].numpy(), s2[e].numpy()))
    want, scale = O.grouped_ffn_fp8act_ref(O.decode(W.bits(x), "bf16"), offsets, wof, with_scale=True)
    for tm in (64, 128):
        y = _ffn_fp8(B, xq, xs, I, torch.from_numpy(offsets).cuda(), E, w13c.cuda(), w2c.cuda(), s13.cuda(),
                     s2.cuda(), tm)
        assert_close(to_f64(y), want, TOL, f"ragged fp8-act tile_m={tm}", scale, rms_tol=RTOL)


def test_grouped_ffn_fp8_long_k_register_ring_kernel():
    """K > 4096 in both GEMMs (H = 4352, I = 4224): the register-ring staging
    runs instead of the LDS-DMA one, for both row tiles."""
    B = _B()
    g = torch.Generator().manual_seed(12)
    H, I = 4352, 4224
    counts = np.array([3, 70])
    E = counts.size
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    x = torch.randn(M, H, generator=g).to(torch.bfloat16)
    w13c, s13 = zip(*[W.quantize_fp8_blocks(torch.randn(2 * I, H, generator=g) * 0.02) for _ in range(E)])
    w2c, s2 = zip(*[W.quantize_fp8_blocks(torch.randn(H, I, generator=g) * 0.02) for _ in range(E)])
    w13c, s13, w2c, s2 = (torch.stack(t).contiguous() for t in (w13c, s13, w2c, s2))
    xq = torch.empty(M, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, H // 128, dtype=torch.uint8, device="cuda")
    B.moe_quant_fp8_rows(x.cuda(), xq, xs)
    wof = lambda e: (O.dequant_fp8_blocks(w13c[e].numpy(), s13[e].numpy()),
                     O.dequant_fp8_blocks(w2c[e].numpy(), s2[e].numpy()))
    want, scale = O.grouped_ffn_fp8act_ref(O.decode(W.bits(x), "bf16"), offsets, wof, with_scale=True)
    for tm in (64, 128):
        y = _ffn_fp8(B, xq, xs, I, torch.from_numpy(offsets).cuda(), E, w13c.cuda(), w2c.cuda(), s13.cuda(),
                     s2.cuda(), tm)
        assert_close(to_f64(y), want, TOL, f"long K fp8-act tile_m={tm}", scale, rms_tol=RTOL)


def test_grouped_ffn_fp8_rejects_bad_shapes():
    B = _B()
    d = lambda *s: torch.zeros(*s, dtype=torch.uint8, device="cuda")
    f = lambda *s: torch.ones(*s, dtype=torch.float32, device="cuda")
    offs = torch.zeros(2, dtype=torch.int32, device="cuda")
    y = torch.zeros(4, 384, dtype=torch.bfloat16, device="cuda")
    ws = d(1 << 16)
    with pytest.raises(B.MoEError) as e:   # H = 384 is not a multiple of 256
        B.moe_grouped_ffn_fp8(d(4, 384), d(4, 3), 128, offs, 1, d(1, 256, 384), d(1, 384, 128), f(1, 2, 3),
                              f(1, 3, 1), y, ws)
    assert e.value.status == B.MOE_ERR_UNSUPPORTED
    y = torch.zeros(4, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoEError) as e:   # 32-row tiles are not offered
        B.moe_grouped_ffn_fp8(d(4, 256), d(4, 2), 128, offs, 1, d(1, 256, 256), d(1, 256, 128), f(1, 2, 2),
                              f(1, 2, 1), y, ws, tile_m=32)
    assert e.value.status == B.MOE_ERR_UNSUPPORTED


def _layer8(inp):
    import combine_dual_overlap_amd as C
    _B()
    return C.DeviceLayer(inp, fp8_act=True)


def _gpu_ids(L, cfg, T0):
    halves = [(0, T0), (T0, cfg.T)]
    return np.vstack([L.view(mb, "topk_ids", torch.int32, (b - a, cfg.k)).cpu().numpy()
                      for mb, (a, b) in enumerate(halves)])


@pytest.mark.parametrize("cid", [3, 4])
@pytest.mark.parametrize("schedule", ["serial", "dbo", "dbo_recv_hook"])
def test_layer_fp8act_small(cid, schedule):
    inp, ov = inputs(cid, True)
    cfg = inp["cfg"]
    L = _layer8(inp)
    print(f"layer fp8-act cfg={cfg.name} schedule={schedule}", flush=True)
    out = L.run(schedule)
    torch.cuda.synchronize()
    T0 = (cfg.T + 1) // 2
    ids = _gpu_ids(L, cfg, T0)
    ref = O.moe_layer_expert(dict(ov, fp8_act=True, forced_ids=ids.astype(np.int32)))
    assert_close(to_f64(out), ref["out"], TOL, f"out fp8-act {cfg.name} {schedule}", ref["scale"], rms_tol=RTOL)


@pytest.mark.parametrize("cid", [3, 4])
def test_layer_fp8act_dbo_equals_serial_bitwise(cid):
    inp, _ = inputs(cid, True)
    L = _layer8(inp)
    base = L.run("serial").clone()
    for _ in range(5):
        out = L.run("dbo")
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), base.view(torch.int16))


@pytest.mark.parametrize("cid", [3, 4])
def test_layer_fp8act_full_size_sampled(cid):
    inp, ov = inputs(cid, False)
    cfg = inp["cfg"]
    L = _layer8(inp)
    print(f"full layer fp8-act cfg={cfg.name} T={cfg.T}", flush=True)
    out = L.run("dbo")
    torch.cuda.synchronize()
    T0 = (cfg.T + 1) // 2
    ids = _gpu_ids(L, cfg, T0)
    rng = np.random.default_rng(100 + cid)
    sample = np.unique(np.concatenate([[0, T0 - 1, T0, cfg.T - 1], rng.integers(0, cfg.T, 12)]))
    ref = O.moe_layer_expert(dict(ov, fp8_act=True, forced_ids=ids.astype(np.int32)), tokens=sample)
    assert_close(to_f64(out[torch.from_numpy(sample).cuda()]), ref["out"], TOL, f"out fp8-act {cfg.name}",
                 ref["scale"], rms_tol=RTOL)
