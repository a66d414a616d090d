"""The parity rule itself (CPU): the two checks of helpers.assert_close must
accept a correct implementation that rounds as the GPU path does, and must
reject the plausible mistakes a kernel could make.  Every mistake is planted
in a copy of the oracle's computation, on the CPU.

Correct-but-rounded: the layer computed from the oracle's own routing and
expert weights with the GPU path's roundings written out (fp8 weight value
times its block scale rounded to bf16, h, y and out rounded to bf16).

Planted mistakes (each must fail the committed check):
  * the whole output 10 % too large;
  * fp8 block scales read one K block off, only the first K block's scale,
    one mean scale per matrix (block-scale indexing bugs);
  * the last slot of every token dropped;
  * gate and up swapped in SwiGLU.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import assert_close, tol_for


def _bf16(a: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (via float32, round to nearest even) -> float64."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float64)).float().to(torch.bfloat16).double().numpy()


def _layer(ov, ids, w, weights_of, rnd=lambda a: a, swap=False, drop_last=False):
    """out[t] = sum_j w[t, j] * SwiGLU_e(x[t]) over local slots (+ shared),
    with rnd applied to h, y and out as the GPU rounds them."""
    cfg = ov["cfg"]
    x = O.decode(ov["x"], ov["act"])
    out = np.zeros((x.shape[0], cfg.H))
    k_used = cfg.k - 1 if drop_last else cfg.k
    for el in range(cfg.E_loc):
        rows, slots = np.nonzero(ids[:, :k_used] == el + cfg.expert_begin)
        if rows.size == 0:
            continue
        w13, w2 = weights_of(el)
        I = w13.shape[0] // 2
        g, u = x[rows] @ w13[:I].T, x[rows] @ w13[I:].T
        if swap:
            g, u = u, g
        y = rnd(rnd(O.silu(g) * u) @ w2.T)
        np.add.at(out, rows, w[rows, slots][:, None] * y)
    for w13, w2 in O.shared_weights(ov):
        I = w13.shape[0] // 2
        out += rnd(rnd(O.silu(x @ w13[:I].T) * (x @ w13[I:].T)) @ w2.T)
    return rnd(out)


def _fp8_weights(ov, s13, s2):
    return lambda e: (O.dequant_fp8_blocks(ov["w13"][e], s13[e]), O.dequant_fp8_blocks(ov["w2"][e], s2[e]))


def _cases(cid):
    cfg = W.get_config(cid, small=True)
    ov = W.oracle_view(W.make_inputs(cfg))
    ref = O.moe_layer_expert(ov)
    ids, w = ref["ids"], ref["w"]
    exact = lambda e: O.expert_weights(ov, e)
    out = {"x1.10": ref["out"] * 1.10,
           "drop last slot": _layer(ov, ids, w, exact, drop_last=True),
           "gate/up swapped": _layer(ov, ids, w, exact, swap=True)}
    if cfg.wdt == "fp8":
        s13, s2 = ov["w13_scale"], ov["w2_scale"]
        out["scale K block + 1"] = _layer(ov, ids, w, _fp8_weights(ov, np.roll(s13, -1, axis=2),
                                                                  np.roll(s2, -1, axis=2)))
        out["first K block scale only"] = _layer(ov, ids, w, _fp8_weights(
            ov, np.broadcast_to(s13[:, :, :1], s13.shape), np.broadcast_to(s2[:, :, :1], s2.shape)))
        out["one mean scale"] = _layer(ov, ids, w, _fp8_weights(
            ov, np.broadcast_to(s13.mean(axis=(1, 2), keepdims=True), s13.shape),
            np.broadcast_to(s2.mean(axis=(1, 2), keepdims=True), s2.shape)))
        rounded_w = lambda e: tuple(_bf16(m) for m in exact(e))
    else:
        rounded_w = exact
    emulated = _layer(ov, ids, w, rounded_w, rnd=_bf16)
    return cfg, ref, emulated, out


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_rule_accepts_gpu_roundings_and_rejects_planted_mistakes(cid):
    cfg, ref, emulated, mutants = _cases(cid)
    tol = tol_for(cfg)
    worst = assert_close(emulated, ref["out"], tol, f"{cfg.name} bf16 roundings", ref["scale"])
    # strict first-order bound of the roundings: at most 2^-8 of A each (bf16
    # has an 8-bit significand; h, y, out, and the fp8 weights one more)
    n_round = 4 if cfg.wdt == "fp8" else 3
    assert worst <= n_round * 2.0 ** -8, "the correct arithmetic exceeds its derived error bound"
    for name, got in mutants.items():
        with pytest.raises(AssertionError):
            assert_close(got, ref["out"], tol, f"{cfg.name} planted: {name}", ref["scale"])


def test_fp8_block_scales_differ_across_blocks():
    """The fp8 workloads draw each 128x128 block at its own magnitude, so
    block scales of one matrix spread over about a factor 2^8."""
    for cid in (3, 4):
        inp = W.make_inputs(W.get_config(cid, small=True))
        for s in (inp["w13_scale"], inp["w2_scale"]):
            r = (s.amax(dim=(1, 2)) / s.amin(dim=(1, 2))).log2()
            assert float(r.min()) > 3.0, (cid, r)


@pytest.mark.parametrize("cid", [3, 4])
def test_rule_with_fp8_activations_rejects_planted_mistakes(cid):
    """fp8 activations: elementwise 5e-2 of A, output-relative 1e-2.  The
    correct output rounded to bf16 passes; a 10 % error and the block-scale
    indexing mistakes fail."""
    from helpers import rms_tol_for
    cfg = W.get_config(cid, small=True)
    ov = dict(W.oracle_view(W.make_inputs(cfg)), fp8_act=True)
    ref = O.moe_layer_expert(ov)
    tol, rtol = tol_for(cfg, fp8_act=True), rms_tol_for(cfg, fp8_act=True)
    assert_close(_bf16(ref["out"]), ref["out"], tol, f"{cfg.name} fp8-act, out rounded", ref["scale"], rms_tol=rtol)
    s13, s2 = ov["w13_scale"], ov["w2_scale"]
    mutants = {
        "x1.10": ref["out"] * 1.10,
        "scale K block + 1": O.moe_layer_expert(dict(ov, w13_scale=np.roll(s13, -1, axis=2),
                                                     w2_scale=np.roll(s2, -1, axis=2)))["out"],
        "first K block scale only": O.moe_layer_expert(dict(
            ov, w13_scale=np.ascontiguousarray(np.broadcast_to(s13[:, :, :1], s13.shape)),
            w2_scale=np.ascontiguousarray(np.broadcast_to(s2[:, :, :1], s2.shape))))["out"],
    }
    for name, got in mutants.items():
        with pytest.raises(AssertionError):
            assert_close(got, ref["out"], tol, f"{cfg.name} fp8-act planted: {name}", ref["scale"], rms_tol=rtol)
