"""Shared helpers of the GPU parity tests: tolerance rule, oracle/GPU glue,
cached workloads."""
import functools

import numpy as np
import torch

import oracle as O
from oracle.routing import route_cfg
import workloads as W

# Tolerances of the floating-point outputs: |gpu - ref| <= tol * (|ref| + rms(ref)).
# bf16 / fp8-weight values are the ones the layer's statement fixes (1e-2 and
# 5e-2); the rms term keeps elements near zero from demanding a relative
# accuracy no bf16 rounding can give.  fp32 (tiny config): 1e-4.
TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 5e-2}


def tol_for(cfg) -> float:
    if cfg.act == "f32":
        return TOL["f32"]
    return TOL["fp8"] if cfg.wdt == "fp8" else TOL["bf16"]


def assert_close(gpu, ref, tol, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(gpu - ref)
    bound = tol * (np.abs(ref) + rms)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / (bound + 1e-300)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} outside tol {tol}; worst at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r} (rms {rms:.3g}, max abs err {err.max():.3g})")
    return float(err.max()) if err.size else 0.0


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


@functools.lru_cache(maxsize=None)
def inputs(cid: int, small: bool, seed: int = 0):
    cfg = W.get_config(cid, small=small)
    inp = W.make_inputs(cfg, seed)
    return inp, W.oracle_view(inp)


def oracle_ids_from_logits(gpu_logits: np.ndarray, cfg, forced=None):
    """The oracle's selection and weights applied to the logits the GPU compared."""
    return route_cfg(np.asarray(gpu_logits, np.float64), cfg, forced)


def grouped_margins(logits: np.ndarray, cfg):
    """Per token: smallest f64 gap around the group cut and the expert cut of
    group-limited sigmoid routing (where float rounding could flip a choice)."""
    s = O.sigmoid(np.asarray(logits, np.float64))
    T, E = s.shape
    G, per = cfg.n_groups, E // cfg.n_groups
    g = np.sort(s.reshape(T, G, per), axis=2)[:, :, per - cfg.group_topn:].sum(2)
    gs = -np.sort(-g, axis=1)
    gm = gs[:, cfg.topk_groups - 1] - gs[:, cfg.topk_groups]
    return gm


def check_ids(gpu_ids, gpu_logits, cfg, forced=None, what="ids"):
    """GPU ids must equal the oracle's selection on the GPU's own logits; for
    group-limited routing a row may differ only where the f64 group margin is
    below 2^-20 (either choice is correct there)."""
    ref_ids, ref_w = oracle_ids_from_logits(gpu_logits, cfg, forced)
    gpu_ids = np.asarray(gpu_ids)
    diff = (gpu_ids != ref_ids).any(1)
    if diff.any():
        assert cfg.score == "sigmoid" and cfg.n_groups > 1, f"{what}: {diff.sum()} rows differ"
        m = grouped_margins(gpu_logits, cfg)
        assert (m[diff] < 2.0 ** -20).all(), f"{what}: rows differ away from a near-tie"
    return ref_ids, ref_w, diff
