"""Shared helpers of the GPU parity tests: tolerance rule, oracle/GPU glue,
cached workloads."""
import functools
import os

import numpy as np
import torch

import oracle as O
from oracle.routing import route_cfg
import workloads as W

# Tolerances of the floating-point outputs.  Two checks, both must hold:
#  * elementwise, relative to the magnitude of what each element sums:
#    |gpu - ref| <= tol * (A + rms(A)/100), with A the oracle's per-element sum
#    of |terms| (for the layer: sum_j |w_j| (|h_j| |W2|^T), plus the shared
#    experts).  bf16 keeps an 8-bit significand, so one rounding errs by at
#    most u = 2^-8 relative.  The GPU rounds h, y_perm and out once each; the
#    register-staged fp8 tiles (32-row tiles, launches with a dense group)
#    round each weight once more (code value times its block scale, to bf16),
#    the DMA-staged ones never do.  The y_perm and out roundings contribute at
#    most u * A each; the h and weight roundings enter through sums over the
#    intermediate (or K) dimension whose errors have independent signs
#    (about u * A / sqrt(I)).  So about 2u * A = 0.8 % of A, and tol = 1e-2
#    holds for bf16 and fp8 weights alike, even where the weighted expert
#    outputs cancel (the strict worst case, every rounding aligned, would be
#    3u-4u * A);
#  * over the whole output, relative to the output:
#    ||gpu - ref||_2 <= tol * ||ref||_2 (the "rel" reading of the layer's
#    statement).  Independent roundings of relative size <= 2^-8 give a
#    relative RMS error near 2^-8 / sqrt(3) per rounding, about 0.2 %.
# The layer's statement allows 1e-2 (bf16) and 5e-2 (fp8 weights); both
# checks use 1e-2 for fp8 weights too, which the bound above supports.
# fp32 (tiny config): 1e-4.  Without a scale the elementwise rule falls back
# to tol * (|ref| + rms(ref)).
# fp8 activations: h is itself quantised to fp8, a decision that fp32 (GPU)
# and float64 (oracle) sums can take one code apart where h sits on a
# rounding boundary; one such flip moves one term by an fp8 step (1/16 to
# 1/8 of it), which is a few % of A where that term dominates (measured up to
# 2.7 % of A on the Qwen3-shaped layer).  The elementwise check then takes
# the statement's fp8 figure, 5e-2, while the output-relative check stays at
# 1e-2; the FFN test also checks the h codes themselves against the oracle.
TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 1e-2, "fp8_act": 5e-2}
RMS_TOL_FP8_ACT = 1e-2


def tol_for(cfg, fp8_act: bool = False) -> float:
    if cfg.act == "f32":
        return TOL["f32"]
    if fp8_act:
        return TOL["fp8_act"]
    return TOL["fp8"] if cfg.wdt == "fp8" else TOL["bf16"]


def rms_tol_for(cfg, fp8_act: bool = False) -> float:
    return RMS_TOL_FP8_ACT if fp8_act else tol_for(cfg)


# Margins of every passing check of this session, printed at the end of the
# run (tests/conftest.py): (test, what, worst err/A over tol, rel RMS over its tol).
MARGINS = []


def _margin_log(line: str):
    """Appends a parity margin line to $PARITY_LOG (if set)."""
    path = os.environ.get("PARITY_LOG")
    if path:
        test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(f"{test} | {line}\n")


def assert_close(gpu, ref, tol, what="", scale=None, rms_tol=None):
    """Both parity checks (see above).  rms_tol defaults to tol.  Returns the
    worst elementwise err/A (in units of A) and prints it with the relative
    RMS error."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite values"
    rms_tol = tol if rms_tol is None else rms_tol
    err = np.abs(gpu - ref)
    if scale is None:
        rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
        bound = tol * (np.abs(ref) + rms)
    else:
        scale = np.asarray(scale, np.float64)
        assert (np.abs(ref) <= scale * (1 + 1e-12) + 1e-300).all(), f"{what}: |ref| exceeds its term magnitude"
        rms = float(np.sqrt(np.mean(scale ** 2))) if scale.size else 0.0
        bound = tol * (scale + rms / 100)
    ref_norm = float(np.sqrt(np.sum(ref ** 2)))
    rel_rms = float(np.sqrt(np.sum(err ** 2))) / ref_norm if ref_norm > 0 else float(np.sqrt(np.sum(err ** 2)))
    worst = float((err / (bound / tol + 1e-300)).max()) if err.size else 0.0
    line = (f"{what}: max abs err {err.max() if err.size else 0:.3g}, worst err/A {worst:.3g} "
            f"(tol {tol}), rel RMS {rel_rms:.3g} (tol {rms_tol}), n {err.size}")
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / (bound + 1e-300)), err.shape)
        _margin_log("FAIL " + line)
        raise AssertionError(f"{what}: {bad.sum()} of {err.size} outside tol {tol}; worst at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r} bound {bound[i]!r} (max abs err {err.max():.3g})")
    if rel_rms > rms_tol:
        _margin_log("FAIL " + line)
        raise AssertionError(f"{what}: relative RMS error {rel_rms:.4g} above {rms_tol}")
    print("  " + line)
    _margin_log(line)
    MARGINS.append((os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], what, worst / tol,
                    rel_rms / rms_tol if rms_tol > 0 else 0.0))
    return worst


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


@functools.lru_cache(maxsize=None)
def inputs(cid: int, small: bool, seed: int = 0):
    cfg = W.get_config(cid, small=small)
    inp = W.make_inputs(cfg, seed)
    return inp, W.oracle_view(inp)


@functools.lru_cache(maxsize=None)
def routing_inputs(cid: int, small: bool, seed: int = 0):
    """The same draws without the expert weights (routing and dispatch only)."""
    cfg = W.get_config(cid, small=small)
    inp = W.make_inputs(cfg, seed, weights=False)
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


def check_routing(gpu_ids, gpu_logits, oracle_logits, cfg, forced=None, what="ids"):
    """check_ids, plus: the GPU logits equal the oracle's float64 logits to
    fp32 accuracy, and every row where the oracle's own float64 selection
    differs from the GPU's is a near-tie (the swapped experts' float64 logits,
    or for group-limited routing the group scores at the cut, within 2e-4)."""
    gl = np.asarray(gpu_logits, np.float64)
    ol = np.asarray(oracle_logits, np.float64)
    assert (np.abs(gl - ol) <= 1e-4 + 1e-6 * np.abs(ol)).all(), f"{what}: logits differ"
    check_ids(gpu_ids, gl, cfg, forced, what)
    own_ids, _ = route_cfg(ol, cfg, forced)
    gpu_ids = np.asarray(gpu_ids)
    rows = np.nonzero((own_ids != gpu_ids).any(1))[0]
    gm = grouped_margins(ol, cfg) if (cfg.score == "sigmoid" and cfg.n_groups > 1) else None
    for t in rows:
        j = int(np.nonzero(own_ids[t] != gpu_ids[t])[0][0])
        a, b = int(gpu_ids[t, j]), int(own_ids[t, j])
        near = abs(ol[t, a] - ol[t, b]) < 2e-4 or (gm is not None and gm[t] < 2e-4)
        assert near, f"{what}: token {t} slot {j} picks {a} not {b} away from a near-tie"
    assert len(rows) <= max(2, 0.01 * len(gpu_ids)), f"{what}: {len(rows)} near-tie rows"
    return len(rows)


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
