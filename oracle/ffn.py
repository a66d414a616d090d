"""SwiGLU expert FFN (oracle).

The pages name the expert as GEMM + act-and-mul ("[Core/DBO][1/N]", the
per-step latency discussion: the batched MoE GEMM kernel and the act_and_mul
kernel both grow under DBO) and a fused SiLU-mul ("[Core/DBO][1/N]", CI
discussion).  Reading: per expert, W13 stacks the gate rows [0, I) over the
up rows [I, 2I); h = silu(x G^T) * (x U^T); y = h W2^T, silu(g) = g/(1+e^-g).
"""
import numpy as np


def silu(g: np.ndarray) -> np.ndarray:
    # for g below about -709, e^-g overflows to inf and g / inf = -0, the limit
    # of silu; the overflow is expected there and not reported
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_expert(x: np.ndarray, w13: np.ndarray, w2: np.ndarray, with_scale: bool = False):
    """x [n, H] f64, w13 [2I, H] f64, w2 [H, I] f64 -> y [n, H] f64.

    with_scale: also return |h| |W2|^T, the magnitude of the terms each output
    element sums (the scale of a first-order rounding-error bound of the down
    projection; it bounds |y| by the triangle inequality)."""
    I = w13.shape[0] // 2
    gate = x @ w13[:I].T
    up = x @ w13[I:].T
    h = silu(gate) * up
    y = h @ w2.T
    if with_scale:
        return y, np.abs(h) @ np.abs(w2).T
    return y


def grouped_ffn_ref(x_perm: np.ndarray, offsets: np.ndarray, weights_of, with_scale: bool = False):
    """Rows [offsets[e], offsets[e+1]) of x_perm belong to local expert e;
    weights_of(e) -> (w13 f64, w2 f64).  Returns y_perm [M, H] f64 for the
    M = offsets[-1] dispatched rows (and the per-element term magnitude)."""
    x_perm = np.asarray(x_perm, np.float64)
    M = int(offsets[-1])
    y = np.zeros((M, x_perm.shape[1]), np.float64)
    s = np.zeros_like(y)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            w13, w2 = weights_of(e)
            y[a:b], s[a:b] = swiglu_expert(x_perm[a:b], w13, w2, with_scale=True)
    return (y, s) if with_scale else y
