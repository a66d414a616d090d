"""fp8 quantisation of activations (oracle; test infrastructure).

The pages name a fused SiLU-mul + fp8 quantisation op that feeds an fp8 GEMM
("[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM", CI discussion)
and run an FP8 model ("[Perf] Fix DBO overlap: capture DeepEP event before
yield", Test Plan), but print no scaling rule.  Reading (the usual
fine-grained fp8 GEMM input format): each row of an activation matrix is cut
into groups of 128 consecutive columns; a group is stored as OCP E4M3 (fn)
codes plus one power-of-two scale 2^e, e the smallest integer >= -127 with
amax(|group|) <= 448 * 2^e (an 8-bit exponent-only scale, E8M0); code =
round-to-nearest-even of value / 2^e.  Dividing by a power of two is exact,
so the codes depend on the values alone, not on the precision they are
computed in.  Real value of a stored element = code value * 2^e.

The expert with fp8 activations: the dispatched rows x are quantised this
way, gate/up use the dequantised rows, h = silu(gate) * up is quantised the
same way (groups of 128 of the I columns), and the down projection uses the
dequantised h.
"""
import numpy as np

from .numerics import FP8_E4M3FN_TABLE, decode
from .ffn import silu

GROUP = 128
FP8_MAX = 448.0
E_MIN = -127                 # smallest exponent an E8M0 scale holds (byte 0)
E8M0_BIAS = 127

# Magnitudes of the codes 0x00..0x7E (0 .. 448), strictly increasing with
# the code: for a non-negative code c, its value is c's position in this list.
_POS = FP8_E4M3FN_TABLE[:0x7F]


def fp8_e4m3fn_encode(v) -> np.ndarray:
    """Round float64 values to the nearest E4M3 (fn) code, ties to the even
    code (the code whose mantissa's last bit is 0).  |v| must be <= 448 plus
    half a step (464 exclusive) and not NaN.  The sign bit is kept, also for
    values that round to zero."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(np.isnan(a)) or np.any(a >= 464.0):
        raise ValueError("value outside the E4M3 (fn) range")
    hi = np.searchsorted(_POS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def group_exponent(amax) -> np.ndarray:
    """Smallest integer e >= -127 with amax <= 448 * 2^e (amax >= 0, finite)."""
    a = np.asarray(amax, dtype=np.float64)
    # frexp: a = m * 2^p with 0.5 <= m < 1; since 448 = 0.875 * 2^9 the answer
    # is p - 9 or p - 8.  Start below it and step up while the bound fails.
    _, p = np.frexp(a)
    e = p.astype(np.int64) - 10
    for _ in range(3):
        e = np.where(a > FP8_MAX * np.ldexp(1.0, e), e + 1, e)
    e = np.maximum(np.where(a == 0.0, E_MIN, e), E_MIN)
    ok = (a <= FP8_MAX * np.ldexp(1.0, e)) & ((e == E_MIN) | (a > FP8_MAX * np.ldexp(1.0, e - 1)))
    assert ok.all()
    return e


def quant_rows_fp8(x) -> tuple:
    """x [n, K] float64 (K a multiple of 128) -> (codes uint8 [n, K],
    exponents int64 [n, K/128]).  Stored scale byte of a group = e + 127."""
    x = np.asarray(x, dtype=np.float64)
    n, K = x.shape
    if K % GROUP:
        raise ValueError("row length must be a multiple of 128")
    g = x.reshape(n, K // GROUP, GROUP)
    e = group_exponent(np.abs(g).max(axis=2, initial=0.0))
    scaled = g * np.ldexp(1.0, -e)[:, :, None]
    codes = fp8_e4m3fn_encode(scaled).reshape(n, K)
    return codes, e


def dequant_rows_fp8(codes, exps) -> np.ndarray:
    """Real values of quantised rows: code value * 2^e of the code's group."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, K = codes.shape
    vals = decode(codes, "fp8").reshape(n, K // GROUP, GROUP)
    return (vals * np.ldexp(1.0, np.asarray(exps))[:, :, None]).reshape(n, K)


def fp8_roundtrip_rows(x) -> np.ndarray:
    """x -> dequant(quant(x)): what an fp8 consumer of x sees."""
    return dequant_rows_fp8(*quant_rows_fp8(x))


def swiglu_expert_fp8act(x, w13, w2, with_scale: bool = False):
    """SwiGLU expert with fp8 activations: x [n, H] f64 (the rows as stored,
    before quantisation), w13 [2I, H], w2 [H, I] f64 -> y [n, H] f64.
    with_scale: also return |hq| |W2|^T (the down projection's term magnitude)."""
    I = w13.shape[0] // 2
    xq = fp8_roundtrip_rows(x)
    gate = xq @ w13[:I].T
    up = xq @ w13[I:].T
    h = silu(gate) * up
    hq = fp8_roundtrip_rows(h)
    y = hq @ w2.T
    if with_scale:
        return y, np.abs(hq) @ np.abs(w2).T
    return y


def grouped_ffn_fp8act_ref(x_perm, offsets, weights_of, with_scale: bool = False):
    """grouped_ffn_ref with fp8 activations: rows [offsets[e], offsets[e+1])
    of x_perm (float64 values of the stored bf16 rows) use local expert e."""
    x_perm = np.asarray(x_perm, np.float64)
    M = int(offsets[-1])
    y = np.zeros((M, x_perm.shape[1]), np.float64)
    s = np.zeros_like(y)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            w13, w2 = weights_of(e)
            y[a:b], s[a:b] = swiglu_expert_fp8act(x_perm[a:b], w13, w2, with_scale=True)
    return (y, s) if with_scale else y
