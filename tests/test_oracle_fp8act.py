"""Pins of the oracle's fp8-activation path (per-row, per-128-column fp8
quantisation with power-of-two scales; the SwiGLU expert that quantises x and
h) against hand-derived values, closed forms and torch's own float8 cast.
No GPU."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from conftest import read_golden

RNG = np.random.default_rng(77)


def _torch_encode(v: np.ndarray) -> np.ndarray:
    """torch's float32 -> float8_e4m3fn cast (round to nearest even), as codes.
    The values must be float32 numbers: torch casts float64 through float32,
    which rounds twice."""
    v32 = np.ascontiguousarray(v, np.float32)
    assert np.array_equal(v32.astype(np.float64), np.asarray(v, np.float64))
    return torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_quant_rows(x: np.ndarray):
    """The same quantisation written with torch primitives only: amax per
    group, the exponent from torch.frexp, the codes from torch's float8 cast.
    (torch casts float64 through float32: for a value within float32 rounding
    of an fp8 tie that rounds twice; the seeded inputs here hold none.)"""
    t = torch.from_numpy(x).double()
    n, K = t.shape
    g = t.view(n, K // 128, 128)
    amax = g.abs().amax(dim=2)
    m, p = torch.frexp(amax / 448.0)           # amax/448 = m * 2^p, 0.5 <= m < 1 (exact: /448 scales by 7*2^6)
    e = torch.where(m == 0.5, p - 1, p)        # 2^e >= amax/448, smallest such power of two
    e = torch.where(amax == 0, torch.full_like(e, -127), torch.clamp(e, min=-127))
    scaled = g * torch.pow(2.0, -e.double())[:, :, None]
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, K)
    return codes.numpy(), e.numpy().astype(np.int64)


# ------------------------------------------------------------------ encoder

def _between_codes_and_ties():
    """float32 values: every code, every exact tie, the float32 neighbours of
    each tie, and random points between codes."""
    pos = O.FP8_E4M3FN_TABLE[:0x7F].astype(np.float32)
    mids = (pos[:-1] + pos[1:]) / np.float32(2)          # exact ties
    inner = (pos[:-1] + (pos[1:] - pos[:-1]) * RNG.uniform(0.01, 0.99, size=pos.size - 1)).astype(np.float32)
    vals = np.concatenate([pos, mids, inner, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1e9))])
    return np.concatenate([vals, -vals]).astype(np.float64)


def test_encode_matches_torch_cast_on_ties_subnormals_and_signs():
    v = _between_codes_and_ties()
    v = v[np.abs(v) <= 448.0]
    got = O.fp8_e4m3fn_encode(v)
    want = _torch_encode(v)
    assert np.array_equal(got, want)


def test_encode_matches_torch_cast_on_random_values():
    v = np.concatenate([RNG.standard_normal(50000) * 60, RNG.standard_normal(20000) * 1e-3,
                        RNG.uniform(-448, 448, 20000)]).astype(np.float32).astype(np.float64)
    assert np.array_equal(O.fp8_e4m3fn_encode(v), _torch_encode(v))


def test_encode_roundtrips_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = np.array([O.fp8_e4m3fn_value(int(c)) for c in codes])
    vals = np.where(codes == 0x80, -0.0, vals)
    assert np.array_equal(O.fp8_e4m3fn_encode(vals), codes)


def test_encode_ties_go_to_even_codes():
    pos = O.FP8_E4M3FN_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    got = O.fp8_e4m3fn_encode(mids).astype(int)
    assert np.all(got % 2 == 0)
    assert np.all((got == np.arange(0x7E)) | (got == np.arange(1, 0x7F)))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.fp8_e4m3fn_encode(np.array([464.0]))
    with pytest.raises(ValueError):
        O.fp8_e4m3fn_encode(np.array([np.nan]))


# ------------------------------------------------------------------ scales

def test_group_exponent_closed_forms():
    for j in range(-120, 121, 7):
        b = 448.0 * 2.0 ** j
        assert O.group_exponent(b) == j                       # exactly at the bound
        assert O.group_exponent(np.nextafter(b, np.inf)) == j + 1
        assert O.group_exponent(np.nextafter(b, 0)) == j
        assert O.group_exponent(b / 2 + b / 4) == j           # 0.75 * bound still needs 2^j
    assert O.group_exponent(0.0) == -127
    assert O.group_exponent(2.0 ** -140) == -127              # clamped at the E8M0 minimum
    assert O.group_exponent(1.0) == -8                        # 448 * 2^-9 < 1 <= 448 * 2^-8
    assert O.group_exponent(3.5) == -7


def test_quant_rows_golden():
    g = read_golden("fp8_act_quant_handcalc.txt")
    x = np.zeros((2, 256))
    for key, vals in g.items():
        if key.startswith("x."):
            _, r, c = key.split(".")
            x[int(r), int(c)] = float(vals[0])
    assert np.array_equal(O.decode(W.bits(torch.from_numpy(x).to(torch.bfloat16)), "bf16"), x)  # bf16 values
    codes, e = O.quant_rows_fp8(x)
    want_codes = np.zeros((2, 256), np.uint8)
    for key, vals in g.items():
        kind, r, c = key.split(".")
        if kind == "exp":
            assert e[int(r), int(c)] == int(vals[0]), key
        elif kind == "code":
            want_codes[int(r), int(c)] = int(vals[0], 16)
    assert np.array_equal(codes, want_codes)


def test_quant_rows_matches_torch_primitives():
    n, K = 64, 640
    mag = 2.0 ** RNG.integers(-30, 30, size=(n, K // 128, 1))   # very different groups
    x = (RNG.standard_normal((n, K // 128, 128)) * mag).reshape(n, K)
    x[3, :128] = 0.0                                           # an all-zero group
    x[5, 128:256] = 448.0 * 2.0 ** -4                          # amax exactly at a bound
    x = O.decode(W.bits(torch.from_numpy(x).to(torch.bfloat16)), "bf16")
    codes, e = O.quant_rows_fp8(x)
    tc, te = _torch_quant_rows(x)
    assert np.array_equal(e, te)
    assert np.array_equal(codes, tc)


def test_quant_error_within_half_step_and_zero_groups_exact():
    x = RNG.standard_normal((32, 512)) * 3
    x[0, :128] = 0
    xq = O.fp8_roundtrip_rows(x)
    assert np.all(xq[0, :128] == 0)
    codes, e = O.quant_rows_fp8(x)
    step_floor = np.repeat(np.ldexp(1.0, e - 9), 128, axis=1)  # subnormal step 2^-9 scaled
    err = np.abs(xq - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, step_floor / 2) * (1 + 1e-12))


def test_quant_is_lossless_on_representable_rows():
    codes = RNG.integers(0, 0x7F, size=(16, 256)).astype(np.uint8)
    codes |= (RNG.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    codes[:, 0] = 0x7E                                        # every group reaches 448 * 2^e
    codes[:, 128] = 0xFE
    e = RNG.integers(-20, 20, size=(16, 2))
    x = O.dequant_rows_fp8(codes, e)
    c2, e2 = O.quant_rows_fp8(x)
    assert np.array_equal(e2, e)
    assert np.array_equal(O.dequant_rows_fp8(c2, e2), x)


# ------------------------------------------------------------------ expert

def _weights(H, I, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal((2 * I, H)) * 0.05, g.standard_normal((H, I)) * 0.05


def test_swiglu_fp8act_matches_torch_pipeline():
    H, I = 256, 384
    x = RNG.standard_normal((24, H))
    w13, w2 = _weights(H, I, 5)

    def tq(a):
        c, e = _torch_quant_rows(a)
        return O.dequant_rows_fp8(c, e)

    tx = tq(x)
    g = tx @ w13[:I].T
    u = tx @ w13[I:].T
    h = torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u
    y_ref = tq(h) @ w2.T
    assert np.allclose(O.swiglu_expert_fp8act(x, w13, w2), y_ref, rtol=1e-12, atol=1e-12)


def test_swiglu_fp8act_quantises_both_x_and_h():
    H, I = 128, 256
    x = RNG.standard_normal((8, H))
    w13, w2 = _weights(H, I, 6)
    y8 = O.swiglu_expert_fp8act(x, w13, w2)
    # with x already fp8-exact only h is quantised: differs from the plain expert
    xq = O.fp8_roundtrip_rows(x)
    y_plain_xq = O.swiglu_expert(xq, w13, w2)
    assert np.allclose(O.swiglu_expert_fp8act(xq, w13, w2), y8, rtol=0, atol=0)
    assert not np.allclose(y8, y_plain_xq, rtol=0, atol=1e-9)
    # and the quantisation error stays at the fp8 level (3 mantissa bits)
    y = O.swiglu_expert(x, w13, w2)
    _, s = O.swiglu_expert(x, w13, w2, with_scale=True)
    assert np.all(np.abs(y8 - y) <= 0.2 * s + 1e-12)


def test_grouped_fp8act_ref_rows():
    H, I = 128, 128
    offsets = np.array([0, 3, 3, 10])
    xs = RNG.standard_normal((12, H))
    ws = [_weights(H, I, 10 + e) for e in range(3)]
    y = O.grouped_ffn_fp8act_ref(xs, offsets, lambda e: ws[e])
    assert y.shape == (10, H)
    assert np.array_equal(y[0:3], O.swiglu_expert_fp8act(xs[0:3], *ws[0]))
    assert np.array_equal(y[3:10], O.swiglu_expert_fp8act(xs[3:10], *ws[2]))


def test_layer_fp8act_uses_fp8_expert_for_routed_and_bf16_for_shared():
    cfg = W.get_config(4, small=True).replace(T=48)
    ov = W.oracle_view(W.make_inputs(cfg, seed=2))
    ref = O.moe_layer_expert(ov)
    ov8 = dict(ov, fp8_act=True)
    r8 = O.moe_layer_expert(ov8)
    tok = O.moe_layer_token(ov8, tokens=np.arange(0, 48, 5))
    assert np.allclose(r8["out"][::5], tok["out"], rtol=1e-10, atol=1e-12)
    assert np.array_equal(r8["ids"], ref["ids"])
    diff = np.abs(r8["out"] - ref["out"])
    assert diff.max() > 0 and np.all(diff <= 0.2 * ref["scale"] + 1e-12)
