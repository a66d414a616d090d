"""Exact decoding of stored values into float64 (oracle; test infrastructure).

The pages run an FP8 model ("[Perf] Fix DBO overlap ...", Test Plan:
Qwen3-30B-A3B-Instruct-2507-FP8) and an fp8 SiLU-mul quantisation op
("[Core/DBO][1/N]", CI discussion) but fix no format.  Reading: OCP 8-bit
floating point E4M3 ("fn" variant: no infinities, S.1111.111 is NaN, max
448), one fp32 scale per 128x128 weight block, real weight = code value x
block scale.  bf16 is IEEE binary32 with the low 16 bits dropped.
"""
import math

import numpy as np


def fp8_e4m3fn_value(code: int) -> float:
    """Value of one E4M3 (fn) code: 1 sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); the single
    pattern with exponent 15 and mantissa 7 is NaN; no infinities."""
    code = int(code) & 0xFF
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


FP8_E4M3FN_TABLE = np.array([fp8_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored raw values -> float64, exactly.

    dtype "f32": float32 array; "bf16": uint16 bit patterns (the high half of
    a binary32); "fp8": uint8 E4M3 codes (unscaled)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return FP8_E4M3FN_TABLE[np.asarray(a, dtype=np.uint8)]
    raise ValueError(dtype)


def dequant_fp8_blocks(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """Real [R, C] matrix from E4M3 codes and per-(128 x 128)-block fp32
    scales: W[r, c] = value(code[r, c]) * scale[r // 128, c // 128]."""
    R, C = codes.shape
    vals = decode(codes, "fp8")
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    rows = np.arange(R) // block
    cols = np.arange(C) // block
    return vals * s[rows[:, None], cols[None, :]]
