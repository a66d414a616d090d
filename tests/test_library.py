"""Host-side checks of libdbomoe.so (no GPU): it loads, exports every entry
point include/dbomoe.h declares, and its argument validation rejects bad
calls before touching a device."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "dbomoe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


def test_build_and_load():
    from combine_dual_overlap_amd import binding
    assert binding.lib() is not None


def test_every_declared_symbol_is_exported():
    from combine_dual_overlap_amd import binding
    names = _declared()
    assert len(names) >= 17, names
    L = binding.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(binding.EXPORTED) == names


def test_status_strings():
    from combine_dual_overlap_amd import binding
    for s in range(0, -6, -1):
        assert binding.status_string(s).startswith("MOE_")
    assert binding.status_string(-99) == "unknown moe_status"


def test_workspace_queries():
    from combine_dual_overlap_amd import binding as B
    assert B.moe_dispatch_workspace_size(4096, 8, 128) >= 128 * 128 * 4
    assert B.moe_dispatch_workspace_size(-1, 8, 128) == 0
    assert B.moe_ffn_workspace_size(1000, 768, B.MOE_BF16) >= 1000 * 768 * 2
    assert B.moe_route_workspace_size(2048, 7168, 256) >= 2048 * 256 * 4


def _desc(B, **kw):
    p = B.route_params(64, 6)
    d = B.moe_layer_desc(2048, 1408, B.MOE_BF16, B.MOE_BF16, p, 0, 64, 256, 512, 768, None, None, 0, None, None)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_layer_workspace_size_and_validation():
    from combine_dual_overlap_amd import binding as B
    d = _desc(B)
    n = B.moe_layer_workspace_size(d, 256)
    # two halves, each holding at least x_perm and y_perm for 256*6 rows
    assert n >= 2 * 2 * 256 * 6 * 2048 * 2
    assert B.moe_layer_workspace_size(_desc(B, I=1400), 256) == 0          # I % 64 != 0
    assert B.moe_layer_workspace_size(_desc(B, expert_end=65), 256) == 0   # beyond E
    assert B.moe_layer_workspace_size(_desc(B, w13=513), 256) == 0         # misaligned weight pointer
    lay = B.moe_layer_workspace_layout(d, 256, 1)
    assert lay["logits"] == n // 2 and all(v % 256 == 0 for v in lay.values())


def test_ffn_auto_tile_choice():
    from combine_dual_overlap_amd import binding as B
    # decode-sized experts (Poisson(12) rows: the largest fits 32)
    assert B.moe_ffn_auto_tile(B.MOE_BF16, B.MOE_BF16, 2048, 1408, 12, 128, 2816) == 32
    assert B.moe_ffn_auto_tile(B.MOE_BF16, B.MOE_FP8_E4M3FN, 7168, 2048, 12) == 32
    # about 36 rows per expert (the largest fits 64); about 64 (the largest
    # does not: one 128-row tile each rather than a second, nearly empty one)
    assert B.moe_ffn_auto_tile(B.MOE_BF16, B.MOE_FP8_E4M3FN, 7168, 2048, 36) == 64
    assert B.moe_ffn_auto_tile(B.MOE_BF16, B.MOE_FP8_E4M3FN, 7168, 2048, 64) == 128
    # prefill-sized experts
    assert B.moe_ffn_auto_tile(B.MOE_BF16, B.MOE_FP8_E4M3FN, 2048, 768, 256) == 128
    assert B.moe_ffn_auto_tile(B.MOE_F32, B.MOE_F32, 128, 256, 8) == 32
    # invalid shapes
    assert B.moe_ffn_auto_tile(B.MOE_BF16, B.MOE_BF16, 2048, 1400, 12) == 0
    assert B.moe_ffn_auto_tile(B.MOE_BF16, B.MOE_FP8_E4M3FN, 2048, 192, 12) == 0


def test_entry_points_reject_bad_arguments_without_a_device():
    from combine_dual_overlap_amd import binding as B
    L = B.lib()
    A = 1 << 20      # aligned fake addresses: validation fails before any device access
    # k out of range
    assert L.moe_dispatch(A, B.MOE_BF16, 10, 128, A, 0, 8, 0, 8, 0, A, A, None, A, A, A, A, 1 << 20, None) \
        == B.MOE_ERR_INVALID_ARG
    # misaligned x
    assert L.moe_dispatch(A + 4, B.MOE_BF16, 10, 128, A, 2, 8, 0, 8, 0, A, A, None, A, A, A, A, 1 << 20, None) \
        == B.MOE_ERR_MISALIGNED
    # workspace too small
    assert L.moe_dispatch(A, B.MOE_BF16, 10, 128, A, 2, 8, 0, 8, 0, A, A, None, A, A, A, A, 16, None) \
        == B.MOE_ERR_WORKSPACE
    # fp8 weights need I % 128
    assert L.moe_grouped_ffn(A, B.MOE_BF16, 256, 192, A, 4, 100, A, A, B.MOE_FP8_E4M3FN, A, A, A, 0, A,
                             1 << 30, None) == B.MOE_ERR_UNSUPPORTED
    # scales given for bf16 weights
    assert L.moe_grouped_ffn(A, B.MOE_BF16, 256, 192, A, 4, 100, A, A, B.MOE_BF16, A, A, A, 0, A,
                             1 << 30, None) == B.MOE_ERR_INVALID_ARG
    # fp32 activations with bf16 weights
    assert L.moe_grouped_ffn(A, B.MOE_F32, 256, 192, A, 4, 100, A, A, B.MOE_BF16, None, None, A, 0, A,
                             1 << 30, None) == B.MOE_ERR_UNSUPPORTED
    # tile height out of range
    assert L.moe_grouped_ffn(A, B.MOE_BF16, 256, 192, A, 4, 100, A, A, B.MOE_BF16, None, None, A, 48, A,
                             1 << 30, None) == B.MOE_ERR_INVALID_ARG
    # 16-row tiles are not offered
    assert L.moe_grouped_ffn(A, B.MOE_BF16, 4096, 192, A, 4, 100, A, A, B.MOE_BF16, None, None, A, 16, A,
                             1 << 30, None) == B.MOE_ERR_INVALID_ARG
    # combine: out aliasing y_perm
    assert L.moe_combine(A, B.MOE_BF16, 4, 128, 2, A, A, None, A, None) == B.MOE_ERR_INVALID_ARG
    # route: group-limited with k larger than the kept groups hold
    p = B.route_params(16, 8, "sigmoid", True, n_groups=8, topk_groups=2, group_topn=2)
    assert L.moe_route_topk(A, B.MOE_BF16, 4, 128, A, None, None, ctypes.byref(p), None, A, A, A, 1 << 20,
                            None) == B.MOE_ERR_INVALID_ARG
    # T == 0 is a no-op
    assert L.moe_combine(A, B.MOE_BF16, 0, 128, 2, A, A, None, A + 256, None) == B.MOE_OK
