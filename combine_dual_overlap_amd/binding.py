"""ctypes binding of libdbomoe.so: the C ABI of include/dbomoe.h, same names.

Argument marshalling only: tensors become device pointers, streams become
hipStream_t handles, and a non-zero moe_status becomes a MoEError.  Every step
of the layer runs in the library's HIP kernels; there is no fallback path.  If
the library is not built, loading raises instead of degrading.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdbomoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_MISALIGNED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = \
    0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16, MOE_FP8_E4M3FN = 0, 1, 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
DBO_SCHED_UNSPLIT, DBO_SCHED_SERIAL, DBO_SCHED_DBO, DBO_SCHED_DBO_LATE_EVENT, DBO_SCHED_DBO_RECV_HOOK = 0, 1, 2, 3, 4
SCHEDULES = {"unsplit": 0, "serial": 1, "dbo": 2, "dbo_late_event": 3, "dbo_recv_hook": 4}

EXPORTED = [
    "moe_route_workspace_size", "moe_route_topk", "moe_dispatch_workspace_size", "moe_dispatch",
    "moe_get_device_error", "moe_ffn_workspace_size", "moe_ffn_auto_tile", "moe_grouped_ffn", "moe_combine",
    "dbo_ctx_create", "dbo_ctx_destroy", "dbo_ctx_set_timing", "dbo_ctx_ffn_times", "dbo_ctx_comm_times",
    "dbo_ctx_last_stats",
    "moe_layer_workspace_size", "moe_layer_workspace_layout", "dbo_moe_layer", "moe_status_string",
    "moe_quant_fp8_rows", "moe_dispatch_fp8", "moe_ffn_fp8_workspace_size", "moe_grouped_ffn_fp8",
    "moe_dispatch_send", "moe_dispatch_recv", "moe_dispatch_noalloc_max_workspace", "moe_dispatch_noalloc",
]


class moe_route_params(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("k", ctypes.c_int32), ("score", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("group_topn", ctypes.c_int32),
                ("routed_scale", ctypes.c_float)]


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("act", ctypes.c_int32),
                ("wdt", ctypes.c_int32), ("route", moe_route_params),
                ("expert_begin", ctypes.c_int32), ("expert_end", ctypes.c_int32),
                ("w_router", ctypes.c_void_p), ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w13_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
                ("shared_I", ctypes.c_int32), ("shared_w13", ctypes.c_void_p),
                ("shared_w2", ctypes.c_void_p), ("fp8_act", ctypes.c_int32)]


class dbo_opts(ctypes.Structure):
    _fields_ = [("schedule", ctypes.c_int32), ("min_tokens_to_split", ctypes.c_int32),
                ("split_at", ctypes.c_int32), ("comm_cu_budget", ctypes.c_int32),
                ("ffn_tile_m", ctypes.c_int32)]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_LIB = None
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


def lib():
    """The loaded library.  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m combine_dual_overlap_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "moe_route_workspace_size": (_sz, [_i64, _i32, _i32]),
            "moe_route_topk": (_i32, [_vp, _i32, _i64, _i32, _vp, _vp, _vp, ctypes.POINTER(moe_route_params),
                                      _vp, _vp, _vp, _vp, _sz, _vp]),
            "moe_dispatch_workspace_size": (_sz, [_i64, _i32, _i32]),
            "moe_dispatch": (_i32, [_vp, _i32, _i64, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
            "moe_get_device_error": (_i32, [_vp, ctypes.POINTER(_i32), _vp]),
            "moe_dispatch_noalloc_max_workspace": (_sz, []),
            "moe_dispatch_noalloc": (_i32, [_vp, _i32, _i64, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                            _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
            "moe_ffn_workspace_size": (_sz, [_i64, _i32, _i32]),
            "moe_ffn_auto_tile": (_i32, [_i32, _i32, _i32, _i32, _i64, _i64, _i32]),
            "moe_grouped_ffn": (_i32, [_vp, _i32, _i32, _i32, _vp, _i32, _i64, _vp, _vp, _i32, _vp, _vp,
                                       _vp, _i32, _vp, _sz, _vp]),
            "moe_combine": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
            "dbo_ctx_create": (_i32, [ctypes.POINTER(_vp)]),
            "dbo_ctx_destroy": (None, [_vp]),
            "dbo_ctx_set_timing": (_i32, [_vp, _i32]),
            "dbo_ctx_ffn_times": (_i32, [_vp, _i32, ctypes.POINTER(ctypes.c_float)]),
            "dbo_ctx_comm_times": (_i32, [_vp, _i32, ctypes.POINTER(ctypes.c_float)]),
            "dbo_ctx_last_stats": (_i32, [_vp, ctypes.POINTER(_i64)]),
            "moe_layer_workspace_size": (_sz, [ctypes.POINTER(moe_layer_desc), _i64]),
            "moe_layer_workspace_layout": (_i32, [ctypes.POINTER(moe_layer_desc), _i64, _i32,
                                                  ctypes.POINTER(_i64)]),
            "dbo_moe_layer": (_i32, [_vp, ctypes.POINTER(moe_layer_desc), _vp, _i64, _vp, _vp, _vp,
                                     ctypes.POINTER(dbo_opts), _vp, _sz, _vp, _vp]),
            "moe_status_string": (ctypes.c_char_p, [_i32]),
            "moe_quant_fp8_rows": (_i32, [_vp, _i64, _i32, _vp, _vp, _vp]),
            "moe_dispatch_fp8": (_i32, [_vp, _i64, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
            "moe_ffn_fp8_workspace_size": (_sz, [_i64, _i32]),
            "moe_dispatch_send": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _sz, _vp]),
            "moe_dispatch_recv": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
            "moe_grouped_ffn_fp8": (_i32, [_vp, _vp, _i32, _i32, _vp, _i32, _i64, _vp, _vp, _vp, _vp,
                                           _vp, _i32, _vp, _sz, _vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_FP8_E4M3FN
    raise ValueError(f"unsupported dtype {t.dtype}")


def stream_handle(s=None):
    if s is None:
        s = torch.cuda.current_stream()
    return s.cuda_stream


def route_params(E, k, score="softmax", renormalize=False, n_groups=1, topk_groups=1, group_topn=2,
                 routed_scale=1.0) -> moe_route_params:
    return moe_route_params(E, k, MOE_SCORE_SOFTMAX if score == "softmax" else MOE_SCORE_SIGMOID,
                            int(bool(renormalize)), n_groups, topk_groups if n_groups > 1 else 1,
                            group_topn if n_groups > 1 else 1, float(routed_scale))


# ------------------------------------------------------------------ entry points

def moe_route_workspace_size(T: int, H: int, E: int) -> int:
    return lib().moe_route_workspace_size(T, H, E)


def moe_route_topk(x, w_router, params: moe_route_params, topk_ids, topk_w, ws, logits_out=None,
                   logit_bias=None, forced_ids=None, stream=None):
    T, H = x.shape
    _check(lib().moe_route_topk(ptr(x), dtype_code(x), T, H, ptr(w_router), ptr(logit_bias), ptr(forced_ids),
                                ctypes.byref(params), ptr(logits_out), ptr(topk_ids), ptr(topk_w), ptr(ws),
                                ws.numel() * ws.element_size(), stream_handle(stream)), "moe_route_topk")


def moe_dispatch_workspace_size(T: int, k: int, E_loc: int) -> int:
    return lib().moe_dispatch_workspace_size(T, k, E_loc)


def moe_dispatch(x, topk_ids, E_total, expert_begin, expert_end, counts, offsets, perm, inv, x_perm, ws,
                 tile_m=0, tile_offsets=None, stream=None):
    T, H = x.shape
    k = topk_ids.shape[1] if topk_ids.dim() == 2 else 1
    _check(lib().moe_dispatch(ptr(x), dtype_code(x), T, H, ptr(topk_ids), k, E_total, expert_begin, expert_end,
                              tile_m, ptr(counts), ptr(offsets), ptr(tile_offsets), ptr(perm), ptr(inv),
                              ptr(x_perm), ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream)),
           "moe_dispatch")


def moe_dispatch_noalloc_max_workspace() -> int:
    return lib().moe_dispatch_noalloc_max_workspace()


def moe_dispatch_noalloc(x, topk_ids, E_total, expert_begin, expert_end, counts, offsets, perm, inv, x_perm,
                         tile_m=0, tile_offsets=None, stream=None):
    T, H = x.shape
    k = topk_ids.shape[1] if topk_ids.dim() == 2 else 1
    _check(lib().moe_dispatch_noalloc(ptr(x), dtype_code(x), T, H, ptr(topk_ids), k, E_total, expert_begin,
                                      expert_end, tile_m, ptr(counts), ptr(offsets), ptr(tile_offsets), ptr(perm),
                                      ptr(inv), ptr(x_perm), stream_handle(stream)), "moe_dispatch_noalloc")


def moe_dispatch_send(topk_ids, E_total, expert_begin, expert_end, counts, offsets, perm, inv, ws, tile_m=0,
                      tile_offsets=None, stream=None):
    T = topk_ids.shape[0]
    k = topk_ids.shape[1] if topk_ids.dim() == 2 else 1
    _check(lib().moe_dispatch_send(ptr(topk_ids), T, k, E_total, expert_begin, expert_end, tile_m, ptr(counts),
                                   ptr(offsets), ptr(tile_offsets), ptr(perm), ptr(inv), ptr(ws),
                                   ws.numel() * ws.element_size(), stream_handle(stream)), "moe_dispatch_send")


def moe_dispatch_recv(x, k, inv, x_perm, xq_scale=None, stream=None):
    T, H = x.shape
    _check(lib().moe_dispatch_recv(ptr(x), dtype_code(x), T, H, k, ptr(inv), ptr(x_perm), ptr(xq_scale),
                                   stream_handle(stream)), "moe_dispatch_recv")


def moe_get_device_error(dispatch_ws, stream=None) -> int:
    code = ctypes.c_int32(0)
    _check(lib().moe_get_device_error(ptr(dispatch_ws), ctypes.byref(code), stream_handle(stream)),
           "moe_get_device_error")
    return code.value


def moe_ffn_workspace_size(cap_rows: int, I: int, act: int) -> int:
    return lib().moe_ffn_workspace_size(cap_rows, I, act)


def moe_ffn_auto_tile(act: int, wdt: int, H: int, I: int, rows_per_expert: int, rows1: int = 0,
                      I1: int = 0) -> int:
    return lib().moe_ffn_auto_tile(act, wdt, H, I, rows_per_expert, rows1, I1)


def moe_grouped_ffn(x_perm, I, offsets, E_loc, w13, w2, y_perm, ws, w13_scale=None, w2_scale=None,
                    tile_m=0, cap_rows=None, stream=None):
    cap = x_perm.shape[0] if cap_rows is None else cap_rows
    H = x_perm.shape[1]
    _check(lib().moe_grouped_ffn(ptr(x_perm), dtype_code(x_perm), H, I, ptr(offsets), E_loc, cap, ptr(w13),
                                 ptr(w2), dtype_code(w13), ptr(w13_scale), ptr(w2_scale), ptr(y_perm), tile_m,
                                 ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream)),
           "moe_grouped_ffn")


def moe_quant_fp8_rows(x, q, scale, stream=None):
    n, K = x.shape
    _check(lib().moe_quant_fp8_rows(ptr(x), n, K, ptr(q), ptr(scale), stream_handle(stream)), "moe_quant_fp8_rows")


def moe_dispatch_fp8(x, topk_ids, E_total, expert_begin, expert_end, counts, offsets, perm, inv, xq_perm,
                     xq_scale, ws, tile_m=0, tile_offsets=None, stream=None):
    T, H = x.shape
    k = topk_ids.shape[1] if topk_ids.dim() == 2 else 1
    _check(lib().moe_dispatch_fp8(ptr(x), T, H, ptr(topk_ids), k, E_total, expert_begin, expert_end, tile_m,
                                  ptr(counts), ptr(offsets), ptr(tile_offsets), ptr(perm), ptr(inv), ptr(xq_perm),
                                  ptr(xq_scale), ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream)),
           "moe_dispatch_fp8")


def moe_ffn_fp8_workspace_size(cap_rows: int, I: int) -> int:
    return lib().moe_ffn_fp8_workspace_size(cap_rows, I)


def moe_grouped_ffn_fp8(xq_perm, xq_scale, I, offsets, E_loc, w13, w2, w13_scale, w2_scale, y_perm, ws,
                        tile_m=0, cap_rows=None, stream=None):
    cap = xq_perm.shape[0] if cap_rows is None else cap_rows
    H = xq_perm.shape[1]
    _check(lib().moe_grouped_ffn_fp8(ptr(xq_perm), ptr(xq_scale), H, I, ptr(offsets), E_loc, cap, ptr(w13),
                                     ptr(w2), ptr(w13_scale), ptr(w2_scale), ptr(y_perm), tile_m, ptr(ws),
                                     ws.numel() * ws.element_size(), stream_handle(stream)),
           "moe_grouped_ffn_fp8")


def moe_combine(y_perm, T, k, inv, topk_w, out, shared_out=None, stream=None):
    H = out.shape[1]
    _check(lib().moe_combine(ptr(y_perm), dtype_code(out), T, H, k, ptr(inv), ptr(topk_w), ptr(shared_out),
                             ptr(out), stream_handle(stream)), "moe_combine")


class DboContext:
    """Owns a dbo_ctx (the per-microbatch HIP events)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib().dbo_ctx_create(ctypes.byref(h)), "dbo_ctx_create")
        self.handle = h

    def close(self):
        if self.handle:
            lib().dbo_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_timing(self, enable: bool):
        _check(lib().dbo_ctx_set_timing(self.handle, int(enable)), "dbo_ctx_set_timing")

    def ffn_times(self, back: int = 0):
        """[A gate/up, A down, B gate/up, B down] ms of the timed call `back` calls ago."""
        ms = (ctypes.c_float * 4)()
        _check(lib().dbo_ctx_ffn_times(self.handle, back, ms), "dbo_ctx_ffn_times")
        return list(ms)

    def comm_times(self, back: int = 0):
        """[A dispatch, B dispatch, A combine, B combine] ms of the timed call `back` calls ago."""
        ms = (ctypes.c_float * 4)()
        _check(lib().dbo_ctx_comm_times(self.handle, back, ms), "dbo_ctx_comm_times")
        return list(ms)

    def last_stats(self) -> dict:
        s = (ctypes.c_int64 * 6)()
        _check(lib().dbo_ctx_last_stats(self.handle, s), "dbo_ctx_last_stats")
        return dict(schedule=s[0], T0=s[1], yields_a=s[2], yields_b=s[3], stages=s[4], records=s[5])


def moe_layer_workspace_size(desc: moe_layer_desc, T_max: int) -> int:
    return lib().moe_layer_workspace_size(ctypes.byref(desc), T_max)


def moe_layer_workspace_layout(desc: moe_layer_desc, T: int, mb: int) -> dict:
    off = (ctypes.c_int64 * 12)()
    _check(lib().moe_layer_workspace_layout(ctypes.byref(desc), T, mb, off), "moe_layer_workspace_layout")
    names = ["logits", "topk_ids", "topk_w", "counts", "offsets", "tile_offsets", "perm", "inv", "x_perm",
             "y_perm", "shared_out", "dispatch_ws"]
    return dict(zip(names, list(off)))


def dbo_moe_layer(ctx: DboContext, desc: moe_layer_desc, x, out, opts: dbo_opts, ws, compute_stream=None,
                  comm_stream=None, forced_ids=None, logit_bias=None):
    T = x.shape[0]
    _check(lib().dbo_moe_layer(ctx.handle, ctypes.byref(desc), ptr(x), T, ptr(forced_ids), ptr(logit_bias),
                               ptr(out), ctypes.byref(opts), ptr(ws), ws.numel() * ws.element_size(),
                               stream_handle(compute_stream), stream_handle(comm_stream)), "dbo_moe_layer")
