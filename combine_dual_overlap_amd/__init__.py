"""MI355X-native Dual-Batch-Overlap expert-parallel MoE layer.

The compute path is libdbomoe.so (hand-written HIP kernels for gfx950 behind
the C ABI of include/dbomoe.h); `binding` exposes its entry points under the
same names and `device_layer` holds the device-side plumbing of one layer.
"""
from . import binding
from .binding import (moe_route_topk, moe_dispatch, moe_grouped_ffn, moe_combine, dbo_moe_layer,
                      DboContext, MoEError)
from .device_layer import DeviceLayer

__all__ = ["binding", "moe_route_topk", "moe_dispatch", "moe_grouped_ffn", "moe_combine", "dbo_moe_layer",
           "DboContext", "MoEError", "DeviceLayer"]
