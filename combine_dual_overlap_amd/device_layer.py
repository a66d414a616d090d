"""Device-side plumbing around dbo_moe_layer: uploads one layer's weights,
builds the moe_layer_desc, owns the workspace and output, and runs the layer
through the C ABI.  Memory and streams come from torch; every step of the
layer runs in libdbomoe.so.
"""
from __future__ import annotations

import torch

from . import binding as B


def _dev(t, device):
    return None if t is None else t.contiguous().to(device, non_blocking=False)


def concat_shared(shared_w13: list, shared_w2: list):
    """Several always-on SwiGLU experts as ONE expert: gate rows stacked, then
    up rows stacked ([sum I_i, H] each), down matrices side by side.  The sum
    of the experts' outputs equals this expert's output (a layout change of
    the weights, done once at load time)."""
    if not shared_w13:
        return None, None, 0
    gates, ups = [], []
    for w in shared_w13:
        I = w.shape[0] // 2
        gates.append(w[:I])
        ups.append(w[I:])
    w13 = torch.cat(gates + ups, dim=0).contiguous()
    w2 = torch.cat(list(shared_w2), dim=1).contiguous()
    return w13, w2, w2.shape[1]


class DeviceLayer:
    """One MoE layer resident on the GPU.

    `inp` is a dict with x [T,H], w_router [E,H], logit_bias, forced_ids, w13,
    w2, w13_scale, w2_scale, shared_w13, shared_w2 (CPU or device tensors) and
    `cfg` with the routing fields (E, k, score, renormalize, n_groups,
    topk_groups, group_topn, routed_scale, expert_begin, expert_end, H, I).
    fp8_act: run the routed experts with fp8 activations (fp8 weights only).
    """

    def __init__(self, inp: dict, device: str = "cuda", T_max: int = None, fp8_act: bool = False):
        cfg = inp["cfg"]
        self.cfg = cfg
        d = torch.device(device)
        self.device = d
        self.x = _dev(inp["x"], d)
        self.w_router = _dev(inp["w_router"], d)
        self.logit_bias = _dev(inp.get("logit_bias"), d)
        self.forced_ids = _dev(inp.get("forced_ids"), d)
        self.w13 = _dev(inp["w13"], d)
        self.w2 = _dev(inp["w2"], d)
        self.w13_scale = _dev(inp.get("w13_scale"), d)
        self.w2_scale = _dev(inp.get("w2_scale"), d)
        sh13, sh2, shI = concat_shared(inp.get("shared_w13") or [], inp.get("shared_w2") or [])
        self.shared_w13, self.shared_w2 = _dev(sh13, d), _dev(sh2, d)
        self.route = B.route_params(cfg.E, cfg.k, cfg.score, cfg.renormalize, cfg.n_groups, cfg.topk_groups,
                                    cfg.group_topn, cfg.routed_scale)
        self.desc = B.moe_layer_desc(
            cfg.H, cfg.I, B.dtype_code(self.x), B.dtype_code(self.w13), self.route,
            cfg.expert_begin, cfg.expert_end, B.ptr(self.w_router), B.ptr(self.w13), B.ptr(self.w2),
            B.ptr(self.w13_scale), B.ptr(self.w2_scale), shI, B.ptr(self.shared_w13), B.ptr(self.shared_w2),
            int(bool(fp8_act)))
        self.T = self.x.shape[0]
        self.T_max = T_max or self.T
        nbytes = B.moe_layer_workspace_size(self.desc, self.T_max)
        if nbytes == 0:
            raise B.MoEError(B.MOE_ERR_INVALID_ARG, "moe_layer_workspace_size")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=d)
        self.out = torch.empty_like(self.x)
        self.ctx = B.DboContext()
        self.comm = torch.cuda.Stream(device=d)

    def run(self, schedule: str = "dbo", min_tokens_to_split: int = 2, split_at: int = -1,
            comm_cu_budget: int = 0, ffn_tile_m: int = 0, x=None, out=None, forced_ids=None):
        x = self.x if x is None else x
        out = self.out if out is None else out
        forced = self.forced_ids if forced_ids is None else forced_ids
        opts = B.dbo_opts(B.SCHEDULES[schedule], min_tokens_to_split, split_at, comm_cu_budget, ffn_tile_m)
        # the compute stream is the caller's current stream (also under graph
        # capture); the comm stream joins it through the layer's events
        compute = torch.cuda.current_stream(self.device)
        B.dbo_moe_layer(self.ctx, self.desc, x, out, opts, self.ws, compute, self.comm,
                        forced_ids=forced, logit_bias=self.logit_bias)
        return out

    def view(self, mb: int, name: str, dtype, shape, T: int = None):
        """A tensor view of microbatch mb's intermediate `name` inside the
        workspace (layout of a call with T tokens)."""
        off = B.moe_layer_workspace_layout(self.desc, self.T if T is None else T, mb)[name]
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty(0, dtype=dtype).element_size()
        return self.ws[off:off + nbytes].view(dtype).view(*shape)
