"""Seeded synthetic workloads for the DBO MoE layer.

This module only draws inputs: activations, router weights, expert weights
(with the fp8 e4m3fn block quantisation that is their storage format), forced
expert ids and router logit biases.  It holds none of the layer's arithmetic
(no routing, no dispatch, no FFN, no combine); both the CPU oracle and the HIP
path consume exactly the tensors drawn here.

Workload shapes follow the five layer configurations the DBO pages' models
suggest (tiny fp32; DeepSeek-V2-Lite-shaped decode; Qwen3-30B-A3B-shaped fp8
prefill, which stands in for the 8192-token random-prompt prefill bench of
"[Perf] Fix DBO overlap: capture DeepEP event before yield", Test Plan;
DeepSeek-R1-shaped one-GPU expert share; Zipf-skewed uneven split).  Every
tensor has its own torch CPU generator, seeded as
``(cfg_id * 1000 + seed) * 100 + tensor_id``; values are drawn in fp32 and
rounded to nearest-even into the stored dtype.
"""
from __future__ import annotations

import copy
import math
from dataclasses import dataclass, field, asdict
from typing import Optional

import numpy as np
import torch

# tensor ids used in the seed recipe
TID_X, TID_WR, TID_W13, TID_W2, TID_SH_W13, TID_SH_W2, TID_FORCED, TID_ZIPF = 1, 2, 3, 4, 5, 6, 7, 8
TID_W13_SPREAD, TID_W2_SPREAD = 9, 10

FP8_BLOCK = 128
FP8_MAX = 448.0


@dataclass
class LayerConfig:
    name: str
    T: int                      # tokens in the layer call
    H: int                      # hidden size
    E: int                      # routed experts (global)
    k: int                      # experts per token
    I: int                      # SwiGLU intermediate size per expert
    act: str                    # activation dtype: "f32" | "bf16"
    wdt: str                    # expert weight dtype: "f32" | "bf16" | "fp8"
    score: str = "softmax"      # "softmax" | "sigmoid"
    renormalize: bool = False
    n_groups: int = 1           # expert groups for group-limited routing (1 = no limit)
    topk_groups: int = 1        # groups kept
    group_topn: int = 2         # group score = sum of the top-n scores in the group
    routed_scale: float = 1.0
    expert_begin: int = 0       # local expert range [expert_begin, expert_end)
    expert_end: int = -1
    n_shared: int = 0           # always-on shared experts (weight 1)
    shared_I: int = 0           # intermediate size of EACH shared expert
    forced_uniform: bool = False  # per-token uniform-random distinct expert ids
    zipf_alpha: float = 0.0     # Zipf popularity through a router logit bias (0 = off)
    seq_lens: Optional[list] = None  # descriptive request lengths (sum == T)
    x_std: float = 1.0
    w_std: float = 0.02
    wr_std: float = 0.02
    # fp8 weights: each 128x128 block of the N(0, w_std) draw is multiplied by
    # 2^u, u ~ U(-spread, spread), before quantisation, so block scales differ
    # from block to block (as in trained block-quantised checkpoints) and a
    # wrong block-scale index shows in the output.  0 = every block alike.
    fp8_block_spread: float = 0.0
    cfg_id: int = 0

    def __post_init__(self):
        if self.expert_end < 0:
            self.expert_end = self.E

    @property
    def E_loc(self) -> int:
        return self.expert_end - self.expert_begin

    def replace(self, **kw) -> "LayerConfig":
        c = copy.deepcopy(self)
        for key, v in kw.items():
            setattr(c, key, v)
        if "E" in kw and "expert_end" not in kw and self.expert_end == self.E:
            c.expert_end = c.E
        return c

    def as_dict(self) -> dict:
        return asdict(self)


def _c5_seq_lens(T: int, T0: int) -> list:
    """Mostly one-token decode requests plus one long prefill that crosses the split."""
    pre = max(1, T // 6)
    long = max(2, T // 2)
    if pre + long <= T0:
        pre = max(0, T0 - long // 2)
    rest = T - pre - long
    assert rest >= 0
    return [1] * pre + [long] + [1] * rest


CONFIGS = {
    1: LayerConfig("tiny_fp32", T=64, H=128, E=8, k=2, I=256, act="f32", wdt="f32",
                   score="softmax", renormalize=False, cfg_id=1),
    2: LayerConfig("v2lite_decode_bf16", T=256, H=2048, E=64, k=6, I=1408, act="bf16", wdt="bf16",
                   score="softmax", renormalize=False, n_shared=2, shared_I=1408, cfg_id=2),
    3: LayerConfig("qwen3_prefill_fp8w", T=8192, H=2048, E=128, k=8, I=768, act="bf16", wdt="fp8",
                   score="softmax", renormalize=True, forced_uniform=True, fp8_block_spread=4.0, cfg_id=3),
    4: LayerConfig("r1_share_fp8w", T=4096, H=7168, E=256, k=8, I=2048, act="bf16", wdt="fp8",
                   score="sigmoid", renormalize=True, n_groups=8, topk_groups=4, group_topn=2,
                   expert_begin=0, expert_end=32, fp8_block_spread=4.0, cfg_id=4),
    5: LayerConfig("skewed_zipf_bf16", T=6001, H=2048, E=64, k=6, I=1408, act="bf16", wdt="bf16",
                   score="softmax", renormalize=False, zipf_alpha=1.2,
                   seq_lens=[1] * 1000 + [3000] + [1] * 2001, cfg_id=5),
}

# Reduced shapes of the same five structures: small enough for the oracle to
# finish in seconds, still several tiles in every GEMM dimension and ragged
# per-expert row counts.
# The router weight scale grows as sqrt(H_full / H_small) so that router
# logits keep the spread they have at full size.
SMALL = {
    1: CONFIGS[1],
    2: CONFIGS[2].replace(name="v2lite_decode_bf16_small", T=96, H=256, E=16, I=192, shared_I=192,
                          wr_std=0.02 * math.sqrt(2048 / 256)),
    3: CONFIGS[3].replace(name="qwen3_prefill_fp8w_small", T=1024, H=512, E=32, I=256,
                          wr_std=0.02 * math.sqrt(2048 / 512)),
    4: CONFIGS[4].replace(name="r1_share_fp8w_small", T=512, H=1024, E=64, I=256,
                          expert_begin=0, expert_end=16, wr_std=0.02 * math.sqrt(7168 / 1024)),
    5: CONFIGS[5].replace(name="skewed_zipf_bf16_small", T=601, H=256, E=64, I=192,
                          seq_lens=_c5_seq_lens(601, 301), wr_std=0.02 * math.sqrt(2048 / 256)),
}


def get_config(cfg_id: int, small: bool = False) -> LayerConfig:
    return copy.deepcopy((SMALL if small else CONFIGS)[cfg_id])


def _gen(cfg: LayerConfig, seed: int, tid: int) -> torch.Generator:
    return torch.Generator().manual_seed((cfg.cfg_id * 1000 + seed) * 100 + tid)


def _to_store(t: torch.Tensor, dt: str) -> torch.Tensor:
    if dt == "f32":
        return t.contiguous()
    if dt == "bf16":
        return t.to(torch.bfloat16).contiguous()
    raise ValueError(dt)


def quantize_fp8_blocks(w: torch.Tensor):
    """Store a [R, C] fp32 matrix as OCP e4m3fn codes with one fp32 scale per
    128x128 block: s = amax/448 (1 for an all-zero block), code = RNE(w / s).

    Returns (codes uint8 [R, C], scales float32 [ceil(R/128), ceil(C/128)])."""
    R, C = w.shape
    rb, cb = -(-R // FP8_BLOCK), -(-C // FP8_BLOCK)
    pad = torch.zeros(rb * FP8_BLOCK, cb * FP8_BLOCK, dtype=torch.float32)
    pad[:R, :C] = w
    blk = pad.view(rb, FP8_BLOCK, cb, FP8_BLOCK)
    amax = blk.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blk / scale[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).view(rb * FP8_BLOCK, cb * FP8_BLOCK)
    return codes[:R, :C].contiguous(), scale.contiguous()


def _block_spread(g: torch.Generator, spread: float, rows: int, cols: int) -> torch.Tensor:
    """[rows, cols] factor 2^u, one u ~ U(-spread, spread) per 128x128 block."""
    rb, cb = -(-rows // FP8_BLOCK), -(-cols // FP8_BLOCK)
    u = (torch.rand(rb, cb, generator=g) * 2.0 - 1.0) * spread
    f = torch.pow(2.0, u)
    return f.repeat_interleave(FP8_BLOCK, 0).repeat_interleave(FP8_BLOCK, 1)[:rows, :cols]


def _expert_weights(cfg: LayerConfig, seed: int, tid: int, n_exp: int, rows: int, cols: int,
                    spread_tid: int = 0):
    g = _gen(cfg, seed, tid)
    if cfg.wdt == "fp8":
        gs = _gen(cfg, seed, spread_tid) if cfg.fp8_block_spread > 0 else None
        codes = torch.empty(n_exp, rows, cols, dtype=torch.uint8)
        scales = torch.empty(n_exp, -(-rows // FP8_BLOCK), -(-cols // FP8_BLOCK), dtype=torch.float32)
        for e in range(n_exp):
            w = torch.randn(rows, cols, generator=g) * cfg.w_std
            if gs is not None:
                w = w * _block_spread(gs, cfg.fp8_block_spread, rows, cols)
            codes[e], scales[e] = quantize_fp8_blocks(w)
        return codes, scales
    dt = torch.float32 if cfg.wdt == "f32" else torch.bfloat16
    out = torch.empty(n_exp, rows, cols, dtype=dt)
    for e in range(n_exp):
        out[e] = _to_store(torch.randn(rows, cols, generator=g) * cfg.w_std, cfg.wdt)
    return out, None


def make_inputs(cfg: LayerConfig, seed: int = 0, weights: bool = True) -> dict:
    """Draw every input of one layer call as CPU tensors.

    weights=False leaves out the expert weights (w13, w2, their scales and the
    shared experts: None / empty lists), for checks of routing and dispatch
    alone; the other tensors are the same draws as with weights.

    Keys: x [T,H]; w_router [E,H]; logit_bias [E] f32 or None; forced_ids [T,k]
    int32 or None; w13 [E_loc,2I,H] (gate rows [0,I), up rows [I,2I)); w2
    [E_loc,H,I]; w13_scale [E_loc,2I/128,H/128] / w2_scale [E_loc,H/128,I/128]
    (fp8 only, else None); shared_w13 / shared_w2: lists with one [2*I_sh,H] /
    [H,I_sh] tensor per shared expert (empty lists when there are none).
    """
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    if cfg.act == "f32":
        assert cfg.wdt == "f32"
    x = _to_store(torch.randn(T, H, generator=_gen(cfg, seed, TID_X)) * cfg.x_std, cfg.act)
    w_router = _to_store(torch.randn(E, H, generator=_gen(cfg, seed, TID_WR)) * cfg.wr_std, cfg.act)

    logit_bias = None
    if cfg.zipf_alpha > 0:
        perm = torch.randperm(E, generator=_gen(cfg, seed, TID_ZIPF))
        rank = torch.empty(E, dtype=torch.float64)
        rank[perm] = torch.arange(1, E + 1, dtype=torch.float64)
        p = rank.pow(-cfg.zipf_alpha)
        p = p / p.sum()
        bias = torch.log(p)
        bias[perm[-1]] = -1.0e4     # least popular expert is never chosen
        logit_bias = bias.to(torch.float32)

    forced_ids = None
    if cfg.forced_uniform:
        u = torch.rand(T, E, generator=_gen(cfg, seed, TID_FORCED))
        forced_ids = torch.argsort(u, dim=1)[:, :k].to(torch.int32).contiguous()

    w13 = w13_scale = w2 = w2_scale = None
    if weights:
        w13, w13_scale = _expert_weights(cfg, seed, TID_W13, cfg.E_loc, 2 * I, H, TID_W13_SPREAD)
        w2, w2_scale = _expert_weights(cfg, seed, TID_W2, cfg.E_loc, H, I, TID_W2_SPREAD)

    shared_w13, shared_w2 = [], []
    if cfg.n_shared > 0 and weights:
        sh_cfg = cfg.replace(wdt=cfg.act if cfg.wdt == "fp8" else cfg.wdt)
        a, _ = _expert_weights(sh_cfg, seed, TID_SH_W13, cfg.n_shared, 2 * cfg.shared_I, H)
        b, _ = _expert_weights(sh_cfg, seed, TID_SH_W2, cfg.n_shared, H, cfg.shared_I)
        shared_w13 = [a[i].contiguous() for i in range(cfg.n_shared)]
        shared_w2 = [b[i].contiguous() for i in range(cfg.n_shared)]

    return dict(cfg=cfg, seed=seed, x=x, w_router=w_router, logit_bias=logit_bias,
                forced_ids=forced_ids, w13=w13, w2=w2, w13_scale=w13_scale, w2_scale=w2_scale,
                shared_w13=shared_w13, shared_w2=shared_w2, seq_lens=cfg.seq_lens)


def bits(t: Optional[torch.Tensor]):
    """Raw stored values as numpy: bf16 -> uint16 bit patterns, fp8 codes ->
    uint8, f32 -> float32, int32 -> int32.  None passes through."""
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def oracle_view(inp: dict) -> dict:
    """The same inputs as numpy raw-bit arrays plus dtype tags, the form the
    oracle takes.  No arithmetic on values happens here."""
    cfg = inp["cfg"]
    return dict(
        cfg=cfg,
        x=bits(inp["x"]), act=cfg.act,
        w_router=bits(inp["w_router"]),
        logit_bias=bits(inp["logit_bias"]),
        forced_ids=bits(inp["forced_ids"]),
        w13=bits(inp["w13"]), w2=bits(inp["w2"]), wdt=cfg.wdt,
        w13_scale=bits(inp["w13_scale"]), w2_scale=bits(inp["w2_scale"]),
        shared_w13=[bits(t) for t in inp["shared_w13"]],
        shared_w2=[bits(t) for t in inp["shared_w2"]],
        shared_wdt=(cfg.act if cfg.wdt == "fp8" else cfg.wdt),
    )


__all__ = ["LayerConfig", "CONFIGS", "SMALL", "get_config", "make_inputs", "bits",
           "oracle_view", "quantize_fp8_blocks", "FP8_BLOCK"]
