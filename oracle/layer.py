"""The whole MoE layer and its microbatch split (oracle).

The split: a batch is cut into two microbatches that run the same layer
("[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM", Purpose); a
request may straddle the cut, the second microbatch continuing it ("[Core/DBO]
[2/N] ... Prefill support", Purpose); an empty second microbatch must not
occur ("[Core/DBO][2/N]", commit log: guard for an empty second ubatch).
Readings: T0 = ceil(T/2) rows go to the first microbatch; below
min_tokens_to_split, or when a half would be empty, the layer runs unsplit.
Every step after the split acts per token, so the microbatched layer output
is the unsplit output stacked by rows.

Combine (stand-in for the all-to-all combine, same Purpose section):
out[t] = sum over j with a local expert of w[t, j] * y[t, j], plus the
always-on shared experts with weight 1; tokens with no local expert get 0.
"""
import numpy as np

from .numerics import decode, dequant_fp8_blocks
from .routing import router_logits, route_cfg
from .ffn import swiglu_expert
from .quant import swiglu_expert_fp8act


def _routed_expert(ov: dict):
    """The routed experts' FFN: bf16 activations, or fp8 activations when the
    call asks for them (ov["fp8_act"]); the shared experts always keep the
    activation dtype."""
    return swiglu_expert_fp8act if ov.get("fp8_act") else swiglu_expert


def split_point(T: int, min_tokens_to_split: int = 2, split_at: int = -1):
    """Rows of the first microbatch, or None when the layer is not split."""
    if T < max(2, min_tokens_to_split):
        return None
    T0 = (T + 1) // 2 if split_at < 0 else int(split_at)
    if T0 <= 0 or T0 >= T:
        return None
    return T0


def expert_weights(ov: dict, e_local: int):
    """Float64 (w13 [2I, H], w2 [H, I]) of local expert e_local."""
    if ov["wdt"] == "fp8":
        return (dequant_fp8_blocks(ov["w13"][e_local], ov["w13_scale"][e_local]),
                dequant_fp8_blocks(ov["w2"][e_local], ov["w2_scale"][e_local]))
    return decode(ov["w13"][e_local], ov["wdt"]), decode(ov["w2"][e_local], ov["wdt"])


def shared_weights(ov: dict):
    """Float64 (w13, w2) of every shared expert, in order."""
    return [(decode(a, ov["shared_wdt"]), decode(b, ov["shared_wdt"]))
            for a, b in zip(ov["shared_w13"], ov["shared_w2"])]


def _routing(ov: dict):
    cfg = ov["cfg"]
    x = decode(ov["x"], ov["act"])
    bias = None if ov["logit_bias"] is None else np.asarray(ov["logit_bias"], np.float64)
    logits = router_logits(x, decode(ov["w_router"], ov["act"]), bias)
    ids, w = route_cfg(logits, cfg, ov["forced_ids"])
    return x, logits, ids, w


def combine_ref(y_perm: np.ndarray, inv: np.ndarray, w: np.ndarray, shared_out=None,
                with_scale: bool = False):
    """out[t] = sum_j [inv[t*k+j] >= 0] w[t, j] * y_perm[inv[t*k+j]] (+ shared_out[t]).

    with_scale: also return sum_j |w[t, j] * y_perm[...]| (+ |shared_out[t]|),
    the magnitude of the summed terms."""
    T, k = w.shape
    H = y_perm.shape[1]
    out = np.zeros((T, H), np.float64)
    scale = np.zeros((T, H), np.float64)
    inv2 = np.asarray(inv).reshape(T, k)
    for t in range(T):
        for j in range(k):
            pos = int(inv2[t, j])
            if pos >= 0:
                term = float(w[t, j]) * y_perm[pos]
                out[t] += term
                scale[t] += np.abs(term)
    if shared_out is not None:
        out += shared_out
        scale += np.abs(shared_out)
    return (out, scale) if with_scale else out


def moe_layer_token(ov: dict, tokens=None) -> dict:
    """Literal per-token layer.  Routing covers every token; outputs are
    computed for `tokens` (default all) and returned in that order."""
    cfg = ov["cfg"]
    x, logits, ids, w = _routing(ov)
    T = x.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    shared = shared_weights(ov)
    cache = {}
    out = np.zeros((len(tokens), cfg.H), np.float64)
    for r, t in enumerate(tokens):
        for j in range(cfg.k):
            e = int(ids[t, j])
            if cfg.expert_begin <= e < cfg.expert_end:
                el = e - cfg.expert_begin
                if el not in cache:
                    cache[el] = expert_weights(ov, el)
                w13, w2 = cache[el]
                out[r] += float(w[t, j]) * _routed_expert(ov)(x[t:t + 1], w13, w2)[0]
        for w13, w2 in shared:
            out[r] += swiglu_expert(x[t:t + 1], w13, w2)[0]
    return dict(logits=logits, ids=ids, w=w, out=out, tokens=tokens)


def moe_layer_expert(ov: dict, tokens=None) -> dict:
    """The same layer grouped per expert (one expert's weights decoded at a
    time, float64 BLAS).  Same return form as moe_layer_token, plus `scale`:
    per output element, sum over the token's slots of |w| * (|h| |W2|^T) (and
    the shared experts' |h| |W2|^T), the magnitude of every term the element
    sums; |out| <= scale by the triangle inequality."""
    cfg = ov["cfg"]
    x, logits, ids, w = _routing(ov)
    T = x.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    sel_ids = ids[tokens]
    out = np.zeros((len(tokens), cfg.H), np.float64)
    scale = np.zeros_like(out)
    for el in range(cfg.E_loc):
        rows, slots = np.nonzero(sel_ids == el + cfg.expert_begin)
        if rows.size == 0:
            continue
        w13, w2 = expert_weights(ov, el)
        y, s = _routed_expert(ov)(x[tokens[rows]], w13, w2, with_scale=True)
        wr = w[tokens[rows], slots][:, None]
        np.add.at(out, rows, wr * y)
        np.add.at(scale, rows, np.abs(wr) * s)
    for w13, w2 in shared_weights(ov):
        y, s = swiglu_expert(x[tokens], w13, w2, with_scale=True)
        out += y
        scale += s
    return dict(logits=logits, ids=ids, w=w, out=out, scale=scale, tokens=tokens)


def slice_view(ov: dict, a: int, b: int) -> dict:
    """The inputs of rows [a, b) as a layer call of their own."""
    s = dict(ov)
    s["x"] = ov["x"][a:b]
    if ov["forced_ids"] is not None:
        s["forced_ids"] = ov["forced_ids"][a:b]
    s["cfg"] = ov["cfg"].replace(T=b - a)
    return s


def moe_layer_microbatched(ov: dict, min_tokens_to_split: int = 2, split_at: int = -1,
                           layer=moe_layer_expert) -> dict:
    """Split the batch, run the layer on each microbatch, stack the rows."""
    T = ov["cfg"].T
    T0 = split_point(T, min_tokens_to_split, split_at)
    if T0 is None:
        r = layer(ov)
        r["T0"] = None
        return r
    ra = layer(slice_view(ov, 0, T0))
    rb = layer(slice_view(ov, T0, T))
    r = {key: np.vstack([ra[key], rb[key]]) for key in ("logits", "ids", "w", "out", "scale") if key in ra}
    r.update(tokens=np.arange(T), T0=T0)
    return r
