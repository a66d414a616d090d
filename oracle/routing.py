"""Router logits, scores, top-k selection and routing weights (oracle).

The pages never state the routing rule; they only run models that route with
top-k (softmax top-k for DeepSeek-V2-Lite and Qwen3-30B-A3B, sigmoid scores
with group-limited top-k for DeepSeek-R1; "[Core/DBO][1/N]", Test Plan and
"[Perf] Fix DBO overlap ...", Test Plan) and replace the router's choice with
uniform random experts in the prefill benchmark ("[Perf] Fix DBO overlap ...",
Test Result, server command).  Readings, one each:

* logits:   l[t, e] = sum_h x[t, h] * W_r[e, h] + b[e]   (b = 0 unless given)
* softmax:  p = exp(l - max l) / sum exp(l - max l);  selection is on l
            (softmax is monotone), ordered by (value desc, index asc)
* sigmoid:  s = 1 / (1 + exp(-l)); group score = sum of the top-n s in each
            group of E/G consecutive experts; keep the topk_groups best groups
            (ties -> lower group index); select the k best s inside the kept
            groups (value desc, index asc)
* forced:   ids given per token, in the given order; weights are the softmax
            probabilities at those ids
* weights:  w_j = p[ids_j] (softmax) or s[ids_j] (sigmoid); optional
            renormalisation w_j /= sum_j w_j; then w_j *= routed_scale.
"""
import numpy as np


def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """l = x W_r^T (+ b), all float64.  x [T, H], w_router [E, H], bias [E]."""
    logits = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        logits = logits + np.asarray(bias, np.float64)[None, :]
    return logits


def softmax_rows(logits: np.ndarray) -> np.ndarray:
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def sigmoid(logits: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-logits))


def select_topk(values: np.ndarray, k: int) -> np.ndarray:
    """Row-wise k largest, ordered by (value desc, index asc).  A stable sort
    of -value keeps equal values in index order."""
    order = np.argsort(-values, axis=1, kind="stable")
    return order[:, :k]


def select_grouped(scores: np.ndarray, k: int, n_groups: int, topk_groups: int,
                   group_topn: int = 2) -> np.ndarray:
    """Group-limited top-k on per-expert scores [T, E].

    Experts form n_groups groups of E/n_groups consecutive indices.  A group's
    score is the sum of its group_topn largest expert scores; the topk_groups
    best groups are kept (ties -> lower group index); the k best experts of
    the kept groups are returned (value desc, index asc)."""
    T, E = scores.shape
    assert E % n_groups == 0
    per = E // n_groups
    grouped = scores.reshape(T, n_groups, per)
    top_in_group = np.sort(grouped, axis=2)[:, :, per - group_topn:]
    gscore = top_in_group.sum(axis=2)                                   # [T, G]
    kept = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_groups]  # [T, topk_groups]
    keep_mask = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(keep_mask, kept, True, axis=1)
    expert_keep = np.repeat(keep_mask, per, axis=1)                     # [T, E]
    masked = np.where(expert_keep, scores, -np.inf)
    return select_topk(masked, k)


def route(logits: np.ndarray, score: str, k: int, renormalize: bool = False,
          n_groups: int = 1, topk_groups: int = 1, group_topn: int = 2,
          routed_scale: float = 1.0, forced_ids=None):
    """Per-token expert ids [T, k] (int32) and weights [T, k] (float64)."""
    logits = np.asarray(logits, np.float64)
    if score == "softmax":
        probs = softmax_rows(logits)
        if forced_ids is not None:
            ids = np.asarray(forced_ids, np.int64)
        else:
            ids = select_topk(logits, k)
        w = np.take_along_axis(probs, ids, axis=1)
    elif score == "sigmoid":
        s = sigmoid(logits)
        if forced_ids is not None:
            ids = np.asarray(forced_ids, np.int64)
        elif n_groups > 1:
            ids = select_grouped(s, k, n_groups, topk_groups, group_topn)
        else:
            ids = select_topk(s, k)
        w = np.take_along_axis(s, ids, axis=1)
    else:
        raise ValueError(score)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    w = w * routed_scale
    return ids.astype(np.int32), w


def route_cfg(logits: np.ndarray, cfg, forced_ids=None):
    """route() with the parameters of a workloads.LayerConfig."""
    return route(logits, cfg.score, cfg.k, cfg.renormalize, cfg.n_groups, cfg.topk_groups,
                 cfg.group_topn, cfg.routed_scale, forced_ids)
