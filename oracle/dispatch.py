"""Dispatch reference (oracle): the single-GPU stand-in for the all-to-all
dispatch of "[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM",
Purpose (dispatch -> experts -> combine), with device-resident per-expert
counts and a worst-case capacity of tokens x k rows ("DeepEP HT: full decode
CUDA graphs via worst-token dispatch", bot reviews 1 and 2).

Reading: the (token, slot) pairs of a microbatch are numbered p = t * k + j;
only pairs whose expert lies in the local range [e_begin, e_end) are
dispatched; they are counting-sorted by local expert, stable in p.
"""
import numpy as np


def dispatch_ref(ids: np.ndarray, e_begin: int, e_end: int, tile_m: int = 0):
    """ids [T, k] int -> dict(counts [E_loc], offsets [E_loc+1],
    perm [M] (sorted position -> p), inv [T*k] (p -> position or -1),
    tile_offsets [E_loc+1] (tiles of tile_m rows per expert; zeros if tile_m
    is 0), M)."""
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    E_loc = e_end - e_begin
    local = (flat >= e_begin) & (flat < e_end)
    p_local = np.nonzero(local)[0]
    le = flat[p_local] - e_begin
    counts = np.bincount(le, minlength=E_loc).astype(np.int64)
    offsets = np.zeros(E_loc + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(le, kind="stable")
    perm = p_local[order]
    M = perm.shape[0]
    inv = np.full(T * k, -1, np.int64)
    inv[perm] = np.arange(M)
    tile_offsets = np.zeros(E_loc + 1, np.int64)
    if tile_m > 0:
        tile_offsets[1:] = np.cumsum((counts + tile_m - 1) // tile_m)
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                perm=perm.astype(np.int32), inv=inv.astype(np.int32),
                tile_offsets=tile_offsets.astype(np.int32), M=int(M))
