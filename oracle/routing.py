"""Softmax top-k routing and the stable permutation of routed rows by expert.

Test infrastructure (see the package docstring).

"nf4moe - QLoRA for a 743B Fused-MoE", section "The fix: dequant-on-forward for
routed experts": the expert module receives top_k_index and top_k_weights [T, k]
from the router, builds a one-hot expert mask, and for every expert that was hit
gathers its tokens in token order (torch.where over the mask) and later adds the
expert output times the token's routing weight back with index_add_.

Readings: the router is softmax over all E experts followed by top-k, with no
renormalisation unless asked; equal logits go to the lower expert index.  The
routed pairs f = t*k + j are ordered by (expert, t, j), which is the order in
which the page's loop visits them.
"""
from __future__ import annotations

import numpy as np


def route(logits, k: int, renorm: bool = False):
    """fp32 logits [T, E] -> (topk_idx int32 [T, k], topk_w float64 [T, k]).

    Selection compares the float32 logits exactly: descending value, ties to
    the lower expert index.  Weights are the float64 softmax probabilities of
    the chosen experts (optionally divided by their sum).
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # lexsort: last key is primary -> sort by (-logit, index)
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -lg.astype(np.float64)), axis=1)
    idx = order[:, :k].astype(np.int32)
    l64 = lg.astype(np.float64)
    mx = l64.max(axis=1, keepdims=True)
    ex = np.exp(l64 - mx)
    p = ex / ex.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return idx, w


def permute(topk_idx, E: int):
    """Stable counting sort of the R = T*k routed pairs by expert.

    Returns perm [R] (perm[pos] = f = t*k + j), inv [R] (inv[f] = pos) and
    offsets [E+1] (exclusive prefix sum of the per-expert counts), all int32.
    """
    ti = np.asarray(topk_idx, dtype=np.int64)
    T, k = ti.shape
    flat = ti.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert index out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable")           # stable: keeps f order inside an expert
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return perm.astype(np.int32), inv.astype(np.int32), offsets.astype(np.int32)
