"""Top-k gating (the router) as the GPU fuses it with the dispatch layout (test infrastructure only).

Only ``tests/``, the smoke check and the benchmark's CPU baseline use this module.

Page cited: [overlap notes] "DeepEP：年度总结中的计算通信重叠摘记" (notes.kuangjux.top).  Its
section 节点内通信 says DeepEP runs the top-k computation together with the sparse exchange so
that no CPU step sits between them; its section 计算-通信重叠 says DeepEP was designed around
DeepSeek's group-limited gating.  The pages give no formula for either; the readings taken
(numbered after those of ``moe_oracle``):

13. selection: the k largest logits, ties going to the lower expert id, in descending order of
    logit; that order is the slot order j = 0..k-1.  -0.0 and +0.0 are equal logits;
14. group-limited gating: the E experts form G equal contiguous groups; a group's score is the
    largest logit in it; the ``topk_groups`` best groups are kept (ties to the lower group id)
    and selection happens among the experts of kept groups only;
15. weights: softmax over the k selected logits, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), or
    the sigmoid gate normalised over the k selected, w_j = s(l_j) / sum_i s(l_i) with
    s(x) = 1 / (1 + e^-x); computed here in fp64 (sums in slot order) and rounded to fp32.

Selection depends only on comparisons of the fp32 logits, so it is exact and the GPU must match it
bit for bit; the weights involve exp, so the GPU is compared with these fp64-derived values within a
stated tolerance.  Logits must be finite (NaN has no place in an ordering).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def group_mask(logits: np.ndarray, num_groups: int, topk_groups: int) -> np.ndarray:
    """bool [T, E]: experts in the kept groups (reading 14)."""
    T, E = logits.shape
    S = E // num_groups
    score = logits.reshape(T, num_groups, S).max(axis=2)
    # rank groups by (-score, group id); lexsort keys are given last-key-primary
    order = np.lexsort((np.broadcast_to(np.arange(num_groups), score.shape), -score.astype(np.float64)), axis=1)
    keep = np.zeros((T, num_groups), dtype=bool)
    np.put_along_axis(keep, order[:, :topk_groups], True, axis=1)
    return np.repeat(keep, S, axis=1)


def route(logits: np.ndarray, k: int, gate: str = "softmax", num_groups: int = 1, topk_groups: int = 1
          ) -> Tuple[np.ndarray, np.ndarray]:
    """topk_idx int32 [T, k] (slot order) and topk_w float32 [T, k] (readings 13-15)."""
    x = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = x.shape
    assert np.isfinite(x).all(), "logits must be finite"
    assert E % num_groups == 0 and 1 <= topk_groups <= num_groups
    assert 1 <= k <= (E // num_groups) * topk_groups, "fewer allowed experts than k"
    allowed = group_mask(x, num_groups, topk_groups) if num_groups > 1 else np.ones((T, E), dtype=bool)
    key = np.where(allowed, -x.astype(np.float64), np.inf)
    ids = np.broadcast_to(np.arange(E), x.shape)
    order = np.lexsort((ids, key), axis=1)[:, :k]  # ascending (-logit, id)
    sel = np.take_along_axis(x, order, axis=1).astype(np.float64)
    if gate == "softmax":
        e = np.exp(sel - sel[:, :1])
    elif gate == "sigmoid":
        e = 1.0 / (1.0 + np.exp(-sel))
    else:
        raise ValueError(gate)
    w = e / np.cumsum(e, axis=1)[:, -1:]
    return order.astype(np.int32), w.astype(np.float32)


def route_bruteforce(logits, k: int, gate: str = "softmax", num_groups: int = 1, topk_groups: int = 1):
    """The same selection by repeated scans over plain Python lists (tiny inputs)."""
    import math

    out_idx, out_w = [], []
    for row in np.asarray(logits, dtype=np.float32).tolist():
        E = len(row)
        S = E // num_groups
        allowed = [True] * E
        if num_groups > 1:
            scores = [max(row[g * S:(g + 1) * S]) for g in range(num_groups)]
            kept = []
            for _ in range(topk_groups):
                best = None
                for g in range(num_groups):
                    if g not in kept and (best is None or scores[g] > scores[best]):
                        best = g
                kept.append(best)
            allowed = [e // S in kept for e in range(E)]
        chosen = []
        for _ in range(k):
            best = None
            for e in range(E):
                if allowed[e] and e not in chosen and (best is None or row[e] > row[best]):
                    best = e
            chosen.append(best)
        vals = [row[e] for e in chosen]
        if gate == "softmax":
            ex = [math.exp(v - vals[0]) for v in vals]
        else:
            ex = [1.0 / (1.0 + math.exp(-v)) for v in vals]
        tot = 0.0
        for v in ex:
            tot += v
        out_idx.append(chosen)
        out_w.append([float(np.float32(v / tot)) for v in ex])
    return out_idx, out_w
