"""Seeded synthetic inputs for MoE expert-parallel dispatch layout, dispatch and combine.

This module only *draws* inputs: bf16 hidden rows, router logits turned into
top-k expert ids with their gate weights, and bf16 expert outputs.  It holds
none of the layout, dispatch or combine arithmetic.  Both the CPU oracle
(``oracle/``) and the HIP library are fed from here, and neither is imported.

Routing is input synthesis, not part of the hot path: the DeepEP pages describe
the communication kernels as consuming top-k expert ids produced by a gate
(DeepEP overview notes, "intranode communication": top-k is fused with the
sparse exchange), and the group-limited gate it was built to match ("overview":
DeepSeek's group-limited gating).  The five workloads below are the five
configurations this library is measured on; their routing recipes are:

* selection: stable sort of fp32 logits by (-logit, expert id), so ties go to
  the lower id; keep the first k;
* weights: computed in fp64 from the selected logits, then rounded to fp32:
  softmax over the k selected, or sigmoid normalised over the k selected;
* group-limited: group score = max logit of the group, keep the top groups
  (ties -> lower group id), then top-k among the experts of kept groups;
* Zipf skew: logit[t, e] = -s * ln(pos(e)) + Gumbel(0, 1), pos a seeded
  1-based permutation of the experts.  Gumbel-top-k is Plackett-Luce sampling
  without replacement, so the first pick is exactly Zipf(s).

The GPU gate (top-k fused with the layout) is a method step of its own: it is
checked against ``oracle/router.py`` on the logits drawn here
(:func:`config_logits`), never against the routing code of this module, which
only synthesises ids and weights for the layout, dispatch and combine steps.

Bit patterns of bf16 are carried as ``numpy.uint16``; fp32 -> bf16 uses torch's
round-to-nearest-even conversion (a library routine).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

ROOT_SEED = 0xC0DE

__all__ = [
    "Config",
    "CONFIGS",
    "CONFIG_BY_NAME",
    "seed_streams",
    "bf16_bits_from_f32",
    "draw_hidden",
    "draw_expert_outputs",
    "draw_logits",
    "config_logits",
    "route",
    "make_inputs",
    "random_case",
]


@dataclass(frozen=True)
class Config:
    """One workload: shapes, routing recipe and dispatch precision."""

    name: str
    index: int  # seed index: SeedSequence([ROOT_SEED, index])
    num_tokens: int
    hidden: int
    num_experts: int
    num_topk: int
    num_ranks: int
    dispatch_dtype: str  # "bf16" or "fp8"
    routing: str  # "softmax" | "sigmoid" | "group_limited" | "zipf"
    combine_input: str  # "identity" (y = dequantised recv rows) or "random" (y ~ N(0,1) bf16)
    num_groups: int = 0
    topk_groups: int = 0
    zipf_s: float = 0.0

    @property
    def experts_per_rank(self) -> int:
        return self.num_experts // self.num_ranks

    @property
    def capacity(self) -> int:
        """Worst-case receive rows: every token to min(k, R) distinct ranks."""
        return self.num_tokens * min(self.num_topk, self.num_ranks)


CONFIGS: List[Config] = [
    Config("tiny", 0, 64, 256, 16, 4, 4, "bf16", "softmax", "identity"),
    Config("decode", 1, 128, 7168, 256, 8, 8, "fp8", "sigmoid", "random"),
    Config("prefill", 2, 4096, 7168, 256, 8, 8, "bf16", "softmax", "random"),
    Config("group_limited", 3, 4096, 7168, 256, 8, 64, "fp8", "group_limited", "random",
           num_groups=8, topk_groups=4),
    Config("skewed", 4, 16384, 7168, 256, 8, 32, "fp8", "zipf", "random", zipf_s=1.2),
]
CONFIG_BY_NAME: Dict[str, Config] = {c.name: c for c in CONFIGS}


def seed_streams(index: int) -> Tuple[np.random.Generator, ...]:
    """Four independent generators (x, router, y, extra) for workload ``index``."""
    children = np.random.SeedSequence([ROOT_SEED, index]).spawn(4)
    return tuple(np.random.default_rng(c) for c in children)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even, via torch."""
    import torch

    a = np.ascontiguousarray(a, dtype=np.float32)
    t = torch.from_numpy(a).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _normal_bf16(gen: np.random.Generator, rows: int, cols: int, chunk_rows: int = 8192) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = bf16_bits_from_f32(gen.standard_normal((r1 - r0, cols), dtype=np.float32))
    return out


def draw_hidden(gen: np.random.Generator, num_tokens: int, hidden: int) -> np.ndarray:
    """Token hidden rows: fp32 N(0,1) rounded to bf16; uint16 bits [T, H]."""
    return _normal_bf16(gen, num_tokens, hidden)


def draw_expert_outputs(gen: np.random.Generator, num_rows: int, hidden: int) -> np.ndarray:
    """Expert outputs for combine: fp32 N(0,1) rounded to bf16; uint16 bits [rows, H]."""
    return _normal_bf16(gen, num_rows, hidden)


def _stable_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per row; equal scores keep the lower index first."""
    order = np.argsort(-scores, axis=1, kind="stable")
    return order[:, :k]


def _softmax_selected(sel_logits: np.ndarray) -> np.ndarray:
    z = sel_logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32)


def _sigmoid_normalised(sel_logits: np.ndarray) -> np.ndarray:
    s = 1.0 / (1.0 + np.exp(-sel_logits.astype(np.float64)))
    return (s / s.sum(axis=1, keepdims=True)).astype(np.float32)


def draw_logits(cfg: Config, gen_router: np.random.Generator, gen_extra: np.random.Generator,
                num_tokens: Optional[int] = None) -> np.ndarray:
    """Router logits fp32 [T, E] for ``cfg`` (N(0,1), or the Zipf-skewed Gumbel form)."""
    T = cfg.num_tokens if num_tokens is None else num_tokens
    E = cfg.num_experts
    if cfg.routing == "zipf":
        perm = gen_extra.permutation(E)
        pos = np.empty(E, dtype=np.float64)
        pos[perm] = np.arange(1, E + 1, dtype=np.float64)
        u = gen_router.random((T, E))
        u = np.clip(u, np.finfo(np.float64).tiny, 1.0 - 2.0 ** -53)
        gumbel = -np.log(-np.log(u))
        return (-cfg.zipf_s * np.log(pos)[None, :] + gumbel).astype(np.float32)
    return gen_router.standard_normal((T, E), dtype=np.float32)


def config_logits(cfg: Config, num_tokens: Optional[int] = None) -> np.ndarray:
    """The logits :func:`make_inputs` routes for ``cfg`` (drawn for ``num_tokens`` tokens if given)."""
    _g_x, g_router, _g_y, g_extra = seed_streams(cfg.index)
    return draw_logits(cfg, g_router, g_extra, num_tokens)


def route(cfg: Config, gen_router: np.random.Generator, gen_extra: np.random.Generator,
          num_tokens: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k expert ids (int32 [T, k]) and gate weights (fp32 [T, k]) for ``cfg``."""
    T = cfg.num_tokens if num_tokens is None else num_tokens
    E, k = cfg.num_experts, cfg.num_topk
    logits = draw_logits(cfg, gen_router, gen_extra, T)

    if cfg.routing == "group_limited":
        G = cfg.num_groups
        per_group = E // G
        group_score = logits.reshape(T, G, per_group).max(axis=2)
        keep = _stable_topk(group_score, cfg.topk_groups)
        allowed = np.zeros((T, G), dtype=bool)
        np.put_along_axis(allowed, keep, True, axis=1)
        masked = np.where(np.repeat(allowed, per_group, axis=1), logits, np.float32(-np.inf))
        idx = _stable_topk(masked, k)
    else:
        idx = _stable_topk(logits, k)

    sel = np.take_along_axis(logits, idx, axis=1)
    if cfg.routing == "sigmoid":
        w = _sigmoid_normalised(sel)
    else:
        w = _softmax_selected(sel)
    return idx.astype(np.int32), w.astype(np.float32)


def make_inputs(cfg: Config) -> Dict[str, np.ndarray]:
    """x (bf16 bits [T,H]), topk_idx (int32 [T,k]) and topk_w (fp32 [T,k]) for ``cfg``.

    Expert outputs are drawn separately with :func:`draw_expert_outputs` from the
    ``y`` stream once the caller knows how many receive rows it needs.
    """
    g_x, g_router, _g_y, g_extra = seed_streams(cfg.index)
    x = draw_hidden(g_x, cfg.num_tokens, cfg.hidden)
    idx, w = route(cfg, g_router, g_extra)
    return {"x": x, "topk_idx": idx, "topk_w": w}


def y_stream(cfg: Config) -> np.random.Generator:
    """The generator that expert outputs for ``cfg`` are drawn from."""
    return seed_streams(cfg.index)[2]


def random_case(seed: int, num_tokens: int, hidden: int, num_experts: int, num_topk: int,
                num_ranks: int, invalid_frac: float = 0.0, routing: str = "softmax") -> Dict[str, np.ndarray]:
    """A small random case for edge-case sweeps.

    Top-k of N(0,1) logits (distinct ids per token); then a fraction of the
    slots is replaced by out-of-range ids (-1 or >= E), which every step must skip.
    """
    cfg = Config("random", 1000 + seed, num_tokens, hidden, num_experts, num_topk, num_ranks,
                 "bf16", routing, "random")
    g_x, g_router, _g_y, g_extra = seed_streams(cfg.index)
    x = draw_hidden(g_x, num_tokens, hidden)
    idx, w = route(cfg, g_router, g_extra)
    if invalid_frac > 0.0 and idx.size:
        drop = g_extra.random(idx.shape) < invalid_frac
        bad = np.where(g_extra.random(idx.shape) < 0.5, -1, num_experts + 3).astype(np.int32)
        idx = np.where(drop, bad, idx).astype(np.int32)
    return {"x": x, "topk_idx": idx, "topk_w": w}


def with_tokens(cfg: Config, num_tokens: int) -> Config:
    """The same workload recipe at another token count."""
    return replace(cfg, num_tokens=num_tokens)
