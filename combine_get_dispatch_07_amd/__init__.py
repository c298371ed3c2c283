"""MI355X (gfx950) MoE expert-parallel dispatch layout, dispatch and combine.

The compute is the C-ABI library ``libmoe_ep.so`` (HIP kernels, see
``include/moe_ep.h``); this package is its thin Python binding plus helpers
that allocate output buffers with torch (device memory only).

    from combine_get_dispatch_07_amd import MoeShape, alloc_layout, alloc_dispatch, \
        moe_get_dispatch_layout, moe_dispatch, moe_combine
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from ._lib import (LIB_PATH, MoeError, MoeShape, ll_workspace_bytes, max_recv_rows, moe_combine,  # noqa: F401
                   moe_combine_backward, moe_combine_ll, moe_dispatch, moe_dispatch_backward, moe_dispatch_ll,
                   moe_encode_e4m3, moe_layout_dispatch, moe_layout_dispatch_noalloc, Prepared,
                   moe_get_dispatch_layout, moe_route_dispatch, moe_route_layout, status_string, stream_create_cu_range,
                   stream_destroy,
                   workspace_bytes)


def alloc_layout(shape: MoeShape, device="cuda") -> Dict[str, torch.Tensor]:
    """Outputs of moe_get_dispatch_layout, plus the workspace (the dispatch plan)."""
    return {
        "tokens_per_rank": torch.empty(shape.num_ranks, dtype=torch.int32, device=device),
        "tokens_per_expert": torch.empty(shape.num_experts, dtype=torch.int32, device=device),
        "is_token_in_rank": torch.empty((shape.num_tokens, shape.num_ranks), dtype=torch.uint8, device=device),
        # zero-filled once: its first words coordinate the blocks of a launch and every call
        # leaves them zero again
        "workspace": torch.zeros(workspace_bytes(shape), dtype=torch.uint8, device=device),
    }


def alloc_route(shape: MoeShape, device="cuda") -> Dict[str, torch.Tensor]:
    """Outputs of moe_route_layout: the routing (ids, weights) plus everything alloc_layout holds."""
    lay = alloc_layout(shape, device)
    lay["topk_idx"] = torch.empty((shape.num_tokens, shape.num_topk), dtype=torch.int32, device=device)
    lay["topk_w"] = torch.empty((shape.num_tokens, shape.num_topk), dtype=torch.float32, device=device)
    return lay


def run_route(shape: MoeShape, logits: torch.Tensor, lay: Dict[str, torch.Tensor], gate: str = "softmax",
              num_groups: int = 1, topk_groups: int = 1, stream=None) -> None:
    """moe_route_layout: top-k routing of `logits` [T, E] fp32 ("softmax" or "sigmoid" gate, optional
    group limit) fused with the layout; fills lay's ids, weights, counts, mask and plan."""
    moe_route_layout(shape, logits, lay["topk_idx"], lay["topk_w"], lay["tokens_per_rank"], lay["tokens_per_expert"],
                     lay["is_token_in_rank"], lay["workspace"], gate, num_groups, topk_groups, stream)


def alloc_dispatch(shape: MoeShape, dtype: str, device="cuda", capacity: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Outputs of moe_dispatch at the worst-case capacity T * min(k, R) (allocated once, reused)."""
    cap = max_recv_rows(shape) if capacity is None else capacity
    H, k = shape.hidden, shape.num_topk
    fp8 = dtype == "fp8"
    return {
        "recv_x": torch.empty((cap, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=device),
        "recv_scales": torch.empty((cap, H // 128), dtype=torch.float32, device=device) if fp8 else None,
        "recv_src_idx": torch.empty(cap, dtype=torch.int32, device=device),
        "recv_topk_idx": torch.empty((cap, k), dtype=torch.int32, device=device),
        "recv_topk_w": torch.empty((cap, k), dtype=torch.float32, device=device),
        "rank_offsets": torch.empty(shape.num_ranks + 1, dtype=torch.int32, device=device),
        "send_row": torch.empty((shape.num_tokens, shape.num_ranks), dtype=torch.int32, device=device),
        "num_recv": torch.empty(1, dtype=torch.int32, device=device),
    }


def run_layout(shape: MoeShape, topk_idx: torch.Tensor, lay: Dict[str, torch.Tensor], stream=None) -> None:
    """moe_get_dispatch_layout: counts, is_token_in_rank and the dispatch plan into `lay`."""
    moe_get_dispatch_layout(shape, topk_idx, lay["tokens_per_rank"], lay["tokens_per_expert"],
                            lay["is_token_in_rank"], lay["workspace"], stream)


def run_dispatch(shape: MoeShape, dtype: str, x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                 lay: Dict[str, torch.Tensor], d: Dict[str, torch.Tensor], stream=None) -> None:
    """moe_dispatch: rows of `x` packed into d's receive buffers, from the plan in lay["workspace"]."""
    moe_dispatch(shape, dtype, x, topk_idx, topk_w, lay["workspace"], d["recv_x"], d["recv_scales"],
                 d["recv_src_idx"], d["recv_topk_idx"], d["recv_topk_w"], d["rank_offsets"], d["send_row"],
                 d["num_recv"], stream)


def run_layout_dispatch(shape: MoeShape, dtype: str, x: torch.Tensor, topk_idx: torch.Tensor,
                        topk_w: torch.Tensor, lay: Dict[str, torch.Tensor], d: Dict[str, torch.Tensor],
                        stream=None) -> None:
    """run_layout then run_dispatch as one call (one kernel for small batches)."""
    moe_layout_dispatch(shape, dtype, x, topk_idx, topk_w, lay["tokens_per_rank"], lay["tokens_per_expert"],
                        lay["is_token_in_rank"], lay["workspace"], d["recv_x"], d["recv_scales"], d["recv_src_idx"],
                        d["recv_topk_idx"], d["recv_topk_w"], d["rank_offsets"], d["send_row"], d["num_recv"],
                        stream)


def run_route_dispatch(shape: MoeShape, dtype: str, logits: torch.Tensor, x: torch.Tensor,
                       lay: Dict[str, torch.Tensor], d: Dict[str, torch.Tensor], gate: str = "softmax",
                       num_groups: int = 1, topk_groups: int = 1, stream=None, prepare: bool = False):
    """run_route then run_dispatch as one call (one kernel up to 1024 tokens); `lay` from alloc_route."""
    return moe_route_dispatch(shape, dtype, logits, x, lay["topk_idx"], lay["topk_w"], lay["tokens_per_rank"],
                              lay["tokens_per_expert"], lay["is_token_in_rank"], lay["workspace"], d["recv_x"],
                              d["recv_scales"], d["recv_src_idx"], d["recv_topk_idx"], d["recv_topk_w"],
                              d["rank_offsets"], d["send_row"], d["num_recv"], gate, num_groups, topk_groups, stream,
                              prepare)


def prepare_layout(shape: MoeShape, topk_idx: torch.Tensor, lay: Dict[str, torch.Tensor]) -> Prepared:
    """run_layout with its arguments checked once: returns a call taking only the stream."""
    return moe_get_dispatch_layout(shape, topk_idx, lay["tokens_per_rank"], lay["tokens_per_expert"],
                                   lay["is_token_in_rank"], lay["workspace"], prepare=True)


def prepare_dispatch(shape: MoeShape, dtype: str, x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                     lay: Dict[str, torch.Tensor], d: Dict[str, torch.Tensor]) -> Prepared:
    """run_dispatch with its arguments checked once."""
    return moe_dispatch(shape, dtype, x, topk_idx, topk_w, lay["workspace"], d["recv_x"], d["recv_scales"],
                        d["recv_src_idx"], d["recv_topk_idx"], d["recv_topk_w"], d["rank_offsets"], d["send_row"],
                        d["num_recv"], prepare=True)


def prepare_layout_dispatch(shape: MoeShape, dtype: str, x: torch.Tensor, topk_idx: torch.Tensor,
                            topk_w: torch.Tensor, lay: Dict[str, torch.Tensor], d: Dict[str, torch.Tensor]) -> Prepared:
    """run_layout_dispatch with its arguments checked once."""
    return moe_layout_dispatch(shape, dtype, x, topk_idx, topk_w, lay["tokens_per_rank"], lay["tokens_per_expert"],
                               lay["is_token_in_rank"], lay["workspace"], d["recv_x"], d["recv_scales"],
                               d["recv_src_idx"], d["recv_topk_idx"], d["recv_topk_w"], d["rank_offsets"],
                               d["send_row"], d["num_recv"], prepare=True)


def prepare_combine(shape: MoeShape, y: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                    send_row: torch.Tensor, out: torch.Tensor) -> Prepared:
    """moe_combine with its arguments checked once."""
    return moe_combine(shape, y, topk_idx, topk_w, send_row, out, prepare=True)


def alloc_dispatch_ll(shape: MoeShape, dtype: str, device="cuda", capacity: Optional[int] = None
                      ) -> Dict[str, torch.Tensor]:
    """Outputs and workspace of moe_dispatch_ll; per-expert capacity defaults to T."""
    cap = shape.num_tokens if capacity is None else capacity
    E, H = shape.num_experts, shape.hidden
    fp8 = dtype == "fp8"
    return {
        "recv_x": torch.empty((E, cap, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=device),
        "recv_scales": torch.empty((E, cap, H // 128), dtype=torch.float32, device=device) if fp8 else None,
        "recv_src_idx": torch.empty((E, cap), dtype=torch.int32, device=device),
        "recv_count": torch.empty(E, dtype=torch.int32, device=device),
        "slot_pos": torch.empty((shape.num_tokens, shape.num_topk), dtype=torch.int32, device=device),
        "workspace": torch.empty(ll_workspace_bytes(shape), dtype=torch.uint8, device=device),
    }


def run_dispatch_ll(shape: MoeShape, dtype: str, x: torch.Tensor, topk_idx: torch.Tensor,
                    d: Dict[str, torch.Tensor], stream=None) -> None:
    """moe_dispatch_ll: one receive buffer per expert, positions and counts into `d`."""
    moe_dispatch_ll(shape, dtype, x, topk_idx, d["workspace"], d["recv_x"], d["recv_scales"], d["recv_src_idx"],
                    d["recv_count"], d["slot_pos"], stream)
