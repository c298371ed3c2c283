"""Runs the HIP path through the C ABI on seeded inputs and returns numpy results.

Used by the GPU parity tests, the smoke check and nothing else.  Output
buffers are pre-filled with a poison byte so that tests can check which rows
were written; receive buffers get extra guard rows after the capacity.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

import combine_get_dispatch_07_amd as moe

POISON = 0x7B
GUARD_ROWS = 3


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _poison(d: Dict[str, Optional[torch.Tensor]]) -> None:
    """Fills every output with the poison byte; the workspace keeps its zero fill (the library
    requires a zero-filled workspace before its first use)."""
    for k, v in d.items():
        if v is not None and k != "workspace":
            v.view(torch.uint8).fill_(POISON)


class PathResult(dict):
    pass


def run_layout_dispatch(x: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray, E: int, R: int, dtype: str,
                        guard: int = GUARD_ROWS) -> PathResult:
    T, H = x.shape
    k = topk_idx.shape[1]
    shape = moe.MoeShape(T, H, k, E, R)
    xd = to_dev_bf16(x) if T else torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    idx_d = torch.from_numpy(np.ascontiguousarray(topk_idx, dtype=np.int32)).cuda()
    w_d = torch.from_numpy(np.ascontiguousarray(topk_w, dtype=np.float32)).cuda()
    lay = moe.alloc_layout(shape)
    _poison(lay)
    moe.run_layout(shape, idx_d, lay)
    cap = moe.max_recv_rows(shape)
    d = moe.alloc_dispatch(shape, dtype, capacity=cap + guard)
    _poison(d)
    moe.run_dispatch(shape, dtype, xd, idx_d, w_d, lay, d)
    torch.cuda.synchronize()
    r = PathResult()
    r["shape"] = shape
    r["cap"] = cap
    r["tokens_per_rank"] = lay["tokens_per_rank"].cpu().numpy()
    r["tokens_per_expert"] = lay["tokens_per_expert"].cpu().numpy()
    r["is_token_in_rank"] = lay["is_token_in_rank"].cpu().numpy()
    for key in ("recv_src_idx", "recv_topk_idx", "recv_topk_w", "rank_offsets", "send_row", "num_recv"):
        r[key] = d[key].cpu().numpy()
    if dtype == "bf16":
        r["recv_x"] = bf16_to_np(d["recv_x"])
    else:
        r["recv_x"] = d["recv_x"].cpu().numpy()
        r["recv_scales"] = d["recv_scales"].cpu().numpy()
    r["_dev"] = {"x": xd, "idx": idx_d, "w": w_d, "lay": lay, "d": d}
    return r


def run_combine(shape, y: np.ndarray, idx_d: torch.Tensor, w_d: torch.Tensor, send_row_d: torch.Tensor,
                num_y_rows: Optional[int] = None) -> np.ndarray:
    yd = to_dev_bf16(y) if y.shape[0] else torch.empty((0, shape.hidden), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((shape.num_tokens, shape.hidden), dtype=torch.bfloat16, device="cuda")
    out.view(torch.uint8).fill_(POISON)
    moe.moe_combine(shape, yd, idx_d, w_d, send_row_d, out, num_y_rows=num_y_rows)
    torch.cuda.synchronize()
    return bf16_to_np(out)


def run_dispatch_ll(x: np.ndarray, topk_idx: np.ndarray, E: int, cap: int, dtype: str) -> PathResult:
    T, H = x.shape
    k = topk_idx.shape[1]
    shape = moe.MoeShape(T, H, k, E, 1)
    xd = to_dev_bf16(x) if T else torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    idx_d = torch.from_numpy(np.ascontiguousarray(topk_idx, dtype=np.int32)).cuda()
    d = moe.alloc_dispatch_ll(shape, dtype, capacity=cap)
    _poison({k_: v for k_, v in d.items() if k_ != "workspace"})
    moe.run_dispatch_ll(shape, dtype, xd, idx_d, d)
    torch.cuda.synchronize()
    r = PathResult()
    r["shape"] = shape
    for key in ("recv_src_idx", "recv_count", "slot_pos"):
        r[key] = d[key].cpu().numpy()
    r["recv_x"] = bf16_to_np(d["recv_x"]) if dtype == "bf16" else d["recv_x"].cpu().numpy()
    if dtype == "fp8":
        r["recv_scales"] = d["recv_scales"].cpu().numpy()
    r["_dev"] = {"x": xd, "idx": idx_d, "d": d}
    return r


def run_combine_ll(shape, y: np.ndarray, idx_d: torch.Tensor, w: np.ndarray, slot_pos_d: torch.Tensor) -> np.ndarray:
    E, cap, H = y.shape
    yd = to_dev_bf16(y.reshape(E * cap, H)).view(E, cap, H) if y.size else \
        torch.empty((E, cap, H), dtype=torch.bfloat16, device="cuda")
    w_d = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).cuda()
    out = torch.empty((shape.num_tokens, H), dtype=torch.bfloat16, device="cuda")
    out.view(torch.uint8).fill_(POISON)
    moe.moe_combine_ll(shape, yd, idx_d, w_d, slot_pos_d, out)
    torch.cuda.synchronize()
    return bf16_to_np(out)


def run_route(logits: np.ndarray, k: int, E: int, R: int, gate: str = "softmax", num_groups: int = 1,
              topk_groups: int = 1, misalign: bool = False, H: int = 128) -> PathResult:
    """moe_route_layout on fp32 logits [T, E]; with ``misalign`` the logits start 4 bytes past a
    16-byte boundary (the scalar-load path)."""
    T = logits.shape[0]
    shape = moe.MoeShape(T, H, k, E, R)
    flat = np.ascontiguousarray(logits, dtype=np.float32).reshape(-1)
    if misalign:
        buf = torch.empty(flat.size + 4, dtype=torch.float32, device="cuda")
        buf[1:1 + flat.size].copy_(torch.from_numpy(flat))
        ld = buf[1:1 + flat.size].view(T, E)
    else:
        ld = torch.from_numpy(flat).cuda().view(T, E)
    lay = moe.alloc_route(shape)
    _poison(lay)
    moe.run_route(shape, ld, lay, gate, num_groups, topk_groups)
    torch.cuda.synchronize()
    r = PathResult()
    r["shape"] = shape
    for key in ("topk_idx", "topk_w", "tokens_per_rank", "tokens_per_expert", "is_token_in_rank"):
        r[key] = lay[key].cpu().numpy()
    r["_dev"] = {"logits": ld, "lay": lay}
    return r


def dispatch_with_plan(res: PathResult, x: np.ndarray, dtype: str = "bf16") -> PathResult:
    """moe_dispatch of x with the ids, weights and plan moe_route_layout produced."""
    shape = res["shape"]
    lay = res["_dev"]["lay"]
    xd = to_dev_bf16(x) if shape.num_tokens else torch.empty((0, shape.hidden), dtype=torch.bfloat16, device="cuda")
    d = moe.alloc_dispatch(shape, dtype)
    _poison(d)
    moe.run_dispatch(shape, dtype, xd, lay["topk_idx"], lay["topk_w"], lay, d)
    torch.cuda.synchronize()
    out = PathResult()
    for key in ("recv_src_idx", "recv_topk_idx", "recv_topk_w", "rank_offsets", "send_row", "num_recv"):
        out[key] = d[key].cpu().numpy()
    out["recv_x"] = bf16_to_np(d["recv_x"]) if dtype == "bf16" else d["recv_x"].cpu().numpy()
    return out


def run_route_dispatch(logits: np.ndarray, x: np.ndarray, k: int, E: int, R: int, dtype: str, gate: str = "softmax",
                       num_groups: int = 1, topk_groups: int = 1, guard: int = GUARD_ROWS, calls: int = 1,
                       lay=None) -> PathResult:
    """moe_route_dispatch (routing, layout and dispatch in one call) on fp32 logits [T, E] and bf16 x;
    `calls` back-to-back calls on the same buffers (the last one's outputs are returned); `lay` reuses
    an earlier result's workspace and routing buffers."""
    T, H = x.shape
    shape = moe.MoeShape(T, H, k, E, R)
    ld = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda().view(T, E)
    xd = to_dev_bf16(x) if T else torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    lay = moe.alloc_route(shape) if lay is None else lay
    _poison(lay)
    d = moe.alloc_dispatch(shape, dtype, capacity=moe.max_recv_rows(shape) + guard)
    _poison(d)
    for _ in range(calls):
        moe.run_route_dispatch(shape, dtype, ld, xd, lay, d, gate, num_groups, topk_groups)
    torch.cuda.synchronize()
    r = PathResult()
    r["shape"] = shape
    for key in ("topk_idx", "topk_w", "tokens_per_rank", "tokens_per_expert", "is_token_in_rank"):
        r[key] = lay[key].cpu().numpy()
    for key in ("recv_src_idx", "recv_topk_idx", "recv_topk_w", "rank_offsets", "send_row", "num_recv"):
        r[key] = d[key].cpu().numpy()
    r["recv_x"] = bf16_to_np(d["recv_x"]) if dtype == "bf16" else d["recv_x"].cpu().numpy()
    if dtype == "fp8":
        r["recv_scales"] = d["recv_scales"].cpu().numpy()
    r["_dev"] = {"logits": ld, "x": xd, "lay": lay, "d": d}
    return r
