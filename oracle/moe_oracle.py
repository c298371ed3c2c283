"""Vectorised numpy oracle for dispatch layout, dispatch and combine (test infrastructure only).

What is computed, and which passage each step follows
-----------------------------------------------------
Pages cited (titles as they appear on the pages):

* [overlap notes] "DeepEP：年度总结中的计算通信重叠摘记" (notes.kuangjux.top), section
  节点内通信 (intranode communication): a token is sent only to the ranks that
  own one of its top-k experts, recorded in an ``is_token_in_rank`` matrix
  instead of a dense all-to-all; dispatch may carry FP8 (2 bytes -> 1 byte);
  dispatch and combine are the two exchange steps measured there.
* [rocSHMEM notes] mlqm.cn page on rocSHMEM and the RDMA buffer, section 3.2
  (RDMA buffer 的问题): the communication buffer holds the packed rows bound
  for other ranks and the rows received from them, is reused as the combine
  workspace, is allocated once, and must be sized for the worst case.
* [DeepEP overview] "DeepEP：面向MoE的高吞吐低延迟GPU通信库" (ssnai.com): dispatch and
  combine kernels for expert parallelism, with FP8 support.

The pages leave the following open; the readings taken here are the plainest
ones the rest supports:

1. expert e lives on rank floor(e / L), L = E / R experts per rank;
2. ids outside [0, E) are masked: skipped by every step;
3. one receive row per (token, distinct destination rank), not per expert;
4. receive segments are in ascending rank order, rows inside a segment in
   ascending source-token order (stable), at offsets given by an exclusive
   prefix sum of the per-rank token counts;
5. receive-side expert ids are local (e - r*L) or -1, with weight +0.0 for -1;
6. FP8 is OCP E4M3 "fn" with one fp32 dequantisation scale per (row,
   128-channel block): a = max |x| over the block, s = fl32(max(a, 1e-4) / 448),
   q = E4M3_RNE(fl32(x / s));
7. combine is, per token and channel, an fp32 sum in ascending slot order of
   fl32(w_j * y_j) (multiply then add, no fused multiply-add), rounded to bf16
   to nearest-even; tokens with no valid slot give +0.

Precision: the method fixes fp32 for scales and accumulation (the workloads
state fp32 scales and an fp32-accumulated combine), so this oracle computes in
fp32 with numpy's IEEE single-precision operations; ``combine_f64`` gives the
fp64 value the fp32 sum approximates, for error bounds.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

from .numerics import bf16_bits_to_f32, e4m3_encode_rne, e4m3_decode, f32_to_bf16_bits_rne

FP8_BLOCK = 128
AMAX_FLOOR = np.float32(1e-4)
E4M3_MAX = np.float32(448.0)


def _check(topk_idx: np.ndarray, num_experts: int, num_ranks: int) -> int:
    assert topk_idx.ndim == 2
    assert num_ranks >= 1 and num_experts % num_ranks == 0
    return num_experts // num_ranks


def expert_ranks(topk_idx: np.ndarray, num_experts: int, num_ranks: int) -> Tuple[np.ndarray, np.ndarray]:
    """(valid, rank) per slot: valid <=> 0 <= e < E; rank = floor(e / L) (reading 1, 2)."""
    L = _check(topk_idx, num_experts, num_ranks)
    e = topk_idx.astype(np.int64)
    valid = (e >= 0) & (e < num_experts)
    rank = np.where(valid, e // L, -1)
    return valid, rank


def get_dispatch_layout(topk_idx: np.ndarray, num_experts: int, num_ranks: int
                        ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Dispatch layout [overlap notes, intranode communication: the is_token_in_rank filter].

    Returns ``tokens_per_rank`` int32[R], ``tokens_per_expert`` int32[E] and
    ``is_token_in_rank`` uint8[T, R] (0/1):

    * tokens_per_expert[e] = number of (t, j) slots with topk_idx[t, j] == e;
    * is_token_in_rank[t, r] = 1 iff some valid slot of token t has rank r;
    * tokens_per_rank[r] = sum over t of is_token_in_rank[t, r].
    """
    T = topk_idx.shape[0]
    valid, rank = expert_ranks(topk_idx, num_experts, num_ranks)
    ids = topk_idx[valid].astype(np.int64)
    tokens_per_expert = np.bincount(ids, minlength=num_experts).astype(np.int32)
    mask = np.zeros((T, num_ranks), dtype=np.uint8)
    t_of_slot = np.broadcast_to(np.arange(T)[:, None], topk_idx.shape)
    mask[t_of_slot[valid], rank[valid]] = 1
    tokens_per_rank = mask.sum(axis=0, dtype=np.int64).astype(np.int32)
    return tokens_per_rank, tokens_per_expert, mask


def assign_slots(is_token_in_rank: np.ndarray) -> Tuple[np.ndarray, np.ndarray, int]:
    """Receive-row assignment [rocSHMEM notes, 3.2: packed rows in a preallocated buffer] (reading 3, 4).

    rank_offsets int32[R+1] = exclusive prefix sum of per-rank counts;
    send_row int32[T, R] = rank_offsets[r] + #{t' < t : mask[t', r]} where the
    token goes to r, else -1; num_recv = rank_offsets[R].
    """
    m = is_token_in_rank.astype(np.int64) != 0
    counts = m.sum(axis=0)
    rank_offsets = np.zeros(m.shape[1] + 1, dtype=np.int64)
    rank_offsets[1:] = np.cumsum(counts)
    before = np.cumsum(m, axis=0) - m  # tokens t' < t going to r
    send_row = np.where(m, rank_offsets[None, :-1] + before, -1)
    return rank_offsets.astype(np.int32), send_row.astype(np.int32), int(rank_offsets[-1])


def dispatch_metadata(topk_idx: np.ndarray, topk_w: np.ndarray, num_experts: int, num_ranks: int,
                      send_row: np.ndarray, num_recv: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per receive row: source token, local expert ids (or -1) and weights (or +0.0) (reading 5)."""
    T, k = topk_idx.shape
    L = num_experts // num_ranks
    valid, rank = expert_ranks(topk_idx, num_experts, num_ranks)
    recv_src_idx = np.full(num_recv, -1, dtype=np.int32)
    recv_topk_idx = np.full((num_recv, k), -1, dtype=np.int32)
    recv_topk_w = np.zeros((num_recv, k), dtype=np.float32)
    tt, rr = np.nonzero(send_row >= 0)
    rows = send_row[tt, rr]
    recv_src_idx[rows] = tt
    for j in range(k):
        here = valid[tt, j] & (rank[tt, j] == rr)
        local = np.where(here, topk_idx[tt, j].astype(np.int64) - rr * L, -1)
        recv_topk_idx[rows, j] = local
        recv_topk_w[rows, j] = np.where(here, topk_w[tt, j], np.float32(0.0))
    return recv_src_idx, recv_topk_idx, recv_topk_w


def dispatch_rows_bf16(x_bits: np.ndarray, recv_src_idx: np.ndarray) -> np.ndarray:
    """bf16 dispatch payload: receive row i is a bit copy of x[recv_src_idx[i]]."""
    return x_bits[recv_src_idx]


def quantize_fp8_blocks(x_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-128-channel FP8 quantisation of bf16 rows (reading 6) [overlap notes: FP8 dispatch].

    For each row and block b of 128 channels:
      a = max |x| (exact in fp32), s = fl32(max(a, 1e-4) / 448),
      q = E4M3_RNE(fl32(x / s)).
    Returns q uint8[rows, H] and s float32[rows, H/128].
    """
    rows, H = x_bits.shape
    assert H % FP8_BLOCK == 0
    x = bf16_bits_to_f32(x_bits).reshape(rows, H // FP8_BLOCK, FP8_BLOCK)
    a = np.abs(x).max(axis=2)
    s = (np.maximum(a, AMAX_FLOOR) / E4M3_MAX).astype(np.float32)
    v = (x / s[:, :, None]).astype(np.float32)
    q = e4m3_encode_rne(v).reshape(rows, H)
    return q, s


def dispatch_rows_fp8(x_bits: np.ndarray, recv_src_idx: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """FP8 dispatch payload: receive row i is the quantised x[recv_src_idx[i]] with its scales."""
    return quantize_fp8_blocks(x_bits[recv_src_idx])


def dequantize_fp8_to_bf16(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Identity expert on FP8 rows: y = BF16_RNE(fl32(decode(q) * s))."""
    rows, H = q.shape
    v = e4m3_decode(q).reshape(rows, H // FP8_BLOCK, FP8_BLOCK) * s[:, :, None]
    return f32_to_bf16_bits_rne(v.astype(np.float32).reshape(rows, H))


def combine(y_bits: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray, send_row: np.ndarray,
            num_experts: int, num_ranks: int, tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """Top-k weighted combine (reading 7) [overlap notes: combine; rocSHMEM notes 3.2: buffer reuse].

    out[t, c] = BF16_RNE(acc), acc = +0 then, for j ascending over valid slots,
    acc = fl32(acc + fl32(w[t, j] * y[send_row[t, rank(e_tj)], c])).
    ``tokens`` restricts the output to those source tokens (in that order).
    """
    valid, rank = expert_ranks(topk_idx, num_experts, num_ranks)
    t_sel = np.arange(topk_idx.shape[0]) if tokens is None else np.asarray(tokens)
    H = y_bits.shape[1]
    acc = np.zeros((t_sel.size, H), dtype=np.float32)
    for j in range(topk_idx.shape[1]):
        ok = valid[t_sel, j]
        if not ok.any():
            continue
        tj = t_sel[ok]
        rows = send_row[tj, rank[tj, j]]
        assert (rows >= 0).all()
        prod = (topk_w[tj, j][:, None].astype(np.float32) * bf16_bits_to_f32(y_bits[rows])).astype(np.float32)
        acc[ok] = (acc[ok] + prod).astype(np.float32)
    return f32_to_bf16_bits_rne(acc)


def combine_f64(y_bits: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray, send_row: np.ndarray,
                num_experts: int, num_ranks: int, tokens: Optional[np.ndarray] = None
                ) -> Tuple[np.ndarray, np.ndarray]:
    """The exact weighted sum in fp64, and the sum of |w_j * y_j| (for cancellation-aware bounds)."""
    valid, rank = expert_ranks(topk_idx, num_experts, num_ranks)
    t_sel = np.arange(topk_idx.shape[0]) if tokens is None else np.asarray(tokens)
    H = y_bits.shape[1]
    acc = np.zeros((t_sel.size, H), dtype=np.float64)
    mag = np.zeros((t_sel.size, H), dtype=np.float64)
    for j in range(topk_idx.shape[1]):
        ok = valid[t_sel, j]
        tj = t_sel[ok]
        rows = send_row[tj, rank[tj, j]]
        p = topk_w[tj, j][:, None].astype(np.float64) * bf16_bits_to_f32(y_bits[rows]).astype(np.float64)
        acc[ok] += p
        mag[ok] += np.abs(p)
    return acc, mag


# ----------------------------------------------------------------------------------------------
# Low-latency (per-expert) receive layout.
#
# [DeepEP overview] and [overlap notes, 节点间通信] describe a second, low-latency dispatch/combine
# mode for decoding, whose receivers keep one fixed-size buffer per local expert.  Readings taken
# (the pages give no more detail):
#   8. one receive row per (token, distinct valid expert) -- a token naming an expert twice is
#      sent to it once, and both slots read that row back in combine;
#   9. expert e's buffer has `capacity` rows; the row of token t is
#      pos(t, e) = #{t' < t : t' names e} (stable, ascending source token);
#  10. combine: acc = +0, then for j ascending over valid slots,
#      acc = fl32(acc + fl32(w_j * y[e_j, pos(t, e_j)])); out = BF16_RNE(acc).
# Buffers are [E, capacity, ...]: rank r's experts are the contiguous block r*L .. r*L+L-1, so this
# is also R ranks x [L, capacity, ...] as each receiving rank would hold it.

def ll_layout(topk_idx: np.ndarray, num_experts: int) -> Tuple[np.ndarray, np.ndarray]:
    """recv_count int32[E] (distinct tokens per expert) and slot_pos int32[T, k] (pos(t, e_tj) or -1)."""
    T, k = topk_idx.shape
    e = topk_idx.astype(np.int64)
    valid = (e >= 0) & (e < num_experts)
    member = np.zeros((T, num_experts), dtype=np.int64)
    t_of_slot = np.broadcast_to(np.arange(T)[:, None], e.shape)
    member[t_of_slot[valid], e[valid]] = 1
    before = np.cumsum(member, axis=0) - member  # tokens t' < t that name e
    slot_pos = np.where(valid, before[t_of_slot, np.where(valid, e, 0)], -1)
    return member.sum(axis=0).astype(np.int32), slot_pos.astype(np.int32)


def ll_dispatch(x_bits: np.ndarray, topk_idx: np.ndarray, num_experts: int, capacity: int, dtype: str
                ) -> Dict[str, np.ndarray]:
    """Per-expert receive buffers; rows at or beyond recv_count[e] are left as zeros / -1."""
    T, H = x_bits.shape
    recv_count, slot_pos = ll_layout(topk_idx, num_experts)
    assert capacity >= T
    src = np.full((num_experts, capacity), -1, dtype=np.int32)
    tt, jj = np.nonzero(slot_pos >= 0)
    ee = topk_idx[tt, jj].astype(np.int64)
    src[ee, slot_pos[tt, jj]] = tt  # duplicate slots write the same (row, token)
    out = {"recv_count": recv_count, "slot_pos": slot_pos, "recv_src_idx": src}
    flat = src.reshape(-1)
    rows = np.nonzero(flat >= 0)[0]
    if dtype == "bf16":
        rx = np.zeros((num_experts * capacity, H), dtype=np.uint16)
        rx[rows] = x_bits[flat[rows]]
        out["recv_x"] = rx.reshape(num_experts, capacity, H)
    else:
        q, sc = quantize_fp8_blocks(x_bits[flat[rows]]) if rows.size else (
            np.zeros((0, H), np.uint8), np.zeros((0, H // FP8_BLOCK), np.float32))
        rx = np.zeros((num_experts * capacity, H), dtype=np.uint8)
        rs = np.zeros((num_experts * capacity, H // FP8_BLOCK), dtype=np.float32)
        rx[rows], rs[rows] = q, sc
        out["recv_x"] = rx.reshape(num_experts, capacity, H)
        out["recv_scales"] = rs.reshape(num_experts, capacity, H // FP8_BLOCK)
    return out


def ll_combine(y_bits: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray, slot_pos: np.ndarray,
               num_experts: int, tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """Combine from per-expert buffers y[E, capacity, H] (reading 10)."""
    E, cap, H = y_bits.shape
    t_sel = np.arange(topk_idx.shape[0]) if tokens is None else np.asarray(tokens)
    acc = np.zeros((t_sel.size, H), dtype=np.float32)
    flat = y_bits.reshape(E * cap, H)
    for j in range(topk_idx.shape[1]):
        pos = slot_pos[t_sel, j]
        ok = pos >= 0
        if not ok.any():
            continue
        rows = topk_idx[t_sel[ok], j].astype(np.int64) * cap + pos[ok]
        prod = (topk_w[t_sel[ok], j][:, None].astype(np.float32) * bf16_bits_to_f32(flat[rows])).astype(np.float32)
        acc[ok] = (acc[ok] + prod).astype(np.float32)
    return f32_to_bf16_bits_rne(acc)


# ----------------------------------------------------------------------------------------------
# Backward (training).  [DeepEP overview: the library serves training as well as inference and its
# backward path needs its own integration; overlap notes: the kernels target training and prefill.]
# The pages give no formulas; the backward of each forward step is its adjoint (readings):
#  11. combine backward, for receive row i = send_row[t, r]:
#        grad_y[i, c] = BF16_RNE(fp32 sum, j ascending over valid slots of t on rank r, of
#                       fl32(w_tj * g[t, c]))
#      and grad_w[t, j] = sum_c g[t, c] * y[row(t, j), c] (a dot product over H; the exact value is
#      the reference, computed in fp64; invalid slots get 0);
#  12. dispatch backward: grad_x[t, c] = BF16_RNE(fp32 sum, r ascending over ranks t was sent to, of
#      grad_recv[send_row[t, r], c]); grad_topk_w[t, j] = grad_recv_topk_w[send_row[t, rank(e_tj)], j]
#      for valid slots, else 0 (the weight was forwarded unchanged).

def combine_backward(g_bits: np.ndarray, y_bits: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray,
                     send_row: np.ndarray, num_experts: int, num_ranks: int, num_rows: int
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """grad_y bf16 bits [num_rows, H] (reading 11) and grad_w fp64 [T, k] (exact dot products)."""
    T, k = topk_idx.shape
    H = g_bits.shape[1]
    valid, rank = expert_ranks(topk_idx, num_experts, num_ranks)
    g = bf16_bits_to_f32(g_bits)
    acc = np.zeros((num_rows, H), dtype=np.float32)
    for j in range(k):  # ascending slots: each adds its term to the row of its rank
        ok = valid[:, j]
        tt = np.nonzero(ok)[0]
        rows = send_row[tt, rank[tt, j]]
        prod = (topk_w[tt, j][:, None].astype(np.float32) * g[tt]).astype(np.float32)
        acc[rows] = (acc[rows] + prod).astype(np.float32)  # rows are distinct within one j
    grad_y = f32_to_bf16_bits_rne(acc)
    grad_w = np.zeros((T, k), dtype=np.float64)
    yf = bf16_bits_to_f32(y_bits).astype(np.float64)
    for j in range(k):
        tt = np.nonzero(valid[:, j])[0]
        rows = send_row[tt, rank[tt, j]]
        grad_w[tt, j] = (g[tt].astype(np.float64) * yf[rows]).sum(axis=1)
    return grad_y, grad_w


def dispatch_backward(grad_recv_bits: np.ndarray, grad_recv_w: np.ndarray, topk_idx: np.ndarray,
                      send_row: np.ndarray, num_experts: int, num_ranks: int
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """grad_x bf16 bits [T, H] and grad_topk_w fp32 [T, k] (reading 12)."""
    T, R = send_row.shape
    H = grad_recv_bits.shape[1]
    acc = np.zeros((T, H), dtype=np.float32)
    gr = bf16_bits_to_f32(grad_recv_bits)
    for r in range(R):  # ascending ranks
        tt = np.nonzero(send_row[:, r] >= 0)[0]
        acc[tt] = (acc[tt] + gr[send_row[tt, r]]).astype(np.float32)
    valid, rank = expert_ranks(topk_idx, num_experts, num_ranks)
    gw = np.zeros(topk_idx.shape, dtype=np.float32)
    for j in range(topk_idx.shape[1]):
        tt = np.nonzero(valid[:, j])[0]
        gw[tt, j] = grad_recv_w[send_row[tt, rank[tt, j]], j]
    return f32_to_bf16_bits_rne(acc), gw


def run_all(x_bits: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray, num_experts: int,
            num_ranks: int, dtype: str) -> Dict[str, np.ndarray]:
    """Layout, slots, metadata and payload for one workload, as a dict of arrays."""
    tpr, tpe, mask = get_dispatch_layout(topk_idx, num_experts, num_ranks)
    rank_offsets, send_row, num_recv = assign_slots(mask)
    src, ridx, rw = dispatch_metadata(topk_idx, topk_w, num_experts, num_ranks, send_row, num_recv)
    out = {
        "tokens_per_rank": tpr, "tokens_per_expert": tpe, "is_token_in_rank": mask,
        "rank_offsets": rank_offsets, "send_row": send_row, "num_recv": np.int32(num_recv),
        "recv_src_idx": src, "recv_topk_idx": ridx, "recv_topk_w": rw,
    }
    if dtype == "bf16":
        out["recv_x"] = dispatch_rows_bf16(x_bits, src)
    elif dtype == "fp8":
        out["recv_x"], out["recv_scales"] = dispatch_rows_fp8(x_bits, src)
    else:
        raise ValueError(dtype)
    return out
