"""Pure-Python loop oracle for tiny inputs (test infrastructure only).

An independent restatement of the definitions in ``moe_oracle``, written with
plain loops and Python floats so that it shares neither structure nor
arithmetic routines with the vectorised oracle:

* receive rows are numbered by walking (rank, token) pairs in lexicographic
  order, instead of a prefix sum;
* fp32 rounding uses ``struct`` packing of Python (fp64) values.  A single
  fp64 operation on fp32 operands followed by rounding to fp32 is correctly
  rounded for +, * and / (53 >= 2*24 + 2), so this equals IEEE fp32 arithmetic;
* bf16 and E4M3 rounding use ``math.frexp`` and Python's ``round`` (which
  rounds halves to even), instead of bit tricks or table searches.

Only for tiny inputs: every element is a Python-level operation.
"""
from __future__ import annotations

import math
import struct
from typing import Dict, List

import numpy as np


def fl32(v: float) -> float:
    """Round a Python float to the nearest fp32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def bf16_round(v: float) -> int:
    """Nearest bf16 value to fp32 ``v`` (ties to even significand), as bits."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a < 2.0 ** -126:  # bf16 subnormal range: fixed step 2^-133
        r = round(a / 2.0 ** -133) * 2.0 ** -133
    else:
        m, e = math.frexp(a)  # a = m * 2^e, 0.5 <= m < 1; bf16 keeps 8 significant bits
        r = round(m * 256.0) / 256.0 * 2.0 ** e
    r = math.copysign(r, v)
    return struct.unpack("<I", struct.pack("<f", r))[0] >> 16


def e4m3_round(v: float) -> int:
    """Nearest OCP E4M3 value to ``v`` (ties to even significand, saturating at 448), as a code."""
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a >= 448.0:
        return sign | 0x7E
    if a < 2.0 ** -6:  # subnormal range: value = m * 2^-9, m in 0..7 (8 rounds up to the first normal)
        m = round(a / 2.0 ** -9)
        return sign | m  # m == 8 is code 0x08 = 2^-6, the smallest normal
    mant, e = math.frexp(a)  # a = mant * 2^e, mant in [0.5, 1): significand 2*mant in [1, 2)
    exp = e - 1
    sig = round(mant * 2.0 * 8.0)  # 8..16, in units of 1/8
    if sig == 16:
        sig = 8
        exp += 1
    if exp > 8:
        return sign | 0x7E
    code = ((exp + 7) << 3) | (sig - 8)
    return sign | min(code, 0x7E)


def e4m3_value(code: int) -> float:
    e = (code >> 3) & 0xF
    m = code & 7
    mag = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if code & 0x80 else mag


def layout(topk_idx: List[List[int]], E: int, R: int):
    L = E // R
    T = len(topk_idx)
    tpe = [0] * E
    mask = [[0] * R for _ in range(T)]
    for t in range(T):
        for e in topk_idx[t]:
            if 0 <= e < E:
                tpe[e] += 1
                mask[t][e // L] = 1
    tpr = [sum(mask[t][r] for t in range(T)) for r in range(R)]
    return tpr, tpe, mask


def slots(mask: List[List[int]], R: int):
    T = len(mask)
    send_row = [[-1] * R for _ in range(T)]
    row = 0
    offsets = []
    for r in range(R):
        offsets.append(row)
        for t in range(T):
            if mask[t][r]:
                send_row[t][r] = row
                row += 1
    offsets.append(row)
    return offsets, send_row, row


def dispatch(x_bits: np.ndarray, topk_idx: List[List[int]], topk_w: List[List[float]], E: int, R: int,
             dtype: str) -> Dict[str, object]:
    L = E // R
    tpr, tpe, mask = layout(topk_idx, E, R)
    offsets, send_row, n = slots(mask, R)
    T = len(topk_idx)
    H = x_bits.shape[1] if T else 0
    k = len(topk_idx[0]) if T else 0
    src = [-1] * n
    ridx = [[-1] * k for _ in range(n)]
    rw = [[0.0] * k for _ in range(n)]
    rows: List[List[int]] = [[] for _ in range(n)]
    scales: List[List[float]] = [[] for _ in range(n)]
    for t in range(T):
        for r in range(R):
            i = send_row[t][r]
            if i < 0:
                continue
            src[i] = t
            for j, e in enumerate(topk_idx[t]):
                if 0 <= e < E and e // L == r:
                    ridx[i][j] = e - r * L
                    rw[i][j] = topk_w[t][j]
            if dtype == "bf16":
                rows[i] = [int(b) for b in x_bits[t]]
            else:
                q_row: List[int] = []
                s_row: List[float] = []
                for b0 in range(0, H, 128):
                    vals = [bf16_value(int(b)) for b in x_bits[t, b0:b0 + 128]]
                    a = max(abs(v) for v in vals)
                    s = fl32(max(a, fl32(1e-4)) / 448.0)
                    s_row.append(s)
                    q_row.extend(e4m3_round(fl32(v / s)) for v in vals)
                rows[i] = q_row
                scales[i] = s_row
    return {"tokens_per_rank": tpr, "tokens_per_expert": tpe, "is_token_in_rank": mask,
            "rank_offsets": offsets, "send_row": send_row, "num_recv": n, "recv_src_idx": src,
            "recv_topk_idx": ridx, "recv_topk_w": rw, "recv_x": rows, "recv_scales": scales}


def combine(y_bits: np.ndarray, topk_idx: List[List[int]], topk_w: List[List[float]],
            send_row: List[List[int]], E: int, R: int) -> List[List[int]]:
    L = E // R
    H = y_bits.shape[1]
    out = []
    for t in range(len(topk_idx)):
        row_out = []
        for c in range(H):
            acc = 0.0
            for j, e in enumerate(topk_idx[t]):
                if not (0 <= e < E):
                    continue
                i = send_row[t][e // L]
                p = fl32(fl32(topk_w[t][j]) * bf16_value(int(y_bits[i, c])))
                acc = fl32(acc + p)
            row_out.append(bf16_round(acc))
        out.append(row_out)
    return out


def ll_dispatch(x_bits: np.ndarray, topk_idx: List[List[int]], E: int, capacity: int, dtype: str) -> Dict[str, object]:
    """Per-expert buffers: walk tokens in order and append each to every distinct valid expert it names."""
    T = len(topk_idx)
    H = x_bits.shape[1] if T else 0
    count = [0] * E
    slot_pos = []
    src = [[-1] * capacity for _ in range(E)]
    rows: Dict[tuple, List[int]] = {}
    scales: Dict[tuple, List[float]] = {}
    for t in range(T):
        placed: Dict[int, int] = {}
        for e in topk_idx[t]:
            if 0 <= e < E and e not in placed:
                placed[e] = count[e]
                count[e] += 1
        slot_pos.append([placed[e] if 0 <= e < E else -1 for e in topk_idx[t]])
        for e, p in placed.items():
            src[e][p] = t
            if dtype == "bf16":
                rows[(e, p)] = [int(b) for b in x_bits[t]]
            else:
                q_row, s_row = [], []
                for b0 in range(0, H, 128):
                    vals = [bf16_value(int(b)) for b in x_bits[t, b0:b0 + 128]]
                    a = max(abs(v) for v in vals)
                    s = fl32(max(a, fl32(1e-4)) / 448.0)
                    s_row.append(s)
                    q_row.extend(e4m3_round(fl32(v / s)) for v in vals)
                rows[(e, p)] = q_row
                scales[(e, p)] = s_row
    return {"recv_count": count, "slot_pos": slot_pos, "recv_src_idx": src, "rows": rows, "scales": scales}


def ll_combine(y_bits: np.ndarray, topk_idx: List[List[int]], topk_w: List[List[float]],
               slot_pos: List[List[int]]) -> List[List[int]]:
    H = y_bits.shape[2]
    out = []
    for t in range(len(topk_idx)):
        row_out = []
        for c in range(H):
            acc = 0.0
            for j, e in enumerate(topk_idx[t]):
                p = slot_pos[t][j]
                if p < 0:
                    continue
                acc = fl32(acc + fl32(fl32(topk_w[t][j]) * bf16_value(int(y_bits[e, p, c]))))
            row_out.append(bf16_round(acc))
        out.append(row_out)
    return out


def combine_backward(g_bits, y_bits, topk_idx, topk_w, send_row, E: int, R: int, num_rows: int):
    """grad_y (bf16 bits, lists) and grad_w (Python floats, exact sums of fp64 products)."""
    L = E // R
    H = g_bits.shape[1]
    grad_y = [[0] * H for _ in range(num_rows)]
    acc = {}
    for t, ids in enumerate(topk_idx):
        for j, e in enumerate(ids):
            if 0 <= e < E:
                i = send_row[t][e // L]
                row = acc.setdefault(i, [0.0] * H)
                for c in range(H):
                    row[c] = fl32(row[c] + fl32(fl32(topk_w[t][j]) * bf16_value(int(g_bits[t, c]))))
    for i, row in acc.items():
        grad_y[i] = [bf16_round(v) for v in row]
    grad_w = []
    for t, ids in enumerate(topk_idx):
        gw = []
        for j, e in enumerate(ids):
            if 0 <= e < E:
                i = send_row[t][e // L]
                gw.append(math.fsum(bf16_value(int(g_bits[t, c])) * bf16_value(int(y_bits[i, c])) for c in range(H)))
            else:
                gw.append(0.0)
        grad_w.append(gw)
    return grad_y, grad_w


def dispatch_backward(grad_recv_bits, grad_recv_w, topk_idx, send_row, E: int, R: int):
    L = E // R
    H = grad_recv_bits.shape[1]
    grad_x = []
    for t, rows in enumerate(send_row):
        out = []
        for c in range(H):
            acc = 0.0
            for r in range(R):
                if rows[r] >= 0:
                    acc = fl32(acc + bf16_value(int(grad_recv_bits[rows[r], c])))
            out.append(bf16_round(acc))
        grad_x.append(out)
    gw = [[fl32(grad_recv_w[send_row[t][e // L]][j]) if 0 <= e < E else 0.0 for j, e in enumerate(ids)]
          for t, ids in enumerate(topk_idx)]
    return grad_x, gw
