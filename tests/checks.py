"""Property checks shared by the oracle pins and the GPU parity tests.

These test what the definitions imply (closed forms, invariants, bijections,
error bounds) without recomputing the definitions themselves, so they can pin
the oracle and also check GPU results at sizes the oracle cannot afford.
"""
from __future__ import annotations

import numpy as np

from oracle.numerics import bf16_bits_to_f32, e4m3_decode


def check_layout_invariants(topk_idx, E, R, tpr, tpe, mask):
    T, k = topk_idx.shape
    L = E // R
    valid = (topk_idx >= 0) & (topk_idx < E)
    # counts sum to the number of valid slots (T*k when nothing is masked)
    assert int(np.asarray(tpe, dtype=np.int64).sum()) == int(valid.sum())
    mask = np.asarray(mask)
    assert mask.shape == (T, R)
    assert set(np.unique(mask).tolist()) <= {0, 1}
    assert np.array_equal(np.asarray(tpr, dtype=np.int64), mask.sum(axis=0, dtype=np.int64))
    tpe = np.asarray(tpe, dtype=np.int64)
    for r in range(R):
        block = tpe[r * L:(r + 1) * L]
        # with distinct ids per token, the busiest expert bounds the rank count from below
        if all(len(set(row[valid[i]].tolist())) == int(valid[i].sum()) for i, row in enumerate(topk_idx)):
            assert block.max(initial=0) <= tpr[r] <= min(T, int(block.sum()))
    assert int(np.asarray(tpr).sum()) <= T * min(k, R)
    # every token marked for rank r owns a valid expert of r, and vice versa
    for t in range(min(T, 2048)):
        owners = {int(e) // L for e in topk_idx[t] if 0 <= e < E}
        assert set(np.nonzero(mask[t])[0].tolist()) == owners


def check_slot_invariants(mask, rank_offsets, send_row, num_recv):
    mask = np.asarray(mask) != 0
    T, R = mask.shape
    send_row = np.asarray(send_row)
    rank_offsets = np.asarray(rank_offsets)
    assert rank_offsets[0] == 0 and rank_offsets[-1] == num_recv
    assert np.all(np.diff(rank_offsets) == mask.sum(axis=0))
    # -1 exactly where the token does not go
    assert np.array_equal(send_row >= 0, mask)
    rows = send_row[mask]
    # bijection (token, rank) <-> [0, num_recv): each token goes once to each distinct rank
    assert rows.size == num_recv
    assert np.array_equal(np.sort(rows), np.arange(num_recv))
    for r in range(R):
        seg = send_row[mask[:, r], r]
        # inside segment r, rows are consecutive from rank_offsets[r] in ascending token order
        assert np.array_equal(seg, np.arange(rank_offsets[r], rank_offsets[r + 1]))


def check_metadata(topk_idx, topk_w, E, R, send_row, recv_src_idx, recv_topk_idx, recv_topk_w):
    L = E // R
    T, k = topk_idx.shape
    for t in range(T):
        for r in range(R):
            i = send_row[t, r]
            if i < 0:
                continue
            assert recv_src_idx[i] == t
            for j in range(k):
                e = topk_idx[t, j]
                if 0 <= e < E and e // L == r:
                    assert recv_topk_idx[i, j] == e - r * L
                    assert np.float32(recv_topk_w[i, j]).tobytes() == np.float32(topk_w[t, j]).tobytes()
                else:
                    assert recv_topk_idx[i, j] == -1
                    assert np.float32(recv_topk_w[i, j]).tobytes() == np.float32(0.0).tobytes()


def check_fp8_block_properties(x_bits, q, s):
    """Invariants of per-128 E4M3 quantisation that hold whatever the rounding details."""
    rows, H = x_bits.shape
    x = bf16_bits_to_f32(x_bits).reshape(rows, H // 128, 128).astype(np.float64)
    qv = e4m3_decode(q).reshape(rows, H // 128, 128).astype(np.float64)
    s = np.asarray(s, dtype=np.float64)
    a = np.abs(x).max(axis=2)
    mag = (q & 0x7F).reshape(rows, H // 128, 128)
    assert (mag <= 0x7E).all(), "NaN code or above 448"
    big = a > 1e-4
    # the block maximum maps to exactly 448
    assert (mag.max(axis=2)[big] == 0x7E).all()
    # scale: s ~ max(a, 1e-4)/448 within one fp32 rounding
    ref = np.maximum(a, np.float32(1e-4).astype(np.float64)) / 448.0
    assert (np.abs(s - ref) <= ref * 2.0 ** -24 * 1.0001).all()
    # reconstruction error: relative 2^-4 in the normal range, 2^-10 * s absolute in the subnormal range
    v = x / s[:, :, None]
    err = np.abs(qv * s[:, :, None] - x)
    normal = np.abs(v) >= 2.0 ** -6
    bound = np.where(normal, 2.0 ** -4 * np.abs(x), 2.0 ** -10 * s[:, :, None]) * (1 + 2.0 ** -20)
    assert (err <= bound).all()
    # signs agree (zero keeps its sign)
    assert np.array_equal(np.signbit(x), (q.reshape(rows, H // 128, 128) & 0x80) != 0)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (2^(e-7)), with the subnormal floor 2^-133."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)


def check_combine_bound(out_bits, ref64, mag64, k):
    """|out - exact| <= ulp_bf16(exact) + k * 2^-24 * sum |w_j y_j| (fp32 sum error plus bf16 rounding)."""
    out = bf16_bits_to_f32(out_bits).astype(np.float64)
    bound = bf16_ulp(ref64) + k * 2.0 ** -24 * mag64 * 1.01
    assert (np.abs(out - ref64) <= bound).all()


def within_one_bf16_ulp(a_bits, b_bits) -> np.ndarray:
    """Elementwise: the two bf16 values are equal or adjacent (1 ulp), treating +0 and -0 as equal."""
    a = np.asarray(a_bits, dtype=np.uint16).astype(np.int64)
    b = np.asarray(b_bits, dtype=np.uint16).astype(np.int64)

    def ordinal(u):
        return np.where(u & 0x8000, -(u & 0x7FFF), u)

    return np.abs(ordinal(a) - ordinal(b)) <= 1
