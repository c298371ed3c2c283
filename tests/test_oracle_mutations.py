"""Planted mistakes in the oracle (CPU only): each must be caught by the pins.

Each mutant replaces one oracle routine with a plausible wrong variant (a
dropped term, a wrong sign or index, an inclusive instead of exclusive
prefix, another rounding).  The pin suite is then run against the mutated
oracle and must fail.  This shows the pins are sharp enough to catch that
class of error; the real oracle passes the same suite in test_oracle_pins.py.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import numerics as N
from oracle import router as RT
from tests import test_oracle_backward as PB
from tests import test_oracle_ll as PL
from tests import test_oracle_pins as P
from tests import test_oracle_router as PR


def _pin_suite():
    P.test_golden_dequant_bf16()
    P.test_combine_f64_closed_form()
    P.test_golden_layout_dispatch_combine("hand_layout_dispatch_combine.json")
    P.test_golden_layout_dispatch_combine("hand_duplicate_ids.json")
    P.test_golden_fp8_blocks()
    P.test_golden_combine_fp32_order()
    for case in P.TINY_CASES[:5]:
        for dtype in ("bf16", "fp8"):
            P.test_oracle_vs_bruteforce(case, dtype)
    P.test_fp8_edge_rows()
    P.test_identity_round_trip_k1_is_exact()
    P.test_identity_round_trip_weighted(P.W.CONFIG_BY_NAME["tiny"])
    PL.test_golden_low_latency()
    PB.test_golden_backward()
    PB.test_dispatch_backward_rank_order()
    PB.test_combine_backward_slot_order()
    for case in PB.CASES:
        PB.test_backward_vs_bruteforce(case)
    for case in PL.LL_CASES[:3]:
        PL.test_ll_vs_bruteforce(case, "bf16")


def _rank_modulo(topk_idx, E, R):
    e = topk_idx.astype(np.int64)
    valid = (e >= 0) & (e < E)
    return valid, np.where(valid, e % R, -1)


def _slots_inclusive(mask):
    m = mask.astype(np.int64) != 0
    offs = np.zeros(m.shape[1] + 1, dtype=np.int64)
    offs[1:] = np.cumsum(m.sum(axis=0))
    send = np.where(m, offs[None, :-1] + np.cumsum(m, axis=0), -1)
    return offs.astype(np.int32), send.astype(np.int32), int(offs[-1])


def _slots_descending(mask):
    m = mask.astype(np.int64) != 0
    offs = np.zeros(m.shape[1] + 1, dtype=np.int64)
    offs[1:] = np.cumsum(m.sum(axis=0))
    after = np.cumsum(m[::-1], axis=0)[::-1] - m
    send = np.where(m, offs[None, :-1] + after, -1)
    return offs.astype(np.int32), send.astype(np.int32), int(offs[-1])


def _bf16_truncate(x):
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _e4m3_ties_away(x):
    v = np.ascontiguousarray(x, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    t = N.E4M3_MAGNITUDES
    hi = np.minimum(np.searchsorted(t, a), 126)
    lo = np.maximum(hi - 1, 0)
    code = np.where(t[hi] - a <= a - t[lo], hi, lo)
    code = np.where(a >= 448.0, 126, code)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def _quant_reciprocal(x_bits):
    rows, H = x_bits.shape
    x = N.bf16_bits_to_f32(x_bits).reshape(rows, H // 128, 128)
    a = np.maximum(np.abs(x).max(axis=2), np.float32(1e-4))
    s = (a / np.float32(448)).astype(np.float32)
    v = (x * (np.float32(448) / a)[:, :, None]).astype(np.float32)
    return N.e4m3_encode_rne(v).reshape(rows, H), s


def _quant_no_floor(x_bits):
    rows, H = x_bits.shape
    x = N.bf16_bits_to_f32(x_bits).reshape(rows, H // 128, 128)
    a = np.abs(x).max(axis=2)
    s = (a / np.float32(448)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        v = (x / s[:, :, None]).astype(np.float32)
    v = np.nan_to_num(v)
    return N.e4m3_encode_rne(v).reshape(rows, H), s


def _dequant_rounded(q, s, to_bf16):
    rows, H = q.shape
    v = N.e4m3_decode(q).reshape(rows, H // 128, 128) * s[:, :, None]
    return to_bf16(v.astype(np.float32).reshape(rows, H))


def _dequant_truncates(q, s):
    return _dequant_rounded(q, s, _bf16_truncate)


def _dequant_ties_away(q, s):
    def half_away(x):
        u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
        return ((u + np.uint64(0x8000)) >> np.uint64(16)).astype(np.uint16)
    return _dequant_rounded(q, s, half_away)


def _combine_f64_in_fp32(y, idx, w, send_row, E, R, tokens=None):
    valid, rank = O.expert_ranks(idx, E, R)
    t_sel = np.arange(idx.shape[0]) if tokens is None else np.asarray(tokens)
    acc = np.zeros((t_sel.size, y.shape[1]), dtype=np.float32)
    mag = np.zeros((t_sel.size, y.shape[1]), dtype=np.float32)
    for j in range(idx.shape[1]):
        ok = valid[t_sel, j]
        tj = t_sel[ok]
        p = w[tj, j][:, None] * N.bf16_bits_to_f32(y[send_row[tj, rank[tj, j]]])
        acc[ok] += p
        mag[ok] += np.abs(p)
    return acc.astype(np.float64), mag.astype(np.float64)


_orig_combine_f64 = O.combine_f64


def _combine_f64_signed_magnitude(y, idx, w, send_row, E, R, tokens=None):
    acc, _ = _orig_combine_f64(y, idx, w, send_row, E, R, tokens)
    return acc, np.abs(acc)


_orig_layout = O.get_dispatch_layout


def _layout_experts_once_per_token(topk_idx, E, R):
    tpr, _, mask = _orig_layout(topk_idx, E, R)
    tpe = np.zeros(E, dtype=np.int32)
    for row in topk_idx:
        for e in set(int(v) for v in row if 0 <= v < E):
            tpe[e] += 1
    return tpr, tpe, mask


def _layout_of_clamped_ids(topk_idx, E, R):
    return _orig_layout(np.clip(topk_idx, 0, E - 1).astype(np.int32), E, R)


def _quant_amax_per_row(x_bits):
    rows, H = x_bits.shape
    x = N.bf16_bits_to_f32(x_bits).reshape(rows, H // 128, 128)
    a = np.repeat(np.abs(x).max(axis=(1, 2))[:, None], H // 128, axis=1)
    s = (np.maximum(a, np.float32(1e-4)) / np.float32(448)).astype(np.float32)
    v = (x / s[:, :, None]).astype(np.float32)
    return N.e4m3_encode_rne(v).reshape(rows, H), s


_orig_quant = O.quantize_fp8_blocks


def _quant_stores_quantisation_scale(x_bits):
    q, s = _orig_quant(x_bits)
    return q, (np.float32(1.0) / s).astype(np.float32)


_orig_metadata = O.dispatch_metadata
_orig_slots = O.assign_slots
_orig_dbwd = O.dispatch_backward


def _meta_keeps_other_ranks_weights(idx, w, E, R, send_row, n):
    src, ridx, rw = _orig_metadata(idx, w, E, R, send_row, n)
    valid = (idx >= 0) & (idx < E)
    rw = np.where(valid[src], w[src], np.float32(0.0)).astype(np.float32) if n else rw
    return src, ridx, rw


def _slots_unsent_zero(mask):
    offs, send, n = _orig_slots(mask)
    return offs, np.where(send < 0, 0, send).astype(np.int32), n


def _dbwd_descending_ranks(gr, grw, idx, send_row, E, R):
    _, gw = _orig_dbwd(gr, grw, idx, send_row, E, R)
    T = send_row.shape[0]
    acc = np.zeros((T, gr.shape[1]), dtype=np.float32)
    g = N.bf16_bits_to_f32(gr)
    for r in reversed(range(send_row.shape[1])):
        tt = np.nonzero(send_row[:, r] >= 0)[0]
        acc[tt] = (acc[tt] + g[send_row[tt, r]]).astype(np.float32)
    return N.f32_to_bf16_bits_rne(acc), gw


_orig_cbwd = O.combine_backward


def _cbwd_descending_slots(g_bits, y_bits, idx, w, send_row, E, R, n):
    _, gw = _orig_cbwd(g_bits, y_bits, idx, w, send_row, E, R, n)
    valid, rank = O.expert_ranks(idx, E, R)
    g = N.bf16_bits_to_f32(g_bits)
    acc = np.zeros((n, g.shape[1]), dtype=np.float32)
    for j in reversed(range(idx.shape[1])):
        tt = np.nonzero(valid[:, j])[0]
        rows = send_row[tt, rank[tt, j]]
        acc[rows] = (acc[rows] + (w[tt, j][:, None].astype(np.float32) * g[tt]).astype(np.float32)).astype(np.float32)
    return N.f32_to_bf16_bits_rne(acc), gw


_orig_combine = O.combine


def _combine_drop_last(y, idx, w, send_row, E, R, tokens=None):
    return _orig_combine(y, idx[:, :-1], w[:, :-1], send_row, E, R, tokens)


def _combine_fp64(y, idx, w, send_row, E, R, tokens=None):
    acc, _ = O.combine_f64(y, idx, w, send_row, E, R, tokens)
    return N.f32_to_bf16_bits_rne(acc.astype(np.float32))


def _combine_fused(y, idx, w, send_row, E, R, tokens=None):
    valid, rank = O.expert_ranks(idx, E, R)
    t_sel = np.arange(idx.shape[0]) if tokens is None else np.asarray(tokens)
    acc = np.zeros((t_sel.size, y.shape[1]), dtype=np.float32)
    for j in range(idx.shape[1]):
        ok = valid[t_sel, j]
        tj = t_sel[ok]
        rows = send_row[tj, rank[tj, j]]
        exact = w[tj, j][:, None].astype(np.float64) * N.bf16_bits_to_f32(y[rows]).astype(np.float64)
        acc[ok] = (acc[ok].astype(np.float64) + exact).astype(np.float32)
    return N.f32_to_bf16_bits_rne(acc)


def _combine_reversed(y, idx, w, send_row, E, R, tokens=None):
    return _orig_combine(y, idx[:, ::-1].copy(), w[:, ::-1].copy(), send_row, E, R, tokens)


_orig_meta = O.dispatch_metadata


def _meta_global_ids(idx, w, E, R, send_row, n):
    src, ridx, rw = _orig_meta(idx, w, E, R, send_row, n)
    L = E // R
    rows_rank = np.searchsorted(np.cumsum((send_row >= 0).sum(axis=0)), np.arange(n), side="right")
    return src, np.where(ridx >= 0, ridx + rows_rank[:, None] * L, -1).astype(np.int32), rw


def _ll_layout_per_slot(topk_idx, num_experts):
    # positions count every slot, so a token naming an expert twice takes two rows
    T, k = topk_idx.shape
    e = topk_idx.astype(np.int64)
    valid = (e >= 0) & (e < num_experts)
    pos = np.full((T, k), -1, dtype=np.int64)
    count = np.zeros(num_experts, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if valid[t, j]:
                pos[t, j] = count[e[t, j]]
                count[e[t, j]] += 1
    return count.astype(np.int32), pos.astype(np.int32)


_orig_ll_combine = O.ll_combine


def _ll_combine_once_per_expert(y, idx, w, slot_pos, E, tokens=None):
    pos = slot_pos.copy()
    for t in range(idx.shape[0]):
        seen = set()
        for j in range(idx.shape[1]):
            if pos[t, j] >= 0:
                if idx[t, j] in seen:
                    pos[t, j] = -1
                seen.add(idx[t, j])
    return _orig_ll_combine(y, idx, w, pos, E, tokens)


_orig_dbwd = O.dispatch_backward


def _dbwd_drop_last_rank(gr, grw, idx, send_row, E, R):
    sr = send_row.copy()
    sr[:, -1] = -1
    gx, _ = _orig_dbwd(gr, grw, idx, sr, E, R)
    return gx, _orig_dbwd(gr, grw, idx, send_row, E, R)[1]


def _dbwd_weight_of_first_slot(gr, grw, idx, send_row, E, R):
    gx, gw = _orig_dbwd(gr, grw, idx, send_row, E, R)
    valid, rank = O.expert_ranks(idx, E, R)
    for j in range(idx.shape[1]):
        tt = np.nonzero(valid[:, j])[0]
        gw[tt, j] = grw[send_row[tt, rank[tt, j]], 0]
    return gx, gw


_orig_cbwd = O.combine_backward


def _cbwd_unweighted(g, y, idx, w, send_row, E, R, n):
    return _orig_cbwd(g, y, idx, np.ones_like(w), send_row, E, R, n)


def _router_pin_suite():
    PR.test_golden_router()
    for case in PR.SMALL:
        PR.test_router_vs_bruteforce(case)
        PR.test_router_properties(case)


_orig_route = RT.route


def _route_ties_to_higher_id(logits, k, gate="softmax", num_groups=1, topk_groups=1):
    # selection on the experts in reverse id order, mapped back: equal logits prefer the higher id
    x = np.ascontiguousarray(logits, dtype=np.float32)
    E = x.shape[1]
    if num_groups > 1:
        return _orig_route(x, k, gate, num_groups, topk_groups)
    idx, w = _orig_route(x[:, ::-1], k, gate, 1, 1)
    return (E - 1 - idx).astype(np.int32), w


def _group_mask_sum_top2(logits, num_groups, topk_groups):
    T, E = logits.shape
    S = E // num_groups
    g = np.sort(logits.reshape(T, num_groups, S).astype(np.float64), axis=2)
    score = g[:, :, -1] + (g[:, :, -2] if S > 1 else 0.0)
    order = np.lexsort((np.broadcast_to(np.arange(num_groups), score.shape), -score), axis=1)
    keep = np.zeros((T, num_groups), dtype=bool)
    np.put_along_axis(keep, order[:, :topk_groups], True, axis=1)
    return np.repeat(keep, S, axis=1)


def _group_mask_ties_to_higher_group(logits, num_groups, topk_groups):
    T, E = logits.shape
    S = E // num_groups
    score = logits.reshape(T, num_groups, S).max(axis=2).astype(np.float64)
    order = np.lexsort((np.broadcast_to(-np.arange(num_groups), score.shape), -score), axis=1)
    keep = np.zeros((T, num_groups), dtype=bool)
    np.put_along_axis(keep, order[:, :topk_groups], True, axis=1)
    return np.repeat(keep, S, axis=1)


def _route_softmax_over_all(logits, k, gate="softmax", num_groups=1, topk_groups=1):
    idx, w = _orig_route(logits, k, gate, num_groups, topk_groups)
    if gate != "softmax":
        return idx, w
    x = np.asarray(logits, dtype=np.float64)
    p = np.exp(x - x.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    return idx, np.take_along_axis(p, idx.astype(np.int64), axis=1).astype(np.float32)


def _route_sigmoid_unnormalised(logits, k, gate="softmax", num_groups=1, topk_groups=1):
    idx, w = _orig_route(logits, k, gate, num_groups, topk_groups)
    if gate != "sigmoid":
        return idx, w
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), idx.astype(np.int64), axis=1)
    return idx, (1.0 / (1.0 + np.exp(-sel))).astype(np.float32)


def _route_signed_zero_order(logits, k, gate="softmax", num_groups=1, topk_groups=1):
    x = np.array(logits, dtype=np.float32)
    x[(x == 0) & np.signbit(x)] = np.float32(-1e-30)  # -0.0 ranked below +0.0
    return _orig_route(x, k, gate, num_groups, topk_groups)


ROUTER_MUTANTS = {
    "router_ties_to_higher_id": ("route", _route_ties_to_higher_id),
    "router_group_score_sum_top2": ("group_mask", _group_mask_sum_top2),
    "router_group_ties_to_higher_group": ("group_mask", _group_mask_ties_to_higher_group),
    "router_softmax_over_all_experts": ("route", _route_softmax_over_all),
    "router_sigmoid_not_normalised": ("route", _route_sigmoid_unnormalised),
    "router_negative_zero_below_positive_zero": ("route", _route_signed_zero_order),
}


@pytest.mark.parametrize("name", sorted(ROUTER_MUTANTS))
def test_router_pins_catch_mutant(name, monkeypatch):
    attr, fn = ROUTER_MUTANTS[name]
    monkeypatch.setattr(RT, attr, fn)
    with pytest.raises(AssertionError):
        _router_pin_suite()


MUTANTS = {
    "dequant_bf16_truncates": ("dequantize_fp8_to_bf16", _dequant_truncates),
    "dequant_bf16_ties_away": ("dequantize_fp8_to_bf16", _dequant_ties_away),
    "combine_f64_accumulates_in_fp32": ("combine_f64", _combine_f64_in_fp32),
    "combine_f64_magnitude_of_sum": ("combine_f64", _combine_f64_signed_magnitude),
    "dispatch_backward_drops_last_rank": ("dispatch_backward", _dbwd_drop_last_rank),
    "dispatch_backward_weight_slot": ("dispatch_backward", _dbwd_weight_of_first_slot),
    "combine_backward_unweighted": ("combine_backward", _cbwd_unweighted),
    "ll_positions_per_slot": ("ll_layout", _ll_layout_per_slot),
    "ll_combine_duplicate_once": ("ll_combine", _ll_combine_once_per_expert),
    "rank_is_e_mod_R": ("expert_ranks", _rank_modulo),
    "inclusive_prefix": ("assign_slots", _slots_inclusive),
    "descending_tokens_in_segment": ("assign_slots", _slots_descending),
    "bf16_truncation": ("f32_to_bf16_bits_rne", _bf16_truncate),
    "e4m3_ties_away_from_zero": ("e4m3_encode_rne", _e4m3_ties_away),
    "fp8_multiply_by_reciprocal": ("quantize_fp8_blocks", _quant_reciprocal),
    "fp8_no_amax_floor": ("quantize_fp8_blocks", _quant_no_floor),
    "combine_drops_last_slot": ("combine", _combine_drop_last),
    "combine_fp64_accumulate": ("combine", _combine_fp64),
    "combine_reversed_slot_order": ("combine", _combine_reversed),
    "combine_fused_multiply_add": ("combine", _combine_fused),
    "metadata_global_expert_ids": ("dispatch_metadata", _meta_global_ids),
    "expert_counts_once_per_token": ("get_dispatch_layout", _layout_experts_once_per_token),
    "invalid_ids_clamped_not_skipped": ("get_dispatch_layout", _layout_of_clamped_ids),
    "fp8_amax_per_row_not_per_block": ("quantize_fp8_blocks", _quant_amax_per_row),
    "fp8_stores_quantisation_scale": ("quantize_fp8_blocks", _quant_stores_quantisation_scale),
    "metadata_keeps_weights_of_other_ranks": ("dispatch_metadata", _meta_keeps_other_ranks_weights),
    "unsent_send_row_zero": ("assign_slots", _slots_unsent_zero),
    "dispatch_backward_descending_ranks": ("dispatch_backward", _dbwd_descending_ranks),
    "combine_backward_descending_slots": ("combine_backward", _cbwd_descending_slots),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    with pytest.raises(AssertionError):
        _pin_suite()
