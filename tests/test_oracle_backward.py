"""Pins of the backward definitions in the oracle (no GPU)."""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import bruteforce as bf
from oracle import moe_oracle as O
from oracle.numerics import bf16_bits_to_f32, f32_to_bf16_bits_rne

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _layout(idx, E, R):
    _, _, mask = O.get_dispatch_layout(idx, E, R)
    _, send_row, n = O.assign_slots(mask)
    return send_row, n


def test_golden_backward():
    fwd = json.load(open(os.path.join(GOLDEN, "hand_layout_dispatch_combine.json")))
    g = json.load(open(os.path.join(GOLDEN, "hand_backward.json")))
    E, R = fwd["num_experts"], fwd["num_ranks"]
    idx = np.array(fwd["topk_idx"], np.int32)
    w = np.array(fwd["topk_w"], np.float32)
    send_row, n = _layout(idx, E, R)
    gout = f32_to_bf16_bits_rne(np.array([[t + 1, -(t + 1)] for t in range(5)], np.float32))
    y = f32_to_bf16_bits_rne(np.array([[i + 1, -(i + 1) / 2] for i in range(n)], np.float32))
    grw = np.array([[10 * i + j for j in range(3)] for i in range(n)], np.float32)
    gy, gw = O.combine_backward(gout, y, idx, w, send_row, E, R, n)
    assert bf16_bits_to_f32(gy).tolist() == g["expect"]["grad_y"]
    assert gw.tolist() == g["expect"]["grad_w"]
    gx, gtw = O.dispatch_backward(y, grw, idx, send_row, E, R)
    assert bf16_bits_to_f32(gx).tolist() == g["expect"]["grad_x"]
    assert gtw.tolist() == g["expect"]["grad_topk_w"]


def test_dispatch_backward_rank_order():
    """The rank rows of a token are added in ascending rank order, in fp32, then rounded to bf16.

    Worked by hand: one token on four ranks (E = 4, R = 4, k = 4, expert r on rank r) whose receive
    rows hold 1, 2^-8, 2^-24, 2^-24 (all exact in bf16).  Ascending: 1 + 2^-8 is exact; adding
    2^-24 twice rounds back each time (a tie, to the even neighbour), so the sum is 1 + 2^-8, a bf16
    tie that rounds to 1.0.  In descending order 2^-24 + 2^-24 = 2^-23 and the sum is
    1 + 2^-8 + 2^-23 (exact in fp32), which rounds up to 1 + 2^-7 in bf16.
    """
    idx = np.array([[0, 1, 2, 3]], np.int32)
    send_row, n = _layout(idx, 4, 4)
    assert send_row.tolist() == [[0, 1, 2, 3]] and n == 4
    rows = f32_to_bf16_bits_rne(np.array([[1.0] * 8, [2.0 ** -8] * 8, [2.0 ** -24] * 8, [2.0 ** -24] * 8],
                                         np.float32))
    gx, _ = O.dispatch_backward(rows, np.zeros((4, 4), np.float32), idx, send_row, 4, 4)
    assert bf16_bits_to_f32(gx).tolist() == [[1.0] * 8]


def test_combine_backward_slot_order():
    """A rank row's gradient adds the token's slots on that rank in ascending slot order, in fp32.

    Worked by hand: one token, four slots naming experts 0..3, all on the one rank (E = 4, R = 1),
    g = 1 and weights 1, 2^-8, 2^-24, 2^-24: the products are exact and, as in the dispatch backward
    case, ascending order gives 1 + 2^-8 (bf16: 1.0) where descending would give 1 + 2^-8 + 2^-23
    (bf16: 1 + 2^-7).
    """
    idx = np.array([[0, 1, 2, 3]], np.int32)
    w = np.array([[1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24]], np.float32)
    send_row, n = _layout(idx, 4, 1)
    assert send_row.tolist() == [[0]] and n == 1
    g = f32_to_bf16_bits_rne(np.ones((1, 8), np.float32))
    gy, _ = O.combine_backward(g, g.copy(), idx, w, send_row, 4, 1, 1)
    assert bf16_bits_to_f32(gy).tolist() == [[1.0] * 8]


CASES = [(0, 1, 16, 8, 1, 1, 0.0), (1, 23, 16, 16, 4, 4, 0.2), (2, 40, 24, 32, 8, 8, 0.1), (3, 17, 16, 12, 3, 3, 0.3)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}_T{c[1]}_E{c[3]}_k{c[4]}_R{c[5]}")
def test_backward_vs_bruteforce(case):
    seed, T, H, E, k, R, inv = case
    d = W.random_case(seed, T, H, E, k, R, invalid_frac=inv)
    idx, w = d["topk_idx"].copy(), d["topk_w"]
    if T > 2 and k > 1:
        idx[1, 1] = idx[1, 0]  # two slots naming one expert
    send_row, n = _layout(idx, E, R)
    rng = np.random.default_rng(seed)
    g = W.draw_hidden(rng, T, H)
    y = W.draw_hidden(rng, max(n, 1), H)
    gy, gw = O.combine_backward(g, y, idx, w, send_row, E, R, n)
    bgy, bgw = bf.combine_backward(g, y, idx.tolist(), w.tolist(), send_row.tolist(), E, R, n)
    assert gy.tolist() == bgy
    assert np.allclose(gw, np.array(bgw, dtype=np.float64).reshape(gw.shape), rtol=1e-12, atol=1e-12)
    grw = rng.standard_normal((max(n, 1), k)).astype(np.float32)
    gx, gtw = O.dispatch_backward(y, grw, idx, send_row, E, R)
    bgx, bgtw = bf.dispatch_backward(y, grw.tolist(), idx.tolist(), send_row.tolist(), E, R)
    assert gx.tolist() == bgx and gtw.tolist() == bgtw


def test_adjoint_identities():
    """<g, combine(y)> = <grad_y, y> and = sum_j w_j grad_w_j; <gr, dispatch(x)> = <grad_x, x> (fp64)."""
    cfg = W.with_tokens(W.CONFIG_BY_NAME["prefill"], 96)
    d = W.make_inputs(cfg)
    idx, w = d["topk_idx"], d["topk_w"]
    E, R, H = cfg.num_experts, cfg.num_ranks, 64
    send_row, n = _layout(idx, E, R)
    rng = np.random.default_rng(7)
    # small-integer values keep every sum exact, so the bf16 results equal the exact adjoints
    g = f32_to_bf16_bits_rne(rng.integers(-8, 9, (cfg.num_tokens, H)).astype(np.float32))
    y = f32_to_bf16_bits_rne(rng.integers(-8, 9, (n, H)).astype(np.float32))
    w1 = np.ones_like(w)
    out, _ = O.combine_f64(y, idx, w1, send_row, E, R)
    gy, gw = O.combine_backward(g, y, idx, w1, send_row, E, R, n)
    lhs = (bf16_bits_to_f32(g).astype(np.float64) * out).sum()
    assert lhs == (bf16_bits_to_f32(gy).astype(np.float64) * bf16_bits_to_f32(y)).sum()
    assert lhs == gw.sum()
    src, _, _ = O.dispatch_metadata(idx, w, E, R, send_row, n)
    x = f32_to_bf16_bits_rne(rng.integers(-8, 9, (cfg.num_tokens, H)).astype(np.float32))
    gr = y
    gx, _ = O.dispatch_backward(gr, np.zeros((n, cfg.num_topk), np.float32), idx, send_row, E, R)
    lhs = (bf16_bits_to_f32(gr).astype(np.float64) * bf16_bits_to_f32(x[src]).astype(np.float64)).sum()
    assert lhs == (bf16_bits_to_f32(gx).astype(np.float64) * bf16_bits_to_f32(x).astype(np.float64)).sum()


def test_combine_backward_k1_is_a_copy():
    d = W.random_case(11, 60, 128, 16, 1, 4)
    idx = d["topk_idx"]
    send_row, n = _layout(idx, 16, 4)
    g = W.draw_hidden(np.random.default_rng(2), 60, 128)
    gy, _ = O.combine_backward(g, np.zeros((n, 128), np.uint16), idx, np.ones((60, 1), np.float32), send_row, 16, 4, n)
    src, _, _ = O.dispatch_metadata(idx, d["topk_w"], 16, 4, send_row, n)
    assert np.array_equal(gy, np.where(g[src] == 0x8000, np.uint16(0), g[src]))
