"""Pins of the router oracle (top-k gating, oracle/router.py) on the CPU.

* hand-worked cases (tests/golden/hand_router.json): ids picked by hand, weights as closed forms;
* brute force: repeated scans over plain Python lists on small inputs full of ties;
* properties: ids distinct and inside kept groups, no unselected allowed expert beats a selected
  one, weights positive, non-increasing and summing to 1;
* the routing the workload generator applies to the same logits (an independent implementation).
"""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import router as RT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_router.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def test_golden_router():
    for c in _cases():
        x = np.array(c["logits"], dtype=np.float32)
        if c["label"].startswith("no groups"):
            x[0, 0] = -0.0  # JSON keeps the sign, but make the -0.0 explicit
            assert np.signbit(x[0, 0])
        idx, w = RT.route(x, c["k"], c["gate"], c["num_groups"], c["topk_groups"])
        assert idx.tolist() == c["topk_idx"], c["label"]
        ref = np.array(c["topk_w"], dtype=np.float64)
        # the fp64 closed form rounded to fp32 (one rounding) may differ from the oracle's fp32
        # result by at most one unit in the last place
        assert np.all(np.abs(w.astype(np.float64) - ref) <= np.spacing(np.float32(ref)).astype(np.float64)), c["label"]


def _tie_heavy_logits(rng, T, E):
    """Logits on a coarse grid so that equal values (and -0.0 / +0.0) are common."""
    x = (rng.integers(-6, 7, size=(T, E)) * 0.5).astype(np.float32)
    zero = x == 0
    x[zero & (rng.random((T, E)) < 0.5)] = np.float32(-0.0)
    return x


SMALL = [  # (seed, T, E, k, G, topk_groups, gate)
    (0, 24, 8, 2, 1, 1, "softmax"),
    (1, 24, 8, 8, 1, 1, "sigmoid"),
    (2, 24, 16, 4, 4, 2, "softmax"),
    (3, 24, 16, 3, 4, 1, "sigmoid"),
    (4, 16, 32, 5, 8, 3, "softmax"),
    (5, 16, 32, 8, 2, 1, "sigmoid"),
    (6, 16, 24, 6, 8, 2, "softmax"),
]


@pytest.mark.parametrize("case", SMALL)
def test_router_vs_bruteforce(case):
    seed, T, E, k, G, KG, gate = case
    rng = np.random.default_rng(500 + seed)
    x = _tie_heavy_logits(rng, T, E)
    idx, w = RT.route(x, k, gate, G, KG)
    bidx, bw = RT.route_bruteforce(x, k, gate, G, KG)
    assert idx.tolist() == bidx
    np.testing.assert_array_max_ulp(w, np.array(bw, dtype=np.float32), maxulp=1)


def check_router_properties(x, idx, w, k, G, KG, gate):
    """What any correct top-k gate output satisfies (used on GPU results too)."""
    T, E = x.shape
    S = E // G
    assert idx.shape == (T, k) and w.shape == (T, k)
    assert ((idx >= 0) & (idx < E)).all()
    assert all(len(set(r)) == k for r in idx.tolist())
    xs = x.astype(np.float64) + 0.0
    score = xs.reshape(T, G, S).max(axis=2)
    sel = np.take_along_axis(xs, idx.astype(np.int64), axis=1)
    for t in range(T):
        order = sorted(range(G), key=lambda g: (-score[t, g], g))
        kept = set(order[:KG])
        assert all(int(e) // S in kept for e in idx[t])
        # no eligible, unselected expert beats the k-th pick
        eligible = [e for e in range(E) if e // S in kept and e not in set(idx[t].tolist())]
        last = (-sel[t, -1], int(idx[t, -1]))
        assert all((-xs[t, e], e) > last for e in eligible)
        # slots in descending (logit, ascending id) order
        keys = [(-sel[t, j], int(idx[t, j])) for j in range(k)]
        assert keys == sorted(keys)
    assert (w > 0).all() or gate == "softmax"
    assert (np.diff(w.astype(np.float64), axis=1) <= 0).all()
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= (k + 1) * 2.0 ** -24)


@pytest.mark.parametrize("case", SMALL)
def test_router_properties(case):
    seed, T, E, k, G, KG, gate = case
    x = _tie_heavy_logits(np.random.default_rng(900 + seed), T, E)
    idx, w = RT.route(x, k, gate, G, KG)
    check_router_properties(x, idx, w, k, G, KG, gate)


def _gate_of(cfg):
    G = cfg.num_groups if cfg.routing == "group_limited" else 1
    KG = cfg.topk_groups if cfg.routing == "group_limited" else 1
    return ("sigmoid" if cfg.routing == "sigmoid" else "softmax"), G, KG


@pytest.mark.parametrize("cfg", W.CONFIGS, ids=lambda c: c.name)
def test_router_matches_workload_routing(cfg):
    """The workload generator routes its own logits; the oracle must pick the same experts."""
    T = min(cfg.num_tokens, 512)
    logits = W.config_logits(cfg, T)
    g_x, g_router, _g_y, g_extra = W.seed_streams(cfg.index)
    widx, ww = W.route(cfg, g_router, g_extra, num_tokens=T)
    gate, G, KG = _gate_of(cfg)
    idx, w = RT.route(logits, cfg.num_topk, gate, G, KG)
    assert np.array_equal(idx, widx)
    np.testing.assert_array_max_ulp(w, ww, maxulp=1)
    check_router_properties(logits[:64], idx[:64], w[:64], cfg.num_topk, G, KG, gate)


def test_router_softmax_closed_form_two_experts():
    """k = 2 softmax is the logistic function of the logit gap."""
    rng = np.random.default_rng(77)
    x = rng.standard_normal((200, 16)).astype(np.float32)
    idx, w = RT.route(x, 2)
    gap = np.take_along_axis(x, idx[:, 1:2].astype(np.int64), 1).astype(np.float64) - \
        np.take_along_axis(x, idx[:, 0:1].astype(np.int64), 1).astype(np.float64)
    expect = 1.0 / (1.0 + np.exp(gap[:, 0]))
    np.testing.assert_array_max_ulp(w[:, 0], expect.astype(np.float32), maxulp=1)
    # and the first pick is numpy's argmax (first occurrence of the maximum)
    assert np.array_equal(idx[:, 0], np.argmax(x, axis=1))
