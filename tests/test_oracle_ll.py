"""Pins of the low-latency (per-expert) layout in the oracle (no GPU)."""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import bruteforce as bf
from oracle import moe_oracle as O
from oracle.numerics import bf16_bits_to_f32, f32_to_bf16_bits_rne
from tests.checks import check_combine_bound, check_fp8_block_properties

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_low_latency():
    g = json.load(open(os.path.join(GOLDEN, "hand_low_latency.json")))
    E, cap = g["num_experts"], g["capacity"]
    idx = np.array(g["topk_idx"], dtype=np.int32)
    w = np.array(g["topk_w"], dtype=np.float32)
    ex = g["expect"]
    x = np.zeros((idx.shape[0], 128), np.uint16)
    r = O.ll_dispatch(x, idx, E, cap, "bf16")
    assert r["recv_count"].tolist() == ex["recv_count"]
    assert r["slot_pos"].tolist() == ex["slot_pos"]
    assert r["recv_src_idx"].tolist() == ex["recv_src_idx"]
    y = np.zeros((E, cap, 2), np.float32)
    for e in range(E):
        for p in range(cap):
            y[e, p] = [e + 1 + 8 * p, -(e + 1) / 2 - p]
    yb = f32_to_bf16_bits_rne(y)
    assert np.array_equal(bf16_bits_to_f32(yb), y)
    out = O.ll_combine(yb, idx, w, r["slot_pos"], E)
    assert bf16_bits_to_f32(out).tolist() == ex["combine_out"]
    assert bf.ll_combine(yb, idx.tolist(), w.tolist(), r["slot_pos"].tolist()) == out.tolist()


LL_CASES = [(0, 1, 8, 1, 0.0), (1, 37, 16, 4, 0.2), (2, 64, 32, 8, 0.1), (3, 70, 64, 8, 0.0), (4, 9, 12, 3, 0.4)]


@pytest.mark.parametrize("case", LL_CASES, ids=lambda c: f"s{c[0]}_T{c[1]}_E{c[2]}_k{c[3]}")
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_ll_vs_bruteforce(case, dtype):
    seed, T, E, k, inv = case
    d = W.random_case(seed, T, 128, E, k, 1, invalid_frac=inv)
    idx = d["topk_idx"].copy()
    if T > 2:  # a token that names one expert twice
        idx[1, :2] = idx[1, 0] if idx[1, 0] >= 0 else 0
    cap = T + 3
    r = O.ll_dispatch(d["x"], idx, E, cap, dtype)
    b = bf.ll_dispatch(d["x"], idx.tolist(), E, cap, dtype)
    assert r["recv_count"].tolist() == b["recv_count"]
    assert r["slot_pos"].tolist() == b["slot_pos"]
    assert r["recv_src_idx"].tolist() == b["recv_src_idx"]
    for (e, p), row in b["rows"].items():
        assert r["recv_x"][e, p].tolist() == row
        if dtype == "fp8":
            assert r["recv_scales"][e, p].tolist() == b["scales"][(e, p)]
    y = W.draw_expert_outputs(np.random.default_rng(seed), E * cap, 8).reshape(E, cap, 8)
    out = O.ll_combine(y, idx, d["topk_w"], r["slot_pos"], E)
    assert out.tolist() == bf.ll_combine(y, idx.tolist(), d["topk_w"].tolist(), r["slot_pos"].tolist())


@pytest.mark.parametrize("cfg", [W.CONFIG_BY_NAME["decode"], W.CONFIG_BY_NAME["group_limited"]], ids=lambda c: c.name)
def test_ll_invariants(cfg):
    g = W.seed_streams(cfg.index)
    idx, w = W.route(cfg, g[1], g[3])
    T, E = idx.shape[0], cfg.num_experts
    count, pos = O.ll_layout(idx, E)
    _, tpe, _ = O.get_dispatch_layout(idx, E, cfg.num_ranks)
    assert np.array_equal(count, tpe)  # distinct ids per token: one row per slot
    assert int(count.sum()) == T * cfg.num_topk
    for e in range(0, E, 17):
        toks, slots = np.nonzero(idx == e)
        # rows of expert e are 0..count-1 in ascending token order
        assert np.array_equal(pos[toks, slots], np.arange(count[e]))
    # combine through the per-expert layout equals the rank layout's when y rows agree per token
    x = W.draw_hidden(g[0], T, 256)
    r = O.ll_dispatch(x, idx, E, T, "bf16")
    out = O.ll_combine(r["recv_x"], idx, w, r["slot_pos"], E)
    ref64 = bf16_bits_to_f32(x).astype(np.float64) * w.astype(np.float64).sum(axis=1, keepdims=True)
    check_combine_bound(out, ref64, np.abs(ref64), cfg.num_topk)
    if cfg.dispatch_dtype == "fp8":
        q = O.ll_dispatch(x[:64], idx[:64], E, 64, "fp8")
        rows = q["recv_src_idx"].reshape(-1) >= 0
        check_fp8_block_properties(x[q["recv_src_idx"].reshape(-1)[rows]], q["recv_x"].reshape(-1, 256)[rows],
                                   q["recv_scales"].reshape(-1, 2)[rows])
