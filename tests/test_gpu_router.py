"""GPU parity of the router fused with the layout (moe_route_layout) against oracle/router.py.

Bar: expert ids bit-exact (selection only compares fp32 logits); layout outputs bit-exact against
the layout oracle applied to those ids; the dispatch plan left in the workspace gives the oracle's
receive rows; weights within a relative bound derived from the fp32 arithmetic:

* softmax: d = fl(l_j - l_0) carries |d| 2^-24 absolute error, which exp turns into a relative one;
  expf is within 2 ulp (2^-22); the k-term positive sum adds (k - 1) 2^-24; the division 2^-24.
  Bound: (|l_j - l_0| + max_i |l_i - l_0| + k + 2 * 4 + 2) 2^-24 relative to the fp64 weight.
* sigmoid: 1 / (1 + expf(-l)) is within (4 + 2) 2^-24 relative; normalising adds (k + 1) 2^-24.
  Bound: (k + 2 * 6 + 2) 2^-24.
"""
import zlib

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O
from oracle import router as RT
from tests.test_oracle_router import check_router_properties

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness  # noqa: F401  (loads the HIP library; fails loudly if missing)


def H():
    from tests import gpu_harness
    return gpu_harness


def _print_case(label, **kw):
    print(f"[case] {label} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def weight_bound(logits, idx, k, gate):
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), axis=1)
    if gate == "softmax":
        gap = np.abs(sel - sel[:, :1])
        return (gap + gap.max(axis=1, keepdims=True) + k + 10) * 2.0 ** -24
    return np.full(sel.shape, (k + 14) * 2.0 ** -24)


def check_route(res, logits, k, E, R, gate, G, KG):
    idx, w = RT.route(logits, k, gate, G, KG)
    assert np.array_equal(res["topk_idx"], idx), "expert ids differ from the oracle"
    rel = np.abs(res["topk_w"].astype(np.float64) - w.astype(np.float64)) / np.maximum(np.abs(w.astype(np.float64)),
                                                                                      1e-300)
    bound = weight_bound(logits, idx, k, gate)
    assert (rel <= bound).all(), f"weight error {rel.max():.3g} above bound {bound.min():.3g}"
    tpr, tpe, mask = O.get_dispatch_layout(idx, E, R)
    assert np.array_equal(res["tokens_per_expert"], tpe)
    assert np.array_equal(res["tokens_per_rank"], tpr)
    assert np.array_equal(res["is_token_in_rank"], mask)
    return idx, w, mask


def _gate_of(cfg):
    grouped = cfg.routing == "group_limited"
    return ("sigmoid" if cfg.routing == "sigmoid" else "softmax"), (cfg.num_groups if grouped else 1), \
        (cfg.topk_groups if grouped else 1)


@pytest.mark.parametrize("cfg", W.CONFIGS, ids=lambda c: c.name)
def test_route_workloads(cfg):
    """Every workload's own logits at full size: ids, weights, layout, then dispatch with the plan."""
    gate, G, KG = _gate_of(cfg)
    _print_case("route", workload=cfg.name, T=cfg.num_tokens, E=cfg.num_experts, k=cfg.num_topk, gate=gate, G=G)
    logits = W.config_logits(cfg)
    res = H().run_route(logits, cfg.num_topk, cfg.num_experts, cfg.num_ranks, gate, G, KG, H=256)
    idx, w, mask = check_route(res, logits, cfg.num_topk, cfg.num_experts, cfg.num_ranks, gate, G, KG)
    # the plan in the workspace drives dispatch exactly as the layout kernels' plan does
    x = W.draw_hidden(np.random.default_rng(cfg.index + 77), cfg.num_tokens, 256)
    d = H().dispatch_with_plan(res, x)
    offs, send_row, n = O.assign_slots(mask)
    assert np.array_equal(d["send_row"], send_row)
    assert np.array_equal(d["rank_offsets"], offs)
    assert int(d["num_recv"][0]) == n
    src, ridx, rw = O.dispatch_metadata(idx, res["topk_w"], cfg.num_experts, cfg.num_ranks, send_row, n)
    assert np.array_equal(d["recv_src_idx"][:n], src)
    assert np.array_equal(d["recv_topk_idx"][:n], ridx)
    assert np.array_equal(d["recv_topk_w"][:n].view(np.uint32), rw.view(np.uint32))
    assert np.array_equal(d["recv_x"][:n], O.dispatch_rows_bf16(x, src))


def _tie_heavy(rng, T, E):
    x = (rng.integers(-6, 7, size=(T, E)) * 0.5).astype(np.float32)
    zero = x == 0
    x[zero & (rng.random((T, E)) < 0.5)] = np.float32(-0.0)
    return x


EDGES = [  # (label, T, E, k, R, gate, G, KG, ties, misalign)
    ("one token", 1, 256, 8, 8, "softmax", 1, 1, False, False),
    ("fused, ragged chunk", 77, 64, 6, 4, "sigmoid", 1, 1, True, False),
    ("fused maximum", 128, 256, 8, 8, "sigmoid", 8, 4, True, False),
    ("multi-block, ragged", 129, 256, 8, 8, "softmax", 1, 1, True, False),
    ("multi-block, groups of 2 lanes", 700, 128, 5, 16, "softmax", 4, 2, True, False),
    ("E = 8, k = E", 90, 8, 8, 2, "softmax", 2, 2, False, False),
    ("k = 1", 300, 32, 1, 4, "sigmoid", 1, 1, True, False),
    ("k = 16, two slots per lane", 260, 256, 16, 8, "softmax", 8, 4, False, False),
    ("k = 9", 150, 64, 9, 8, "sigmoid", 2, 1, True, False),
    ("scalar loads (V = 3)", 200, 24, 4, 6, "softmax", 1, 1, True, False),
    ("scalar loads (V = 5), R = 5", 65, 40, 3, 5, "sigmoid", 4, 2, True, False),
    ("misaligned logits", 300, 256, 8, 8, "softmax", 8, 4, False, True),
    ("E = 512 (V = 64)", 200, 512, 8, 8, "softmax", 8, 3, False, False),
    ("E = 512, fused", 40, 512, 12, 64, "sigmoid", 1, 1, True, False),
    ("E = 264 (V = 33)", 96, 264, 7, 8, "softmax", 1, 1, True, False),
    ("one group kept of 8", 500, 256, 8, 32, "softmax", 8, 1, True, False),
    ("R = 64", 1000, 256, 8, 64, "softmax", 8, 4, False, False),
    ("E = 1024", 300, 1024, 8, 16, "softmax", 8, 4, True, False),
    ("8 lanes per token, two slots per lane", 150, 40, 12, 5, "softmax", 1, 1, True, False),
    ("8 lanes per token, multi-block", 1500, 24, 5, 4, "sigmoid", 2, 1, True, False),
    ("E = 4096, multi-block", 1100, 4096, 16, 64, "sigmoid", 4, 2, False, False),
]


def _random_shapes(n: int, seed: int = 0x70E):
    """Seeded router shapes inside the limits: E % 8 == 0, k <= 16, G in {1, 2, 4, 8},
    k <= topk_groups * E / G, R | E."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = 8 * int(rng.integers(1, 129))
        G = int(rng.choice([1, 2, 4, 8]))
        if E % G:
            continue
        KG = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(16, KG * (E // G)) + 1))
        Rs = [r for r in (1, 2, 4, 8, 16, 32, 64) if E % r == 0 and r <= E]
        R = int(rng.choice(Rs))
        T = int(rng.integers(1, 3000))
        gate = "softmax" if rng.random() < 0.5 else "sigmoid"
        ties = bool(rng.random() < 0.5)
        out.append((f"rand{len(out)}_T{T}_E{E}_k{k}_G{G}_KG{KG}_R{R}", T, E, k, R, gate, G, KG, ties, False))
    return out


@pytest.mark.parametrize("case", EDGES + _random_shapes(8), ids=lambda c: c[0])
def test_route_edges(case):
    label, T, E, k, R, gate, G, KG, ties, misalign = case
    _print_case(label, T=T, E=E, k=k, R=R, gate=gate, G=G, KG=KG, ties=ties, misalign=misalign)
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    logits = _tie_heavy(rng, T, E) if ties else rng.standard_normal((T, E)).astype(np.float32)
    res = H().run_route(logits, k, E, R, gate, G, KG, misalign=misalign)
    idx, w, _ = check_route(res, logits, k, E, R, gate, G, KG)
    check_router_properties(logits[:32], res["topk_idx"][:32], res["topk_w"][:32], k, G, KG, gate)


def test_route_empty_batch():
    _print_case("empty batch", T=0)
    res = H().run_route(np.zeros((0, 256), np.float32), 8, 256, 8, "softmax", 8, 4)
    assert (res["tokens_per_rank"] == 0).all() and (res["tokens_per_expert"] == 0).all()


def test_route_extreme_logits():
    """Huge, tiny, subnormal and equal-magnitude logits of both signs: selection stays exact."""
    _print_case("extreme logits", T=256, E=64)
    rng = np.random.default_rng(4242)
    vals = np.array([3e38, -3e38, 1e-45, -1e-45, 1e-38, -1e-38, 0.0, -0.0, 1.0, -1.0, 65504.0, 2.0 ** -126],
                    dtype=np.float32)
    logits = vals[rng.integers(0, vals.size, size=(256, 64))]
    res = H().run_route(logits, 8, 64, 8, "sigmoid", 1, 1)
    idx, _ = RT.route(logits, 8, "sigmoid", 1, 1)
    assert np.array_equal(res["topk_idx"], idx)


def test_route_deterministic():
    cfg = W.CONFIG_BY_NAME["prefill"]
    _print_case("determinism", workload=cfg.name)
    logits = W.config_logits(cfg)
    a = H().run_route(logits, 8, 256, 8, "softmax")
    b = H().run_route(logits, 8, 256, 8, "softmax")
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    assert np.array_equal(a["topk_w"].view(np.uint32), b["topk_w"].view(np.uint32))


def test_route_golden_hand_cases():
    """tests/golden/hand_router.json (ids picked by hand, weights as closed forms) through
    moe_route_layout: ids bit-exact, weights within the fp32 bound of the closed-form values."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_router.json")))
    for case in g["cases"]:
        _print_case("golden", case=case["label"][:40].replace(" ", "_"))
        logits = np.array(case["logits"], np.float32)
        T, E, k, G = logits.shape[0], logits.shape[1], case["k"], case["num_groups"]
        # The router needs E % 8 == 0: pad every group with experts no token can pick (logit -1e30),
        # which leaves the groups, their scores and the picks unchanged; ids map e -> e' below.
        E2 = -(-E // 8) * 8
        L, L2 = E // G, E2 // G
        new_id = np.array([(e // L) * L2 + e % L for e in range(E)])
        padded = np.full((T, E2), -1e30, np.float32)
        padded[:, new_id] = logits
        res = H().run_route(padded, k, E2, 1, case["gate"], G, case["topk_groups"])
        back = {int(n): e for e, n in enumerate(new_id)}
        ids = [[back.get(int(v), -1) for v in row] for row in res["topk_idx"]]
        assert ids == case["topk_idx"], case["label"]
        ref = np.array(case["topk_w"], np.float64)
        rel = np.abs(res["topk_w"].astype(np.float64) - ref) / np.abs(ref)
        assert (rel <= weight_bound(padded, res["topk_idx"], k, case["gate"])).all(), case["label"]
