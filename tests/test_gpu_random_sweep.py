"""Seeded random shapes across the library's limits, beyond the edge lists of the other GPU tests:
layout -> dispatch -> combine (rank counts 1..64 including non-powers of two, T on both sides of the
one-block and 4096-token thresholds, masked ids), the fused router, routing and dispatch in one
kernel, and the low-latency path.  Every case is checked against the oracle with the same helpers
(and bars) as the per-path tests: bit-exact layout, slots, metadata, rows, FP8 codes and scales and
combine; router ids bit-exact and weights within the derived fp32 bound."""
import zlib

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O
from tests import test_gpu_ll as LL
from tests import test_gpu_parity as P
from tests import test_gpu_route_dispatch as RD
from tests import test_gpu_router as RT

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _send_shapes(n, seed=0x5EE9):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16, 24, 32, 64]))
        L = int(rng.integers(1, max(2, 512 // R) + 1))
        E = R * L
        k = int(rng.integers(1, min(E, 32) + 1))
        dtype = "fp8" if rng.random() < 0.5 else "bf16"
        H = 128 * int(rng.integers(1, 9)) if dtype == "fp8" else 8 * int(rng.integers(1, 129))
        T = int(rng.choice([int(rng.integers(0, 1100)), int(rng.integers(1000, 9000))]))
        inv = float(rng.choice([0.0, 0.0, 0.1, 0.5]))
        out.append((f"send{i}_T{T}_H{H}_E{E}_k{k}_R{R}_{dtype}", 3000 + i, T, H, E, k, R, dtype, inv))
    return out


@pytest.mark.parametrize("case", _send_shapes(48), ids=lambda c: c[0])
def test_random_send_and_combine(case):
    name, seed, T, H, E, k, R, dtype, inv = case
    print(f"[case] {name} inv={inv}", flush=True)
    d = W.random_case(seed, T, H, E, k, R, invalid_frac=inv)
    _, _, mask = O.get_dispatch_layout(d["topk_idx"], E, R)
    y = W.draw_expert_outputs(np.random.default_rng(seed), max(int(mask.sum()), 1), H)
    _, exact = P.run_case(d["x"], d["topk_idx"], d["topk_w"], E, R, dtype, y=y)
    assert exact


def _route_dispatch_shapes(n, seed=0xD15):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = 8 * int(rng.integers(1, 65))
        G = int(rng.choice([1, 2, 4, 8]))
        if E % G:
            continue
        KG = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(16, KG * (E // G)) + 1))
        R = int(rng.choice([r for r in (1, 2, 4, 8, 16, 32, 64) if E % r == 0]))
        T = int(rng.integers(1, 1100))
        dtype = "fp8" if rng.random() < 0.5 else "bf16"
        H = 128 * int(rng.integers(1, 9)) if dtype == "fp8" else 8 * int(rng.integers(1, 129))
        gate = "softmax" if rng.random() < 0.5 else "sigmoid"
        ties = bool(rng.random() < 0.5)
        out.append((f"rd{len(out)}_T{T}_H{H}_E{E}_k{k}_R{R}_G{G}_KG{KG}_{dtype}_{gate}", T, H, E, k, R, dtype, gate,
                    G, KG, ties))
    return out


@pytest.mark.parametrize("case", _route_dispatch_shapes(24), ids=lambda c: c[0])
def test_random_route_dispatch(case):
    label, T, H, E, k, R, dtype, gate, G, KG, ties = case
    print(f"[case] {label} ties={ties}", flush=True)
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    logits = RT._tie_heavy(rng, T, E) if ties else rng.standard_normal((T, E)).astype(np.float32)
    x = W.draw_hidden(rng, T, H)
    res = RD.H().run_route_dispatch(logits, x, k, E, R, dtype, gate, G, KG)
    RD.check_send(res, logits, x, k, E, R, dtype, gate, G, KG)
    RD.check_same_as_two_calls(res, logits, x, k, E, R, dtype, gate, G, KG)


@pytest.mark.parametrize("case", RT._random_shapes(24, seed=0xA11), ids=lambda c: c[0])
def test_random_router(case):
    label, T, E, k, R, gate, G, KG, ties, misalign = case
    print(f"[case] router {label} {gate} ties={ties}", flush=True)
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    logits = RT._tie_heavy(rng, T, E) if ties else rng.standard_normal((T, E)).astype(np.float32)
    res = RT.H().run_route(logits, k, E, R, gate, G, KG, misalign=misalign)
    RT.check_route(res, logits, k, E, R, gate, G, KG)


@pytest.mark.parametrize("case", LL._ll_random_shapes(24, seed=0xB22), ids=lambda c: c[0])
def test_random_low_latency(case):
    LL._ll_edge(case)
