"""GPU parity of moe_route_dispatch: routing, layout and dispatch in one call (one kernel up to 1024
tokens), through the C ABI, against the oracles.

Bar: expert ids bit-exact against oracle/router.py and weights within the router's derived fp32 bound
(tests/test_gpu_router.py); layout, slots, metadata, bf16 rows, FP8 codes and scales bit-exact
against the dispatch oracle applied to those ids and weights; receive rows at or beyond num_recv
untouched; and every output bit-identical to moe_route_layout followed by moe_dispatch.
"""
import zlib

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O
from tests.test_gpu_router import _gate_of, _tie_heavy, check_route

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness  # noqa: F401  (loads the HIP library; fails loudly if missing)


def H():
    from tests import gpu_harness
    return gpu_harness


def check_send(res, logits, x, k, E, R, dtype, gate, G, KG):
    """Routing against the router oracle, then everything the dispatch writes against the dispatch
    oracle on the routed ids and weights."""
    idx, _, mask = check_route(res, logits, k, E, R, gate, G, KG)
    w = res["topk_w"]
    ref = O.run_all(x, idx, w, E, R, dtype)
    n = int(ref["num_recv"])
    assert int(res["num_recv"][0]) == n
    for key in ("rank_offsets", "send_row"):
        assert np.array_equal(res[key], ref[key]), key
    for key in ("recv_src_idx", "recv_topk_idx", "recv_x"):
        assert np.array_equal(res[key][:n], ref[key]), key
    assert np.array_equal(res["recv_topk_w"][:n].view(np.uint32), ref["recv_topk_w"].view(np.uint32))
    if dtype == "fp8":
        assert np.array_equal(res["recv_scales"][:n].view(np.uint32), ref["recv_scales"].view(np.uint32))
    for key in ("recv_src_idx", "recv_topk_idx", "recv_topk_w", "recv_x"):
        assert (res[key][n:].view(np.uint8) == H().POISON).all(), f"{key} written beyond num_recv"
    return n


def check_same_as_two_calls(res, logits, x, k, E, R, dtype, gate, G, KG):
    """moe_route_layout then moe_dispatch on the same inputs give the same bytes."""
    two = H().run_route(logits, k, E, R, gate, G, KG, H=x.shape[1])
    d = H().dispatch_with_plan(two, x, dtype)
    for key in ("topk_idx", "topk_w", "tokens_per_rank", "tokens_per_expert", "is_token_in_rank"):
        assert np.array_equal(res[key].view(np.uint8), two[key].view(np.uint8)), key
    n = int(res["num_recv"][0])
    for key in ("rank_offsets", "send_row", "num_recv"):
        assert np.array_equal(res[key], d[key]), key
    for key in ("recv_src_idx", "recv_topk_idx", "recv_topk_w", "recv_x"):
        assert np.array_equal(res[key][:n].view(np.uint8), d[key][:n].view(np.uint8)), key


@pytest.mark.parametrize("cfg", W.CONFIGS, ids=lambda c: c.name)
def test_route_dispatch_workloads(cfg):
    """Every workload's own logits and hidden rows at full size (one kernel for tiny and decode)."""
    gate, G, KG = _gate_of(cfg)
    print(f"[case] route_dispatch workload={cfg.name} T={cfg.num_tokens} {cfg.dispatch_dtype}", flush=True)
    logits = W.config_logits(cfg)
    x = W.make_inputs(cfg)["x"]
    res = H().run_route_dispatch(logits, x, cfg.num_topk, cfg.num_experts, cfg.num_ranks, cfg.dispatch_dtype, gate,
                                 G, KG)
    check_send(res, logits, x, cfg.num_topk, cfg.num_experts, cfg.num_ranks, cfg.dispatch_dtype, gate, G, KG)
    if cfg.num_tokens <= 1024:
        check_same_as_two_calls(res, logits, x, cfg.num_topk, cfg.num_experts, cfg.num_ranks, cfg.dispatch_dtype,
                                gate, G, KG)


EDGES = [  # (label, T, H, E, k, R, dtype, gate, G, KG, ties)
    ("one token", 1, 256, 256, 8, 8, "fp8", "sigmoid", 1, 1, False),
    ("ragged first chunk", 17, 136, 64, 6, 4, "bf16", "softmax", 1, 1, True),
    ("one full chunk", 64, 512, 128, 4, 8, "bf16", "softmax", 4, 2, True),
    ("two chunks, one token in the second", 65, 384, 256, 8, 8, "fp8", "sigmoid", 8, 4, True),
    ("8 lanes per token (E % 16 != 0)", 300, 256, 24, 4, 6, "bf16", "softmax", 1, 1, True),
    ("8 lanes, two slots per lane", 200, 128, 40, 12, 8, "fp8", "softmax", 2, 1, False),
    ("R = 64", 500, 256, 256, 8, 64, "bf16", "softmax", 8, 4, False),
    ("FP8 at hidden 7168, two 64-piece groups per wave", 1000, 7168, 256, 8, 8, "fp8", "sigmoid", 1, 1, False),
    ("largest one-kernel batch", 1024, 7168, 256, 8, 32, "fp8", "softmax", 8, 4, False),
    ("bf16 hidden 7168", 333, 7168, 256, 8, 8, "bf16", "softmax", 1, 1, False),
    ("k = 1", 250, 64, 32, 1, 4, "bf16", "sigmoid", 1, 1, True),
    ("just above one kernel", 1025, 256, 64, 6, 8, "fp8", "softmax", 1, 1, True),
]


@pytest.mark.parametrize("case", EDGES, ids=lambda c: c[0])
def test_route_dispatch_edges(case):
    label, T, Hd, E, k, R, dtype, gate, G, KG, ties = case
    print(f"[case] route_dispatch edge '{label}' T={T} H={Hd} E={E} k={k} R={R} {dtype}", flush=True)
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    logits = _tie_heavy(rng, T, E) if ties else rng.standard_normal((T, E)).astype(np.float32)
    x = W.draw_hidden(rng, T, Hd)
    res = H().run_route_dispatch(logits, x, k, E, R, dtype, gate, G, KG)
    check_send(res, logits, x, k, E, R, dtype, gate, G, KG)
    check_same_as_two_calls(res, logits, x, k, E, R, dtype, gate, G, KG)


def test_route_dispatch_repeated_calls_and_shapes_on_one_workspace():
    """Back-to-back calls on one workspace (its sync words must come back to zero after each) give the
    same bytes; so does a smaller batch afterwards on a workspace sized for the larger one."""
    cfg = W.CONFIG_BY_NAME["decode"]
    gate, G, KG = _gate_of(cfg)
    logits = W.config_logits(cfg)
    x = W.make_inputs(cfg)["x"]
    print("[case] route_dispatch repeated calls", flush=True)
    once = H().run_route_dispatch(logits, x, cfg.num_topk, cfg.num_experts, cfg.num_ranks, "fp8", gate, G, KG)
    many = H().run_route_dispatch(logits, x, cfg.num_topk, cfg.num_experts, cfg.num_ranks, "fp8", gate, G, KG,
                                  calls=5)
    for key in ("topk_idx", "send_row", "recv_x", "recv_scales", "num_recv"):
        assert np.array_equal(once[key], many[key]), key
    # the sync words (four, 4 KiB apart), then the expert and the rank accumulators (each rounded up
    # to 256 bytes): the first region of the workspace, zero between calls
    ws = many["_dev"]["lay"]["workspace"].view(torch.int32)
    up = lambda n: (n + 255) // 256 * 256  # noqa: E731
    words = (4 * 4096 + up(4 * cfg.num_experts) + up(4 * cfg.num_ranks)) // 4
    assert int(ws[:words].abs().sum().item()) == 0, "sync words or accumulators not reset"
    small = H().run_route_dispatch(logits[:50], x[:50], cfg.num_topk, cfg.num_experts, cfg.num_ranks, "fp8", gate, G,
                                   KG)
    check_send(small, logits[:50], x[:50], cfg.num_topk, cfg.num_experts, cfg.num_ranks, "fp8", gate, G, KG)


def test_route_dispatch_empty_batch():
    print("[case] route_dispatch empty", flush=True)
    res = H().run_route_dispatch(np.zeros((0, 64), np.float32), np.zeros((0, 256), np.uint16), 4, 64, 8, "bf16")
    assert (res["tokens_per_rank"] == 0).all() and (res["tokens_per_expert"] == 0).all()
    assert (res["rank_offsets"] == 0).all() and int(res["num_recv"][0]) == 0
