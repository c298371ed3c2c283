"""GPU parity of the backward kernels against the oracle.

grad_y, grad_x and the dispatch weight gradients are bit-exact (same fp32 order as the oracle);
the combine weight gradients are fp32 dot products over H, checked against the exact fp64 value
within the fp32 summation bound (H/64 + 16) * 2^-24 * sum |g * y|.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O
from oracle.numerics import bf16_bits_to_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(a):
    from tests.gpu_harness import to_dev_bf16
    if a.dtype == np.uint16:
        return to_dev_bf16(a) if a.size else torch.empty(a.shape, dtype=torch.bfloat16, device="cuda")
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_backward_case(T, H, E, k, R, seed, invalid_frac=0.0, routing_cfg=None):
    import combine_get_dispatch_07_amd as moe
    from tests.gpu_harness import POISON, bf16_to_np
    print(f"[case] backward T={T} H={H} E={E} k={k} R={R}", flush=True)
    if routing_cfg is not None:
        d = W.make_inputs(routing_cfg)
    else:
        d = W.random_case(seed, T, H, E, k, R, invalid_frac=invalid_frac)
    idx, w = d["topk_idx"], d["topk_w"]
    _, _, mask = O.get_dispatch_layout(idx, E, R)
    _, send_row, n = O.assign_slots(mask)
    rng = np.random.default_rng(seed)
    g = W.draw_expert_outputs(rng, T, H)
    y = W.draw_expert_outputs(rng, n, H)
    shape = moe.MoeShape(T, H, k, E, R)
    gy_d = torch.empty((n + 2, H), dtype=torch.bfloat16, device="cuda")
    gy_d.view(torch.uint8).fill_(POISON)
    gw_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_combine_backward(shape, _dev(g), _dev(y), _dev(idx), _dev(w), _dev(send_row), gy_d, gw_d, num_y_rows=n)
    torch.cuda.synchronize()
    gy_ref, gw_ref = O.combine_backward(g, y, idx, w, send_row, E, R, n)
    gy = bf16_to_np(gy_d)
    assert np.array_equal(gy[:n], gy_ref)
    assert (gy[n:].view(np.uint16) == 0x7B7B).all()
    gw = gw_d.cpu().numpy().astype(np.float64)
    valid, rank = O.expert_ranks(idx, E, R)
    mag = np.zeros_like(gw_ref)
    gf = bf16_bits_to_f32(g).astype(np.float64)
    yf = bf16_bits_to_f32(y).astype(np.float64)
    for j in range(k):
        tt = np.nonzero(valid[:, j])[0]
        mag[tt, j] = np.abs(gf[tt] * yf[send_row[tt, rank[tt, j]]]).sum(axis=1)
    bound = (H / 64 + 16) * 2.0 ** -24 * mag + 1e-30
    assert (np.abs(gw - gw_ref) <= bound).all()
    assert (gw[~valid] == 0).all()

    grw = rng.standard_normal((n, k)).astype(np.float32)
    gx_d = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    gtw_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_dispatch_backward(shape, _dev(y), _dev(idx), _dev(send_row), gx_d, _dev(grw), gtw_d)
    torch.cuda.synchronize()
    gx_ref, gtw_ref = O.dispatch_backward(y, grw, idx, send_row, E, R)
    assert np.array_equal(bf16_to_np(gx_d), gx_ref)
    assert np.array_equal(gtw_d.cpu().numpy().view(np.uint32), gtw_ref.view(np.uint32))


def test_backward_prefill_workload():
    cfg = W.CONFIG_BY_NAME["prefill"]
    run_backward_case(cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.num_topk, cfg.num_ranks, 5, routing_cfg=cfg)


@pytest.mark.parametrize("case", [
    # T, H, E, k, R, seed, invalid_frac
    (1, 256, 16, 4, 4, 1, 0.0),
    (300, 512, 64, 6, 16, 2, 0.2),     # R > 8: rank rows compacted, min(k, R) = 6 terms
    (200, 256, 64, 12, 8, 3, 0.1),     # k > 8
    (129, 136, 32, 4, 8, 4, 0.0),      # ragged hidden
    (500, 256, 16, 4, 4, 5, 0.7),      # mostly invalid ids
    (400, 256, 256, 8, 64, 6, 0.1),    # R = 64, the group-limited shape
    (300, 256, 128, 16, 32, 7, 0.1),   # min(k, R) = 16: compacted rows in two batches
    (100, 128, 64, 32, 64, 8, 0.0),    # k = 32: widest combine backward, four batches
    (150, 136, 64, 32, 4, 9, 0.1),     # k = 32 on 4 ranks: eight slots share each y row, ragged hidden
    # larger batches, k <= 8
    (1024, 512, 64, 6, 16, 10, 0.1),   # exactly one token per wave on the full chip
    (2500, 136, 64, 8, 8, 11, 0.2),    # ragged hidden, tokens not a multiple of the waves
    (1100, 64, 16, 1, 4, 12, 0.0),     # one slice per token (8 of 64 lanes in range), k = 1
    (3001, 256, 256, 8, 64, 13, 0.6),  # R = 64, mostly invalid ids
    (4099, 1024, 32, 4, 4, 14, 0.0),   # two slices, duplicate ranks within a token
])
def test_backward_edges(case):
    run_backward_case(*case)


def _bwd_random_shapes(n: int, seed: int = 0xB4C):
    """Seeded shapes inside the limits: R | E, k <= min(E, 32), H % 8 == 0."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 32, 64]))
        L = int(rng.integers(1, max(2, 256 // R) + 1))
        E = R * L
        k = int(rng.integers(1, min(E, 32) + 1))
        H = 8 * int(rng.integers(1, 161))
        T = int(rng.integers(1, 1500))
        inv = float(rng.choice([0.0, 0.1, 0.4]))
        out.append((T, H, E, k, R, 300 + i, inv))
    return out


@pytest.mark.parametrize("case", _bwd_random_shapes(8), ids=lambda c: "T{}_H{}_E{}_k{}_R{}".format(*c[:5]))
def test_backward_random_shapes(case):
    run_backward_case(*case)


def test_combine_backward_without_expert_rows():
    """num_y_rows = 0 (y and grad_y empty): nothing is written to grad_y and every weight gradient is +0."""
    import combine_get_dispatch_07_amd as moe
    T, H, E, k, R = 300, 256, 16, 4, 4
    print(f"[case] backward without expert rows T={T} H={H}", flush=True)
    d = W.random_case(21, T, H, E, k, R)
    _, _, mask = O.get_dispatch_layout(d["topk_idx"], E, R)
    _, send_row, _ = O.assign_slots(mask)
    g = W.draw_expert_outputs(np.random.default_rng(21), T, H)
    empty = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    gw_d = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    shape = moe.MoeShape(T, H, k, E, R)
    moe.moe_combine_backward(shape, _dev(g), empty, _dev(d["topk_idx"]), _dev(d["topk_w"]), _dev(send_row), empty,
                             gw_d, num_y_rows=0)
    torch.cuda.synchronize()
    gw = gw_d.cpu().numpy()
    assert (gw.view(np.uint32) == 0).all()


def test_dispatch_backward_rank_order_on_gpu():
    """Hand case whose bf16 result depends on the order the rank rows are added (see
    test_oracle_backward.test_dispatch_backward_rank_order): ascending order gives exactly 1.0."""
    import combine_get_dispatch_07_amd as moe
    from oracle.numerics import f32_to_bf16_bits_rne
    from tests.gpu_harness import bf16_to_np
    print("[case] dispatch backward rank order", flush=True)
    idx = np.array([[0, 1, 2, 3]], np.int32)
    send_row = np.array([[0, 1, 2, 3]], np.int32)
    rows = f32_to_bf16_bits_rne(np.array([[1.0] * 8, [2.0 ** -8] * 8, [2.0 ** -24] * 8, [2.0 ** -24] * 8],
                                         np.float32))
    shape = moe.MoeShape(1, 8, 4, 4, 4)
    gx_d = torch.empty((1, 8), dtype=torch.bfloat16, device="cuda")
    gtw_d = torch.empty((1, 4), dtype=torch.float32, device="cuda")
    moe.moe_dispatch_backward(shape, _dev(rows), _dev(idx), _dev(send_row), gx_d, _dev(np.zeros((4, 4), np.float32)),
                              gtw_d)
    torch.cuda.synchronize()
    assert (bf16_to_np(gx_d) == 0x3F80).all()


def test_combine_backward_slot_order_on_gpu():
    """Hand case whose bf16 grad_y depends on the order a rank's slots are added (see
    test_oracle_backward.test_combine_backward_slot_order): ascending order gives exactly 1.0."""
    import combine_get_dispatch_07_amd as moe
    from oracle.numerics import f32_to_bf16_bits_rne
    from tests.gpu_harness import bf16_to_np
    print("[case] combine backward slot order", flush=True)
    idx = np.array([[0, 1, 2, 3]], np.int32)
    w = np.array([[1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24]], np.float32)
    ones = f32_to_bf16_bits_rne(np.ones((1, 8), np.float32))
    shape = moe.MoeShape(1, 8, 4, 4, 1)
    gy_d = torch.empty((1, 8), dtype=torch.bfloat16, device="cuda")
    gw_d = torch.empty((1, 4), dtype=torch.float32, device="cuda")
    moe.moe_combine_backward(shape, _dev(ones), _dev(ones), _dev(idx), _dev(w), _dev(np.zeros((1, 1), np.int32)), gy_d,
                             gw_d, num_y_rows=1)
    torch.cuda.synchronize()
    assert (bf16_to_np(gy_d) == 0x3F80).all()


def test_golden_backward_on_gpu():
    """tests/golden/hand_backward.json (on the forward fixture hand_layout_dispatch_combine.json)
    through moe_combine_backward / moe_dispatch_backward.  The fixture's 2-channel rows are repeated
    to 8 channels, so the weight gradients (dot products over the channels) are 4 times the
    fixture's; every value involved is small and exact in fp32."""
    import json
    import os
    import combine_get_dispatch_07_amd as moe
    from oracle.numerics import f32_to_bf16_bits_rne
    from tests.gpu_harness import bf16_to_np
    print("[case] backward golden hand case", flush=True)
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    fwd = json.load(open(os.path.join(here, "hand_layout_dispatch_combine.json")))
    ex = json.load(open(os.path.join(here, "hand_backward.json")))["expect"]
    E, R = fwd["num_experts"], fwd["num_ranks"]
    idx = np.array(fwd["topk_idx"], np.int32)
    w = np.array(fwd["topk_w"], np.float32)
    send_row = np.array(fwd["expect"]["send_row"], np.int32)
    n = fwd["expect"]["num_recv"]
    T, k, Hd = idx.shape[0], idx.shape[1], 8
    g = f32_to_bf16_bits_rne(np.tile(np.array([[t + 1, -(t + 1)] for t in range(T)], np.float32), (1, Hd // 2)))
    y = f32_to_bf16_bits_rne(np.tile(np.array([[i + 1, -(i + 1) / 2] for i in range(n)], np.float32), (1, Hd // 2)))
    grw = np.array([[10 * i + j for j in range(k)] for i in range(n)], np.float32)
    shape = moe.MoeShape(T, Hd, k, E, R)
    gy_d = torch.empty((n, Hd), dtype=torch.bfloat16, device="cuda")
    gw_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_combine_backward(shape, _dev(g), _dev(y), _dev(idx), _dev(w), _dev(send_row), gy_d, gw_d, num_y_rows=n)
    gx_d = torch.empty((T, Hd), dtype=torch.bfloat16, device="cuda")
    gtw_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_dispatch_backward(shape, _dev(y), _dev(idx), _dev(send_row), gx_d, _dev(grw), gtw_d)
    torch.cuda.synchronize()
    tile = lambda a: f32_to_bf16_bits_rne(np.tile(np.array(a, np.float32), (1, Hd // 2)))  # noqa: E731
    assert np.array_equal(bf16_to_np(gy_d), tile(ex["grad_y"]))
    assert gw_d.cpu().numpy().tolist() == (4 * np.array(ex["grad_w"], np.float32)).tolist()
    assert np.array_equal(bf16_to_np(gx_d), tile(ex["grad_x"]))
    assert gtw_d.cpu().numpy().tolist() == ex["grad_topk_w"]
