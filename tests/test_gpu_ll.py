"""GPU parity of the low-latency (per-expert) layout: moe_dispatch_ll / moe_combine_ll against the oracle.

Bar: recv_count, slot_pos, recv_src_idx, bf16 rows, FP8 bytes and scales bit-exact; rows at or
beyond recv_count[e] untouched; combine within 1 bf16 ulp and expected bit-exact.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O
from tests.checks import within_one_bf16_ulp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def G():
    from tests import gpu_harness
    return gpu_harness


def ll_y(count, cap, H, seed):
    """Expert outputs in the per-expert layout: random rows where tokens were received, zeros elsewhere."""
    E = count.size
    y = np.zeros((E, cap, H), np.uint16)
    rows = W.draw_expert_outputs(np.random.default_rng(seed), int(count.sum()), H)
    i = 0
    for e in range(E):
        y[e, :count[e]] = rows[i:i + count[e]]
        i += count[e]
    return y


def run_ll_case(x, idx, w, E, cap, dtype, seed=0):
    print(f"[case] ll T={x.shape[0]} H={x.shape[1]} E={E} k={idx.shape[1]} cap={cap} {dtype}", flush=True)
    res = G().run_dispatch_ll(x, idx, E, cap, dtype)
    count, slot_pos = O.ll_layout(idx, E)
    assert np.array_equal(res["recv_count"], count)
    assert np.array_equal(res["slot_pos"], slot_pos)
    src = res["recv_src_idx"]
    for e in range(E):
        n = count[e]
        tok = np.nonzero((idx == e).any(axis=1))[0]
        assert np.array_equal(src[e, :n], tok), e
        assert (src[e, n:].view(np.uint32) == 0x7B7B7B7B).all()
        assert (res["recv_x"][e, n:].view(np.uint8) == 0x7B).all()
    # every written row: the oracle's per-row payload (bit copy, or FP8 codes and scales, which
    # depend on the source row alone, so each source token is quantised once)
    ee, pp = np.nonzero(np.arange(cap)[None, :] < count[:, None])
    tt = src[ee, pp]
    if dtype == "bf16":
        assert np.array_equal(res["recv_x"][ee, pp], x[tt])
    else:
        q, s = O.quantize_fp8_blocks(x)
        bad = np.nonzero((res["recv_x"][ee, pp] != q[tt]).any(axis=1))[0]
        assert bad.size == 0, f"fp8 bytes differ in {bad.size} rows, first (expert, row) {ee[bad[:1]]}, {pp[bad[:1]]}"
        assert np.array_equal(res["recv_scales"][ee, pp].view(np.uint32), s[tt].view(np.uint32))
    y = ll_y(count, cap, x.shape[1], seed)
    dev = res["_dev"]
    out = G().run_combine_ll(res["shape"], y, dev["idx"], w, dev["d"]["slot_pos"])
    ref = O.ll_combine(y, idx, w, slot_pos, E)
    assert within_one_bf16_ulp(out, ref).all()
    assert np.array_equal(out, ref)
    return res


def test_ll_decode_workload():
    cfg = W.CONFIG_BY_NAME["decode"]
    d = W.make_inputs(cfg)
    run_ll_case(d["x"], d["topk_idx"], d["topk_w"], cfg.num_experts, cfg.num_tokens, "fp8", seed=1)


def _ll_random_shapes(n: int, seed: int = 0x11ED):
    """Seeded shapes for the per-expert layout, kept to E * cap * H <= 2^25 elements per buffer."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.integers(1, 513))
        k = int(rng.integers(1, min(E, 32) + 1))
        dtype = "fp8" if rng.random() < 0.5 else "bf16"
        H = 128 * int(rng.integers(1, 9)) if dtype == "fp8" else 8 * int(rng.integers(1, 129))
        T = int(rng.integers(1, 1300))
        extra = int(rng.integers(0, 4))
        if E * (T + extra) * H > 1 << 25:
            continue
        inv = float(rng.choice([0.0, 0.1, 0.4]))
        out.append((f"rand{len(out)}_T{T}_H{H}_E{E}_k{k}_{dtype}", 200 + len(out), T, H, E, k, dtype, inv, extra))
    return out


LL_RANDOM_SHAPES = _ll_random_shapes(8)


@pytest.mark.parametrize("case", LL_RANDOM_SHAPES, ids=lambda c: c[0])
def test_ll_random_shapes(case):
    _ll_edge(case)


def _ll_edge(case):
    name, seed, T, H, E, k, dtype, inv, extra = case
    d = W.random_case(seed, T, H, E, k, 1, invalid_frac=inv)
    idx = d["topk_idx"].copy()
    if T > 3:
        idx[2, :2] = max(int(idx[2, 0]), 0)  # one token names an expert twice
    run_ll_case(d["x"], idx, d["topk_w"], E, T + extra, dtype, seed=seed)


@pytest.mark.parametrize("case", [
    # name, seed, T, H, E, k, dtype, invalid_frac, capacity extra
    ("small_bf16", 1, 37, 256, 16, 4, "bf16", 0.2, 5),
    ("one_token", 2, 1, 128, 8, 2, "fp8", 0.0, 0),
    ("multiblock", 3, 1100, 256, 64, 6, "bf16", 0.1, 0),
    ("many_experts", 4, 200, 128, 4096, 32, "fp8", 0.1, 0),
    ("fused_wide", 5, 1024, 128, 512, 8, "fp8", 0.0, 0),
    ("ragged_hidden", 6, 300, 136, 32, 4, "bf16", 0.0, 3),
    ("two_pass_wide_hidden", 7, 64, 16896, 16, 4, "bf16", 0.1, 0),  # hidden > 16384: two-pass path
    ("small_last_batch", 8, 129, 256, 64, 8, "fp8", 0.0, 1),        # one token in the last 64-token batch
    # two-pass FP8 above 1024 tokens at each dispatch width (the widest of 14, 7, 4, 2 64-piece
    # groups that still gives >= 4096 waves): hidden 7168 -> 4 groups at 1100 tokens, 7 at 2100,
    # 14 at 4100; hidden 1024 (2 groups per row) -> 2 at 4100
    ("fp8_two_pass_width4", 9, 1100, 7168, 32, 8, "fp8", 0.05, 0),
    ("fp8_two_pass_width7", 10, 2100, 7168, 32, 8, "fp8", 0.0, 0),
    ("fp8_two_pass_width14", 11, 4100, 7168, 8, 4, "fp8", 0.0, 2),
    ("fp8_two_pass_width2", 12, 4100, 1024, 8, 4, "fp8", 0.0, 0),
])
def test_ll_edges(case):
    _ll_edge(case)


def test_ll_empty_and_capacity_error():
    import combine_get_dispatch_07_amd as moe
    res = G().run_dispatch_ll(np.zeros((0, 256), np.uint16), np.zeros((0, 4), np.int32), 16, 0, "bf16")
    assert (res["recv_count"] == 0).all()
    x = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((8, 4), dtype=torch.int32, device="cuda")
    shape = moe.MoeShape(8, 256, 4, 16, 1)
    d = moe.alloc_dispatch_ll(shape, "bf16", capacity=7)
    with pytest.raises(moe.MoeError) as e:
        moe.run_dispatch_ll(shape, "bf16", x, idx, d)
    assert e.value.code == 2


def test_combine_with_no_expert_rows_is_zero():
    d = W.random_case(9, 50, 256, 16, 4, 4)
    from tests import gpu_harness as H
    res = H.run_layout_dispatch(d["x"], d["topk_idx"], d["topk_w"], 16, 4, "bf16")
    out = H.run_combine(res["shape"], np.zeros((0, 256), np.uint16), res["_dev"]["idx"], res["_dev"]["w"],
                        res["_dev"]["d"]["send_row"], num_y_rows=0)
    assert (out == 0).all()


def test_ll_combine_golden_fp32_order():
    """tests/golden/hand_combine_fp32_order.json through the per-expert layout.  There E = R (one
    expert per rank), so expert e's buffer holds exactly rank e's receive segment, in the same token
    order: the expected bf16 outputs, which show the fp32 summation order and the absence of fused
    multiply-add, are the same."""
    import json
    import os
    import combine_get_dispatch_07_amd as moe
    from oracle.numerics import f32_to_bf16_bits_rne
    print("[case] ll golden fp32 order", flush=True)
    g = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                    "hand_combine_fp32_order.json")))
    E = g["num_experts"]
    assert g["num_ranks"] == E
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_w"], np.float32)
    T, Hd = idx.shape[0], 8
    count, slot_pos = O.ll_layout(idx, E)
    rows = np.array(g["y_rows"], np.float32)
    y = np.zeros((E, T, Hd), np.uint16)
    first = np.concatenate([[0], np.cumsum(count)[:-1]])
    for e in range(E):
        y[e, :count[e]] = f32_to_bf16_bits_rne(rows[first[e]:first[e] + count[e], None] * np.ones((1, Hd), np.float32))
    shape = moe.MoeShape(T, Hd, idx.shape[1], E, 1)
    out = G().run_combine_ll(shape, y, torch.from_numpy(idx).cuda(), w, torch.from_numpy(slot_pos).cuda())
    expect = f32_to_bf16_bits_rne(np.array(g["expect_out"], np.float32)[:, None] * np.ones((1, Hd), np.float32))
    assert np.array_equal(out, expect)
    assert np.array_equal(out, O.ll_combine(y, idx, w, slot_pos, E))


def test_ll_golden_hand_case():
    """tests/golden/hand_low_latency.json through moe_dispatch_ll / moe_combine_ll, against the values
    derived by hand (the fixture's 2-channel expert outputs repeated to 8 channels)."""
    import json
    import os
    from oracle.numerics import f32_to_bf16_bits_rne
    print("[case] ll golden hand case", flush=True)
    g = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_low_latency.json")))
    E, cap, ex = g["num_experts"], g["capacity"], g["expect"]
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_w"], np.float32)
    T = idx.shape[0]
    x = f32_to_bf16_bits_rne(np.arange(T * 128, dtype=np.float32).reshape(T, 128) / 64)
    res = G().run_dispatch_ll(x, idx, E, cap, "bf16")
    assert res["recv_count"].tolist() == ex["recv_count"]
    assert res["slot_pos"].tolist() == ex["slot_pos"]
    for e in range(E):
        n = ex["recv_count"][e]
        assert res["recv_src_idx"][e, :n].tolist() == ex["recv_src_idx"][e][:n], e
        assert np.array_equal(res["recv_x"][e, :n], x[ex["recv_src_idx"][e][:n]]), e
    Hd = 8
    y = np.zeros((E, cap, Hd), np.float32)
    for e in range(E):
        for p in range(cap):
            y[e, p] = [e + 1 + 8 * p, -(e + 1) / 2 - p] * (Hd // 2)
    import combine_get_dispatch_07_amd as moe
    shape = moe.MoeShape(T, Hd, idx.shape[1], E, 1)
    out = G().run_combine_ll(shape, f32_to_bf16_bits_rne(y), res["_dev"]["idx"], w, res["_dev"]["d"]["slot_pos"])
    expect = f32_to_bf16_bits_rne(np.tile(np.array(ex["combine_out"], np.float32), (1, Hd // 2)))
    assert np.array_equal(out, expect)
