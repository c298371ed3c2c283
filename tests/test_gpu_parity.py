"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: layout, slots, metadata, bf16 rows, FP8 bytes and scales bit-exact;
combine within 1 bf16 ulp (and, since both sides sum in the same fp32 order
without fused multiply-add, expected bit-exact).  Receive buffers carry poison
and guard rows: rows at or beyond num_recv must stay untouched.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O
from oracle.numerics import E4M3_MAGNITUDES, bf16_bits_to_f32, f32_to_bf16_bits_rne
from tests.checks import (check_combine_bound, check_fp8_block_properties, check_layout_invariants,
                          check_slot_invariants, within_one_bf16_ulp)

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


def check_layout_and_slots(res, idx, E, R):
    tpr, tpe, mask = O.get_dispatch_layout(idx, E, R)
    assert np.array_equal(res["tokens_per_expert"], tpe)
    assert np.array_equal(res["tokens_per_rank"], tpr)
    assert np.array_equal(res["is_token_in_rank"], mask)
    offs, send_row, n = O.assign_slots(mask)
    assert np.array_equal(res["rank_offsets"], offs)
    assert int(res["num_recv"][0]) == n
    assert np.array_equal(res["send_row"], send_row)
    return send_row, n


def check_metadata_and_guards(res, idx, w, E, R, send_row, n):
    src, ridx, rw = O.dispatch_metadata(idx, w, E, R, send_row, n)
    assert np.array_equal(res["recv_src_idx"][:n], src)
    assert np.array_equal(res["recv_topk_idx"][:n], ridx)
    assert np.array_equal(res["recv_topk_w"][:n].view(np.uint32), rw.view(np.uint32))
    poison32 = np.uint32(0x7B7B7B7B)
    for key in ("recv_src_idx", "recv_topk_idx", "recv_topk_w"):
        tail = res[key][n:].view(np.uint32)
        assert (tail == poison32).all(), f"{key} written beyond num_recv"
    tail = res["recv_x"][n:].view(np.uint8)
    assert (tail == 0x7B).all(), "recv_x written beyond num_recv"
    if "recv_scales" in res:
        assert (res["recv_scales"][n:].view(np.uint32) == poison32).all()
    return src


def check_payload(res, x, src, n, dtype):
    """Every receive row against the oracle.  bf16: the oracle's bit copy of the source row.  FP8:
    the oracle's dispatch quantises each receive row, and the quantisation is a function of the row
    alone, so at large sizes each source token is quantised once (in token chunks, to bound host
    memory) and every receive row is compared with its source token's codes and scales."""
    if dtype == "bf16":
        assert np.array_equal(res["recv_x"][:n], O.dispatch_rows_bf16(x, src))
        return
    got_q, got_s = res["recv_x"][:n], res["recv_scales"][:n]
    if n * x.shape[1] <= 50_000_000:
        exp_q, exp_s = O.dispatch_rows_fp8(x, src)
        bad = np.nonzero((got_q != exp_q).any(axis=1))[0]
        assert bad.size == 0, f"fp8 bytes differ in {bad.size} rows, first row {bad[:1]}"
        assert np.array_equal(got_s.view(np.uint32), exp_s.view(np.uint32))
        return
    T, step, seen = x.shape[0], 2048, 0
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        rows = np.nonzero((src >= t0) & (src < t1))[0]
        q_tok, s_tok = O.quantize_fp8_blocks(x[t0:t1])
        bad = np.nonzero((got_q[rows] != q_tok[src[rows] - t0]).any(axis=1))[0]
        assert bad.size == 0, f"fp8 bytes differ in {bad.size} rows, first row {rows[bad[0]]}"
        assert np.array_equal(got_s[rows].view(np.uint32), s_tok[src[rows] - t0].view(np.uint32))
        seen += rows.size
    assert seen == n


def check_combine(res, y, idx, w, E, R, send_row, num_y_rows=None, bound_sample=None):
    """All T outputs against the oracle's fp32 combine (gate: 1 bf16 ulp; returns whether they are
    bit-identical).  The fp64 sanity bound is checked on every token, or on `bound_sample` tokens."""
    dev = res["_dev"]
    out = H().run_combine(res["shape"], y, dev["idx"], dev["w"], dev["d"]["send_row"], num_y_rows=num_y_rows)
    ref = O.combine(y, idx, w, send_row, E, R)
    ok = within_one_bf16_ulp(out, ref)
    assert ok.all(), f"{(~ok).sum()} combine outputs beyond 1 bf16 ulp"
    exact = np.array_equal(out, ref)
    toks = np.arange(idx.shape[0]) if bound_sample is None else np.asarray(bound_sample)
    ref64, mag = O.combine_f64(y, idx, w, send_row, E, R, tokens=toks)
    check_combine_bound(out[toks], ref64, mag, idx.shape[1])
    return out, exact


def run_case(x, idx, w, E, R, dtype, y=None, identity=False, bound_sample=None, combine=True):
    res = H().run_layout_dispatch(x, idx, w, E, R, dtype)
    send_row, n = check_layout_and_slots(res, idx, E, R)
    src = check_metadata_and_guards(res, idx, w, E, R, send_row, n)
    check_payload(res, x, src, n, dtype)
    exact = None
    if identity:
        if dtype == "bf16":
            y = res["recv_x"][:n]
        else:
            y = O.dequantize_fp8_to_bf16(res["recv_x"][:n], res["recv_scales"][:n])
    if y is not None and combine:
        _, exact = check_combine(res, y, idx, w, E, R, send_row, bound_sample=bound_sample)
    return res, exact


# ------------------------------------------------------------------ the five workloads

def _workload(cfg):
    d = W.make_inputs(cfg)
    return d["x"], d["topk_idx"], d["topk_w"]


@pytest.mark.parametrize("cfg", W.CONFIGS, ids=lambda c: c.name)
def test_workload_dispatch_parity(cfg):
    """Full size: layout, slots, metadata and every receive row (bf16 bits, or FP8 codes and scales)."""
    _print_case("workload-dispatch", name=cfg.name, T=cfg.num_tokens, H=cfg.hidden, E=cfg.num_experts,
                k=cfg.num_topk, R=cfg.num_ranks, dtype=cfg.dispatch_dtype)
    x, idx, w = _workload(cfg)
    run_case(x, idx, w, cfg.num_experts, cfg.num_ranks, cfg.dispatch_dtype, combine=False)


@pytest.mark.parametrize("cfg", W.CONFIGS, ids=lambda c: c.name)
def test_workload_combine_parity(cfg):
    """Full size: all T combine outputs against the oracle (bit-identical expected, 1 bf16 ulp gate)."""
    _print_case("workload-combine", name=cfg.name, T=cfg.num_tokens, H=cfg.hidden, E=cfg.num_experts,
                k=cfg.num_topk, R=cfg.num_ranks, dtype=cfg.dispatch_dtype)
    x, idx, w = _workload(cfg)
    E, R, T = cfg.num_experts, cfg.num_ranks, cfg.num_tokens
    res = H().run_layout_dispatch(x, idx, w, E, R, cfg.dispatch_dtype)
    send_row, n = check_layout_and_slots(res, idx, E, R)
    if cfg.combine_input == "identity":
        y = res["recv_x"][:n] if cfg.dispatch_dtype == "bf16" else \
            O.dequantize_fp8_to_bf16(res["recv_x"][:n], res["recv_scales"][:n])
    else:
        y = W.draw_expert_outputs(W.y_stream(cfg), n, cfg.hidden)
    big = T * cfg.hidden > 8_000_000
    sample = np.sort(np.random.default_rng(cfg.index).choice(T, size=1024, replace=False)) if big else None
    _, exact = check_combine(res, y, idx, w, E, R, send_row, bound_sample=sample)
    assert exact, "combine not bit-identical to the fp32-sequenced oracle"


# ------------------------------------------------------------------ edge cases

EDGE = [
    # name, seed, T, H, E, k, R, dtype, invalid_frac
    ("single_token", 1, 1, 256, 16, 4, 4, "bf16", 0.0),
    ("ragged_multiblock", 2, 4097, 512, 64, 6, 16, "bf16", 0.1),
    ("fused_limit", 3, 1024, 256, 32, 4, 8, "fp8", 0.05),
    ("first_multiblock", 4, 1025, 256, 32, 4, 8, "fp8", 0.05),
    ("one_rank", 5, 300, 256, 8, 2, 1, "bf16", 0.0),
    ("top1", 6, 777, 384, 64, 1, 8, "fp8", 0.0),
    ("max_limits", 7, 300, 128, 4096, 32, 64, "fp8", 0.1),
    ("mostly_invalid", 8, 500, 256, 16, 4, 4, "bf16", 0.6),
    ("ragged_slice_fp8", 9, 200, 640, 32, 4, 8, "fp8", 0.0),
    ("ragged_slice_bf16", 10, 200, 136, 32, 4, 8, "bf16", 0.0),
    ("R_not_multiple_of_4", 11, 333, 256, 30, 5, 6, "bf16", 0.1),
    ("R_64_k_8", 12, 2000, 256, 256, 8, 64, "bf16", 0.0),
    ("wide_hidden_fp8", 13, 300, 16384, 64, 8, 8, "fp8", 0.0),     # 2048 16-byte pieces per row
    ("wide_hidden_bf16", 14, 300, 16384, 64, 8, 8, "bf16", 0.05),
    ("many_chunks", 15, 70000, 64, 64, 4, 8, "bf16", 0.05),      # 1094 chunks: multi-pass chunk scans
    ("one_expert_per_rank_k_eq_E", 16, 513, 256, 8, 8, 8, "bf16", 0.0),  # L = 1, every token to every rank
    ("min_hidden_bf16", 17, 1500, 8, 32, 4, 8, "bf16", 0.05),   # one 16-byte piece per row
    ("min_hidden_fp8", 18, 1500, 128, 32, 4, 8, "fp8", 0.05),   # one scale block per row
    # FP8 at hidden 7168 (14 groups of 64 16-byte pieces): the host takes the widest slice of
    # 14, 7, 4, 2 groups that still gives >= 4096 waves (T * slices), so each batch size below
    # runs a different dispatch width: 700 tokens -> 2 groups, 1500 -> 4, 3000 -> 7, 4100 -> 14.
    ("fp8_h7168_width2", 19, 700, 7168, 256, 8, 8, "fp8", 0.02),
    ("fp8_h7168_width4", 20, 1500, 7168, 256, 8, 8, "fp8", 0.02),
    ("fp8_h7168_width7", 21, 3000, 7168, 256, 8, 32, "fp8", 0.02),
    ("fp8_h7168_width14_ragged", 22, 4100, 7168, 128, 8, 16, "fp8", 0.05),
]


def _random_shapes(n: int, seed: int = 0xED6E):
    """Seeded shapes inside the library's limits: R | E, k <= E, H % 8 == 0 (H % 128 for FP8)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 32, 64]))
        L = int(rng.integers(1, max(2, 512 // R) + 1))
        E = R * L
        k = int(rng.integers(1, min(E, 32) + 1))
        dtype = "fp8" if rng.random() < 0.5 else "bf16"
        H = 128 * int(rng.integers(1, 13)) if dtype == "fp8" else 8 * int(rng.integers(1, 161))
        T = int(rng.integers(0, 2600))
        inv = float(rng.choice([0.0, 0.0, 0.1, 0.5]))
        out.append((f"rand{i}_T{T}_H{H}_E{E}_k{k}_R{R}_{dtype}", 100 + i, T, H, E, k, R, dtype, inv))
    return out


RANDOM_SHAPES = _random_shapes(16)


@pytest.mark.parametrize("case", EDGE + RANDOM_SHAPES, ids=lambda c: c[0])
def test_edge_parity(case):
    name, seed, T, Hd, E, k, R, dtype, inv = case
    _print_case("edge", name=name, T=T, H=Hd, E=E, k=k, R=R, dtype=dtype)
    d = W.random_case(seed, T, Hd, E, k, R, invalid_frac=inv)
    _, _, mask = O.get_dispatch_layout(d["topk_idx"], E, R)
    y = W.draw_expert_outputs(np.random.default_rng(seed), max(int(mask.sum()), 1), Hd)
    _, exact = run_case(d["x"], d["topk_idx"], d["topk_w"], E, R, dtype, y=y)
    assert exact


def test_empty_batch():
    _print_case("edge", name="empty")
    x = np.zeros((0, 256), np.uint16)
    idx = np.zeros((0, 4), np.int32)
    w = np.zeros((0, 4), np.float32)
    res = H().run_layout_dispatch(x, idx, w, 16, 4, "bf16")
    assert (res["tokens_per_rank"] == 0).all() and (res["tokens_per_expert"] == 0).all()
    assert (res["rank_offsets"] == 0).all() and int(res["num_recv"][0]) == 0
    assert (res["recv_x"].view(np.uint8) == 0x7B).all()
    out = H().run_combine(res["shape"], np.zeros((0, 256), np.uint16), res["_dev"]["idx"], res["_dev"]["w"],
                          res["_dev"]["d"]["send_row"])
    assert out.shape == (0, 256)


def test_all_tokens_to_one_rank():
    _print_case("edge", name="hot_rank")
    rng = np.random.default_rng(21)
    T, Hd, E, k, R = 3000, 256, 64, 4, 8
    L = E // R
    idx = np.stack([rng.permutation(L)[:k] + 3 * L for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    x = W.draw_hidden(rng, T, Hd)
    y = W.draw_expert_outputs(rng, T, Hd)
    res, exact = run_case(x, idx, w, E, R, "fp8", y=y)
    assert res["tokens_per_rank"].tolist() == [0, 0, 0, T, 0, 0, 0, 0]
    assert exact


def test_duplicate_ids_in_a_row():
    _print_case("edge", name="duplicates")
    rng = np.random.default_rng(22)
    T, Hd, E, k, R = 200, 256, 16, 4, 4
    idx = rng.integers(0, 6, size=(T, k)).astype(np.int32)  # many repeats
    w = rng.random((T, k)).astype(np.float32)
    x = W.draw_hidden(rng, T, Hd)
    _, _, mask = O.get_dispatch_layout(idx, E, R)
    y = W.draw_expert_outputs(rng, int(mask.sum()), Hd)
    _, exact = run_case(x, idx, w, E, R, "bf16", y=y)
    assert exact


def test_fp8_special_rows():
    _print_case("edge", name="fp8_special_rows")
    rng = np.random.default_rng(23)
    Hd = 512
    rows = [np.zeros(Hd, np.float32), np.full(Hd, -0.0, np.float32),
            (rng.standard_normal(Hd) * 1e-6).astype(np.float32),           # amax below the 1e-4 floor
            np.where(rng.random(Hd) < 0.5, 2.0 ** -130, -3 * 2.0 ** -133).astype(np.float32),  # bf16 subnormals
            (rng.standard_normal(Hd) * 3e4).astype(np.float32),
            (rng.standard_normal(Hd) * 1e-30).astype(np.float32)]
    # E4M3 ties: a block with amax 448 * 2^-3 so that x / s = 8 x exactly hits midpoints
    tie = np.zeros(Hd, np.float32)
    tie[0] = 56.0
    mids = ((E4M3_MAGNITUDES[1:] + E4M3_MAGNITUDES[:-1]) / 2) / 8
    tie[1:128] = rng.choice(mids[mids <= 56], 127) * rng.choice([-1, 1], 127)
    rows.append(tie)
    x = f32_to_bf16_bits_rne(np.stack(rows))
    T = x.shape[0]
    idx = np.tile(np.array([[0, 5]], np.int32), (T, 1))
    w = np.full((T, 2), 0.5, np.float32)
    res, _ = run_case(x, idx, w, 8, 2, "fp8")
    n = int(res["num_recv"][0])
    check_fp8_block_properties(x[res["recv_src_idx"][:n]], res["recv_x"][:n], res["recv_scales"][:n])


def test_fp8_sweep_all_bf16_patterns():
    """Every finite bf16 value, quantised against power-of-two scales (exact ties) and random scales."""
    _print_case("edge", name="fp8_sweep")
    rng = np.random.default_rng(24)
    allb = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    fin = allb[np.isfinite(bf16_bits_to_f32(allb))]
    Hd = 7168
    blocks = []
    amaxes = [448.0 * 2.0 ** e for e in range(-20, 8)] + list(np.exp2(rng.uniform(-15, 10, 40)))
    for a in amaxes:
        a_bits = f32_to_bf16_bits_rne(np.float32([a]))[0]
        af = bf16_bits_to_f32(np.uint16([a_bits]))[0]
        vals = fin[np.abs(bf16_bits_to_f32(fin)) <= af]
        vals = rng.permutation(vals)
        for b0 in range(0, vals.size, 127):
            blk = np.zeros(128, np.uint16)
            chunk = vals[b0:b0 + 127]
            blk[0] = a_bits
            blk[1:1 + chunk.size] = chunk
            blocks.append(blk)
    nb = len(blocks)
    per_row = Hd // 128
    pad = (-nb) % per_row
    blocks += [np.zeros(128, np.uint16)] * pad
    x = np.stack(blocks).reshape(-1, Hd)
    T = x.shape[0]
    idx = np.tile(np.array([[0]], np.int32), (T, 1))
    w = np.ones((T, 1), np.float32)
    print(f"[case] fp8 sweep rows={T} blocks={nb}", flush=True)
    run_case(x, idx, w, 8, 8, "fp8")


# ------------------------------------------------------------------ combine-specific

def test_combine_skips_rows_beyond_num_y_rows():
    _print_case("edge", name="num_y_rows")
    d = W.random_case(31, 300, 256, 32, 4, 8)
    x, idx, w = d["x"], d["topk_idx"], d["topk_w"]
    res = H().run_layout_dispatch(x, idx, w, 32, 8, "bf16")
    send_row, n = check_layout_and_slots(res, idx, 32, 8)
    y = W.draw_expert_outputs(np.random.default_rng(1), n, 256)
    limit = n // 2
    dev = res["_dev"]
    out = H().run_combine(res["shape"], y[:limit], dev["idx"], dev["w"], dev["d"]["send_row"], num_y_rows=limit)
    L = 32 // 8
    rows = np.take_along_axis(send_row, np.where(idx >= 0, idx // L, 0), axis=1)
    idx_cut = np.where(rows < limit, idx, -1).astype(np.int32)
    ref = O.combine(y[:limit], idx_cut, w, send_row, 32, 8)
    assert np.array_equal(out, ref)


def test_bf16_round_trip_identity_expert():
    """Dispatch then identity-expert combine returns sum_j w_j x = x for normalised weights."""
    cfg = W.CONFIG_BY_NAME["prefill"]
    c = W.with_tokens(cfg, 512)
    _print_case("roundtrip", T=c.num_tokens)
    d = W.make_inputs(c)
    x, idx, w = d["x"], d["topk_idx"], d["topk_w"]
    res, exact = run_case(x, idx, w, c.num_experts, c.num_ranks, "bf16", identity=True)
    assert exact
    n = int(res["num_recv"][0])
    dev = res["_dev"]
    out = H().run_combine(res["shape"], res["recv_x"][:n], dev["idx"], dev["w"], dev["d"]["send_row"])
    xf = bf16_bits_to_f32(x).astype(np.float64) * w.astype(np.float64).sum(axis=1, keepdims=True)
    check_combine_bound(out, xf, np.abs(xf), c.num_topk)
    assert within_one_bf16_ulp(out, x).all()


def test_run_to_run_identical():
    cfg = W.CONFIG_BY_NAME["group_limited"]
    c = W.with_tokens(cfg, 1500)
    _print_case("determinism", T=c.num_tokens)
    d = W.make_inputs(c)
    a = H().run_layout_dispatch(d["x"], d["topk_idx"], d["topk_w"], c.num_experts, c.num_ranks, "fp8")
    b = H().run_layout_dispatch(d["x"], d["topk_idx"], d["topk_w"], c.num_experts, c.num_ranks, "fp8")
    for key in ("tokens_per_rank", "tokens_per_expert", "is_token_in_rank", "send_row", "recv_x", "recv_scales",
                "recv_src_idx", "recv_topk_idx", "recv_topk_w"):
        assert np.array_equal(a[key], b[key]), key
    # and both runs against the oracle (1500 tokens at hidden 7168 runs the 4-group FP8 width)
    send_row, n = check_layout_and_slots(a, d["topk_idx"], c.num_experts, c.num_ranks)
    src = check_metadata_and_guards(a, d["topk_idx"], d["topk_w"], c.num_experts, c.num_ranks, send_row, n)
    check_payload(a, d["x"], src, n, "fp8")
    y = W.draw_expert_outputs(np.random.default_rng(3), n, c.hidden)
    o1 = H().run_combine(a["shape"], y, a["_dev"]["idx"], a["_dev"]["w"], a["_dev"]["d"]["send_row"])
    o2 = H().run_combine(a["shape"], y, a["_dev"]["idx"], a["_dev"]["w"], a["_dev"]["d"]["send_row"])
    assert np.array_equal(o1, o2)
    assert np.array_equal(o1, O.combine(y, d["topk_idx"], d["topk_w"], send_row, c.num_experts, c.num_ranks))


def test_layout_invariants_at_full_size():
    cfg = W.CONFIG_BY_NAME["skewed"]
    _print_case("invariants", name=cfg.name)
    g = W.seed_streams(cfg.index)
    idx, w = W.route(cfg, g[1], g[3])
    x = np.zeros((cfg.num_tokens, 128), np.uint16)
    res = H().run_layout_dispatch(x, idx, w, cfg.num_experts, cfg.num_ranks, "bf16")
    check_layout_invariants(idx, cfg.num_experts, cfg.num_ranks, res["tokens_per_rank"], res["tokens_per_expert"],
                            res["is_token_in_rank"])
    check_slot_invariants(res["is_token_in_rank"], res["rank_offsets"], res["send_row"], int(res["num_recv"][0]))


def test_combine_golden_fp32_order():
    """The hand-worked fixture in which the fp32 summation order and the absence of fused
    multiply-add show in the bf16 output (tests/golden/hand_combine_fp32_order.json), on the GPU."""
    import json
    import os
    import combine_get_dispatch_07_amd as moe
    _print_case("edge", name="golden_fp32_order")
    g = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                    "hand_combine_fp32_order.json")))
    E, R = g["num_experts"], g["num_ranks"]
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_w"], np.float32)
    _, _, mask = O.get_dispatch_layout(idx, E, R)
    _, send_row, n = O.assign_slots(mask)
    Hd = 8
    y = f32_to_bf16_bits_rne(np.array(g["y_rows"], np.float32)[:, None] * np.ones((1, Hd), np.float32))
    assert y.shape[0] == n
    shape = moe.MoeShape(idx.shape[0], Hd, idx.shape[1], E, R)
    out = H().run_combine(shape, y, torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda(),
                          torch.from_numpy(send_row).cuda())
    expect = f32_to_bf16_bits_rne(np.array(g["expect_out"], np.float32)[:, None] * np.ones((1, Hd), np.float32))
    assert np.array_equal(out, expect)


@pytest.mark.parametrize("fixture", ["hand_layout_dispatch_combine.json", "hand_duplicate_ids.json"])
def test_golden_hand_cases(fixture):
    """The hand-worked layout / dispatch / combine fixtures through the GPU path, compared with the
    values derived by hand in the fixture (the fixture's 2-channel rows repeated to 8 channels)."""
    import json
    import os
    _print_case("golden", name=fixture)
    g = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", fixture)))
    E, R, ex = g["num_experts"], g["num_ranks"], g["expect"]
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_w"], np.float32)
    T, Hd = idx.shape[0], 8
    x = f32_to_bf16_bits_rne(np.arange(T * Hd, dtype=np.float32).reshape(T, Hd))
    res = H().run_layout_dispatch(x, idx, w, E, R, "bf16")
    n = ex["num_recv"]
    assert res["tokens_per_expert"].tolist() == ex["tokens_per_expert"]
    assert res["is_token_in_rank"].tolist() == ex["is_token_in_rank"]
    assert res["tokens_per_rank"].tolist() == ex["tokens_per_rank"]
    assert res["rank_offsets"].tolist() == ex["rank_offsets"] and int(res["num_recv"][0]) == n
    assert res["send_row"].tolist() == ex["send_row"]
    assert res["recv_src_idx"][:n].tolist() == ex["recv_src_idx"]
    assert res["recv_topk_idx"][:n].tolist() == ex["recv_topk_idx"]
    assert res["recv_topk_w"][:n].tolist() == ex["recv_topk_w"]
    assert np.array_equal(res["recv_x"][:n], x[ex["recv_src_idx"]])
    y = f32_to_bf16_bits_rne(np.tile(np.array([[i + 1, -(i + 1) / 2] for i in range(n)], np.float32), (1, Hd // 2)))
    dev = res["_dev"]
    out = H().run_combine(res["shape"], y, dev["idx"], dev["w"], dev["d"]["send_row"])
    expect = f32_to_bf16_bits_rne(np.tile(np.array(ex["combine_out"], np.float32), (1, Hd // 2)))
    assert np.array_equal(out, expect)


def test_golden_fp8_blocks():
    """tests/golden/hand_fp8_blocks.json (codes and scales worked out by hand, ties included) through
    an FP8 dispatch of one token per block on the GPU."""
    import json
    import os
    _print_case("golden", name="hand_fp8_blocks")
    g = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_fp8_blocks.json")))
    for blk in g["blocks"]:
        vals = np.zeros(128, np.float32)
        vals[:len(blk["values"])] = blk["values"]
        codes = np.zeros(128, np.uint8)
        codes[:len(blk["codes"])] = blk["codes"]
        x = f32_to_bf16_bits_rne(vals)[None, :]
        assert np.array_equal(bf16_bits_to_f32(x)[0], vals), blk["name"]  # the values are exact in bf16
        res = H().run_layout_dispatch(x, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32), 1, 1, "fp8")
        assert int(res["num_recv"][0]) == 1
        assert res["recv_x"][0].tolist() == codes.tolist(), blk["name"]
        assert res["recv_scales"][0].tolist() == [blk["scale"]], blk["name"]
