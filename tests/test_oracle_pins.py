"""Pins of the CPU oracle to things other than itself (no GPU).

* hand-worked golden cases (tests/golden/, each derivation written out);
* library routines: torch's fp32->bf16 and fp32->float8_e4m3fn conversions;
* closed forms: E4M3 code values, all-codes round trip, midpoint ties;
* an independent brute-force loop oracle on tiny random inputs;
* invariants on all five workloads;
* error bounds against an fp64 sum.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import bruteforce as bf
from oracle import moe_oracle as O
from oracle.numerics import (E4M3_MAGNITUDES, bf16_bits_to_f32, e4m3_decode, e4m3_encode_rne,
                             f32_to_bf16_bits_rne)
from tests.checks import (check_combine_bound, check_fp8_block_properties, check_layout_invariants,
                          check_metadata, check_slot_invariants)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_exact(values):
    f = np.asarray(values, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_bits_to_f32(bits).view(np.uint32), f.view(np.uint32)), "fixture value not exact in bf16"
    return bits


# ---------------------------------------------------------------- golden, hand-worked

@pytest.mark.parametrize("fixture", ["hand_layout_dispatch_combine.json", "hand_duplicate_ids.json"])
def test_golden_layout_dispatch_combine(fixture):
    g = json.load(open(os.path.join(GOLDEN, fixture)))
    E, R = g["num_experts"], g["num_ranks"]
    idx = np.array(g["topk_idx"], dtype=np.int32)
    w = np.array(g["topk_w"], dtype=np.float32)
    ex = g["expect"]
    tpr, tpe, mask = O.get_dispatch_layout(idx, E, R)
    assert tpe.tolist() == ex["tokens_per_expert"]
    assert mask.tolist() == ex["is_token_in_rank"]
    assert tpr.tolist() == ex["tokens_per_rank"]
    offs, send_row, n = O.assign_slots(mask)
    assert offs.tolist() == ex["rank_offsets"] and n == ex["num_recv"]
    assert send_row.tolist() == ex["send_row"]
    src, ridx, rw = O.dispatch_metadata(idx, w, E, R, send_row, n)
    assert src.tolist() == ex["recv_src_idx"]
    assert ridx.tolist() == ex["recv_topk_idx"]
    assert rw.tolist() == ex["recv_topk_w"]
    y = np.array([[i + 1, -(i + 1) / 2] for i in range(n)], dtype=np.float32)
    out = O.combine(_bf16_exact(y), idx, w, send_row, E, R)
    assert bf16_bits_to_f32(out).tolist() == ex["combine_out"]
    # the loop oracle agrees on the same hand case
    b = bf.dispatch(np.zeros((idx.shape[0], 2), np.uint16), idx.tolist(), w.tolist(), E, R, "bf16")
    assert b["send_row"] == ex["send_row"] and b["recv_topk_idx"] == ex["recv_topk_idx"]


def test_golden_combine_fp32_order():
    g = json.load(open(os.path.join(GOLDEN, "hand_combine_fp32_order.json")))
    E, R = g["num_experts"], g["num_ranks"]
    idx = np.array(g["topk_idx"], dtype=np.int32)
    w = np.array(g["topk_w"], dtype=np.float64)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w), "weights must be exact in fp32"
    w = w.astype(np.float32)
    tpr, tpe, mask = O.get_dispatch_layout(idx, E, R)
    offs, send_row, n = O.assign_slots(mask)
    y = _bf16_exact(np.array(g["y_rows"], dtype=np.float32)[:, None] * np.ones((1, 8), np.float32))
    assert n == y.shape[0]
    out = O.combine(y, idx, w, send_row, E, R)
    expect = np.array(g["expect_out"], dtype=np.float32)[:, None] * np.ones((1, 8), np.float32)
    assert np.array_equal(bf16_bits_to_f32(out).view(np.uint32), expect.view(np.uint32))
    assert bf.combine(y, idx.tolist(), w.tolist(), send_row.tolist(), E, R) == out.tolist()


def test_golden_fp8_blocks():
    g = json.load(open(os.path.join(GOLDEN, "hand_fp8_blocks.json")))
    for blk in g["blocks"]:
        vals = np.zeros(128, dtype=np.float32)
        vals[:len(blk["values"])] = blk["values"]
        codes = np.zeros(128, dtype=np.uint8)
        codes[:len(blk["codes"])] = blk["codes"]
        # -0.0 entries keep their sign bit
        x = _bf16_exact(vals)[None, :]
        q, s = O.quantize_fp8_blocks(x)
        assert s.tolist() == [[blk["scale"]]], blk["name"]
        assert q[0].tolist() == codes.tolist(), blk["name"]
        # the loop oracle too
        b = bf.dispatch(x, [[0]], [[1.0]], 1, 1, "fp8")
        assert b["recv_x"][0] == codes.tolist() and b["recv_scales"][0] == [blk["scale"]]


# ---------------------------------------------------------------- number formats vs library routines

def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    # exact ties, near-ties and subnormals
    ties = (rng.integers(0, 2 ** 16, size=50_000, dtype=np.uint32) << 16) | 0x8000
    near = ties + rng.integers(-2, 3, size=ties.size).astype(np.int64).astype(np.uint32)
    sub = rng.integers(0, 2 ** 23, size=50_000, dtype=np.uint32) | (rng.integers(0, 2, 50_000, dtype=np.uint32) << 31)
    u = np.concatenate([u, ties, near, sub])
    f = u.view(np.float32)
    with np.errstate(invalid="ignore"):
        f = f[np.isfinite(f) & (np.abs(f.astype(np.float64)) < 3.3e38)]
    ours = f32_to_bf16_bits_rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_table_closed_form():
    # code 0x08 is the first normal (2^-6), 0x01 the smallest subnormal, 0x7E the largest value
    assert E4M3_MAGNITUDES[0x01] == 2.0 ** -9
    assert E4M3_MAGNITUDES[0x07] == 7 * 2.0 ** -9
    assert E4M3_MAGNITUDES[0x08] == 2.0 ** -6
    assert E4M3_MAGNITUDES[0x38] == 1.0
    assert E4M3_MAGNITUDES[0x7E] == 448.0
    assert np.all(np.diff(E4M3_MAGNITUDES) > 0)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    dec = e4m3_decode(codes)
    # every finite code round-trips exactly (254 codes, +0 and -0 included)
    assert np.array_equal(e4m3_encode_rne(dec), codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(dec.view(np.uint32), ref.view(np.uint32))


def test_e4m3_encoder_matches_torch():
    rng = np.random.default_rng(2)
    # every finite bf16 pattern below 464 (the first magnitude that would round past 448)
    allb = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    fb = bf16_bits_to_f32(allb)
    fb = fb[np.isfinite(fb) & (np.abs(fb) < 464.0)]
    # random fp32 spread over the E4M3 range, all midpoints between neighbouring codes and their neighbours
    rnd = (rng.standard_normal(300_000) * np.exp2(rng.uniform(-12, 8, 300_000))).astype(np.float32)
    mids = ((E4M3_MAGNITUDES[1:] + E4M3_MAGNITUDES[:-1]) / 2).astype(np.float32)
    mid_nb = np.concatenate([np.nextafter(mids, np.float32(0)), mids, np.nextafter(mids, np.float32(1e9))])
    allv = np.concatenate([fb, rnd, mid_nb, -mid_nb, np.float32([0.0, -0.0, 448.0, -448.0, 463.99])])
    allv = allv[np.abs(allv) < 464.0]
    ours = e4m3_encode_rne(allv)
    ref = torch.from_numpy(allv.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_bruteforce_encoders_agree():
    rng = np.random.default_rng(3)
    vals = np.concatenate([(rng.standard_normal(4000) * np.exp2(rng.uniform(-12, 8, 4000))).astype(np.float32),
                           ((E4M3_MAGNITUDES[1:] + E4M3_MAGNITUDES[:-1]) / 2).astype(np.float32)])
    vals = vals[np.abs(vals) < 464]
    assert [bf.e4m3_round(float(v)) for v in vals] == e4m3_encode_rne(vals).tolist()
    f = (rng.standard_normal(4000) * np.exp2(rng.uniform(-140, 20, 4000))).astype(np.float32)
    assert [bf.bf16_round(float(v)) for v in f] == f32_to_bf16_bits_rne(f).tolist()


# ---------------------------------------------------------------- brute force on tiny random inputs

TINY_CASES = [
    # (seed, T, H, E, k, R, invalid_frac)
    (0, 1, 128, 8, 1, 1, 0.0),
    (1, 7, 128, 16, 4, 4, 0.1),
    (2, 33, 256, 16, 4, 2, 0.1),
    (3, 64, 128, 32, 8, 8, 0.1),
    (4, 70, 128, 64, 8, 16, 0.1),
    (5, 5, 128, 12, 3, 3, 0.3),
    (6, 0, 128, 16, 4, 4, 0.0),
    (7, 19, 128, 8, 8, 8, 0.0),
    (8, 40, 128, 16, 2, 16, 0.5),
]


@pytest.mark.parametrize("case", TINY_CASES, ids=lambda c: f"s{c[0]}_T{c[1]}_E{c[3]}_k{c[4]}_R{c[5]}")
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_oracle_vs_bruteforce(case, dtype):
    seed, T, H, E, k, R, inv = case
    d = W.random_case(seed, T, H, E, k, R, invalid_frac=inv)
    x, idx, w = d["x"], d["topk_idx"], d["topk_w"]
    ref = O.run_all(x, idx, w, E, R, dtype)
    b = bf.dispatch(x, idx.tolist(), w.tolist(), E, R, dtype)
    assert ref["tokens_per_rank"].tolist() == b["tokens_per_rank"]
    assert ref["tokens_per_expert"].tolist() == b["tokens_per_expert"]
    assert ref["is_token_in_rank"].tolist() == [list(r) for r in b["is_token_in_rank"]]
    assert ref["rank_offsets"].tolist() == b["rank_offsets"]
    assert ref["send_row"].tolist() == b["send_row"]
    assert ref["recv_src_idx"].tolist() == b["recv_src_idx"]
    assert ref["recv_topk_idx"].tolist() == b["recv_topk_idx"]
    assert ref["recv_topk_w"].tolist() == b["recv_topk_w"]
    n = int(ref["num_recv"])
    if n:
        assert ref["recv_x"].tolist() == b["recv_x"]
        if dtype == "fp8":
            assert ref["recv_scales"].tolist() == b["recv_scales"]
    # combine on random expert outputs
    y = W.draw_expert_outputs(np.random.default_rng(seed + 100), max(n, 1), 16)
    out = O.combine(y, idx, w, ref["send_row"], E, R)
    bout = bf.combine(y, idx.tolist(), w.tolist(), ref["send_row"].tolist(), E, R)
    assert out.tolist() == bout


# ---------------------------------------------------------------- invariants on the five workloads

@pytest.mark.parametrize("cfg", W.CONFIGS, ids=lambda c: c.name)
def test_workload_invariants(cfg):
    g_x, g_router, _g_y, g_extra = W.seed_streams(cfg.index)
    idx, w = W.route(cfg, g_router, g_extra)
    E, R, T = cfg.num_experts, cfg.num_ranks, cfg.num_tokens
    tpr, tpe, mask = O.get_dispatch_layout(idx, E, R)
    check_layout_invariants(idx, E, R, tpr, tpe, mask)
    assert int(tpe.sum()) == T * cfg.num_topk  # no masked ids in the workloads: counts sum to tokens x topk
    offs, send_row, n = O.assign_slots(mask)
    check_slot_invariants(mask, offs, send_row, n)
    sub = slice(0, min(T, 512))
    src, ridx, rw = O.dispatch_metadata(idx, w, E, R, send_row, n)
    check_metadata(idx[sub], w[sub], E, R, send_row[sub], src, ridx, rw)
    # dispatch payload on a few hundred tokens' rows
    x = W.draw_hidden(g_x, min(T, 256), cfg.hidden)
    rows = np.nonzero(src < x.shape[0])[0]
    if cfg.dispatch_dtype == "bf16":
        assert np.array_equal(O.dispatch_rows_bf16(x, src[rows]), x[src[rows]])
    else:
        q, s = O.dispatch_rows_fp8(x, src[rows])
        check_fp8_block_properties(x[src[rows]], q, s)


# ---------------------------------------------------------------- FP8 properties, edge rows

def test_fp8_edge_rows():
    rng = np.random.default_rng(4)
    H = 512
    rows = []
    rows.append(np.zeros(H, np.float32))  # all zero: s = 1e-4/448, every code +0
    neg0 = np.zeros(H, np.float32)
    neg0[::2] = -0.0
    rows.append(neg0)
    tiny = (rng.standard_normal(H) * 1e-6).astype(np.float32)  # amax below the 1e-4 floor
    rows.append(tiny)
    sub = np.zeros(H, np.float32)
    sub[:64] = np.float32(2.0 ** -130)  # bf16 subnormals
    sub[64:70] = -np.float32(3 * 2.0 ** -133)
    rows.append(sub)
    big = (rng.standard_normal(H) * 3e4).astype(np.float32)
    rows.append(big)
    one_hot = np.zeros(H, np.float32)
    one_hot[5] = 7.0
    one_hot[200] = -0.001
    rows.append(one_hot)
    x = f32_to_bf16_bits_rne(np.stack(rows))
    q, s = O.quantize_fp8_blocks(x)
    check_fp8_block_properties(x, q, s)
    assert (q[0] == 0).all() and (q[1][::2] == 0x80).all() and (q[1][1::2] == 0).all()
    floor_s = np.float32(np.float32(1e-4) / np.float32(448.0))
    assert (s[0] == floor_s).all() and (s[2] == floor_s).all()
    assert q[5][5] == 0x7E


# ---------------------------------------------------------------- combine: fp64 bound and round trips

@pytest.mark.parametrize("cfg", [W.CONFIG_BY_NAME["tiny"], W.CONFIG_BY_NAME["decode"]], ids=lambda c: c.name)
def test_combine_error_bound(cfg):
    g_x, g_router, g_y, g_extra = W.seed_streams(cfg.index)
    idx, w = W.route(cfg, g_router, g_extra)
    tpr, tpe, mask = O.get_dispatch_layout(idx, cfg.num_experts, cfg.num_ranks)
    offs, send_row, n = O.assign_slots(mask)
    y = W.draw_expert_outputs(g_y, n, 512)
    toks = np.arange(min(cfg.num_tokens, 64))
    out = O.combine(y, idx, w, send_row, cfg.num_experts, cfg.num_ranks, tokens=toks)
    ref, mag = O.combine_f64(y, idx, w, send_row, cfg.num_experts, cfg.num_ranks, tokens=toks)
    check_combine_bound(out, ref, mag, cfg.num_topk)


def test_identity_round_trip_k1_is_exact():
    # one expert per token with weight 1: dispatch then identity combine returns x exactly (-0 -> +0)
    d = W.random_case(11, 50, 256, 16, 1, 4)
    x, idx = d["x"], d["topk_idx"]
    w = np.ones_like(d["topk_w"])
    ref = O.run_all(x, idx, w, 16, 4, "bf16")
    out = O.combine(ref["recv_x"], idx, w, ref["send_row"], 16, 4)
    expect = np.where(x == 0x8000, np.uint16(0), x)
    assert np.array_equal(out, expect)


@pytest.mark.parametrize("cfg", [W.CONFIG_BY_NAME["tiny"]], ids=lambda c: c.name)
def test_identity_round_trip_weighted(cfg):
    # dispatch then identity combine returns sum_j w_j * x = x (normalised weights) up to fp32 rounding
    d = W.make_inputs(cfg)
    x, idx, w = d["x"], d["topk_idx"], d["topk_w"]
    ref = O.run_all(x, idx, w, cfg.num_experts, cfg.num_ranks, "bf16")
    out = O.combine(ref["recv_x"], idx, w, ref["send_row"], cfg.num_experts, cfg.num_ranks)
    xs = bf16_bits_to_f32(x).astype(np.float64) * w.astype(np.float64).sum(axis=1, keepdims=True)
    check_combine_bound(out, xs, np.abs(xs), cfg.num_topk)
    # normal values come back exactly
    normal = np.abs(bf16_bits_to_f32(x)) >= 2.0 ** -120
    assert np.array_equal(out[normal], x[normal])


def test_fp8_identity_round_trip():
    cfg = W.CONFIG_BY_NAME["decode"]
    d = W.make_inputs(W.with_tokens(cfg, 16))
    x, idx, w = d["x"], d["topk_idx"], d["topk_w"]
    ref = O.run_all(x, idx, w, cfg.num_experts, cfg.num_ranks, "fp8")
    y = O.dequantize_fp8_to_bf16(ref["recv_x"], ref["recv_scales"])
    out = O.combine(y, idx, w, ref["send_row"], cfg.num_experts, cfg.num_ranks)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    got = bf16_bits_to_f32(out).astype(np.float64)
    # per-element E4M3 error (2^-4 relative + subnormal floor) survives the convex combination
    blk_amax = np.abs(xf).reshape(16, -1, 128).max(axis=2).repeat(128, axis=1)
    assert (np.abs(got - xf) <= 2.0 ** -4 * np.abs(xf) + 2.0 ** -10 * blk_amax / 448 * 2 + 2.0 ** -7 * np.abs(xf)).all()


def test_golden_dequant_bf16():
    """tests/golden/hand_dequant_bf16.json: the identity expert on FP8 rows, BF16_RNE(fl32(decode(q) * s)),
    on products that land on or next to bf16 midpoints (ties to even up and down, a negative tie, a
    subnormal code), worked out by hand."""
    g = json.load(open(os.path.join(GOLDEN, "hand_dequant_bf16.json")))
    cases = g["cases"]
    q = np.zeros((len(cases), 128), np.uint8)
    s = np.zeros((len(cases), 1), np.float32)
    for i, c in enumerate(cases):
        q[i, 0] = c["code"]
        s[i, 0] = c["scale"]
        assert float(np.float32(c["scale"])) == c["scale"], c["name"]  # the scales are exact in fp32
    y = O.dequantize_fp8_to_bf16(q, s)
    assert y[:, 0].tolist() == [c["bf16"] for c in cases]
    assert (y[:, 1:] == 0).all()  # code 0x00 -> +0


def test_combine_f64_closed_form():
    """combine_f64 returns the exact weighted sum and the sum of magnitudes.  Closed forms:
    token 0: w = (1, 1, 1) on rows (2^24, 1, -2^24) -> exact sum 1 (an fp32 running sum gives 0:
    2^24 + 1 rounds to 2^24), magnitude 2^25 + 1; token 1: w = (0.5, 0.25) on rows (3, -5) and an
    invalid third slot -> 0.5*3 - 0.25*5 = 0.25, magnitude 1.5 + 1.25 = 2.75."""
    E, R = 4, 4  # one expert per rank: expert e's row is the token's row on rank e
    idx = np.array([[0, 1, 2], [1, 3, -1]], np.int32)
    w = np.array([[1.0, 1.0, 1.0], [0.5, 0.25, 0.75]], np.float32)
    _, _, mask = O.get_dispatch_layout(idx, E, R)
    _, send_row, n = O.assign_slots(mask)
    # ranks: token 0 -> 0, 1, 2; token 1 -> 1, 3; segment sizes 1, 2, 1, 1
    assert n == 5 and send_row.tolist() == [[0, 1, 3, -1], [-1, 2, -1, 4]]
    rows = np.zeros((n, 2), np.float32)
    rows[send_row[0, 0]] = 2.0 ** 24
    rows[send_row[0, 1]] = 1.0
    rows[send_row[0, 2]] = -(2.0 ** 24)
    rows[send_row[1, 1]] = 3.0
    rows[send_row[1, 3]] = -5.0
    y = _bf16_exact(rows)
    acc, mag = O.combine_f64(y, idx, w, send_row, E, R)
    assert acc.dtype == np.float64 and mag.dtype == np.float64
    assert acc[:, 0].tolist() == [1.0, 0.25] and acc[:, 1].tolist() == [1.0, 0.25]
    assert mag[:, 0].tolist() == [2.0 ** 25 + 1, 2.75]
    assert O.combine_f64(y, idx, w, send_row, E, R, tokens=np.array([1]))[0][:, 0].tolist() == [0.25]
    # the fp32-sequenced oracle differs here by exactly the lost 1
    assert bf16_bits_to_f32(O.combine(y, idx, w, send_row, E, R))[:, 0].tolist() == [0.0, 0.25]
