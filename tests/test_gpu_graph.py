"""The path captured in a HIP graph: layout (or the fused router) -> dispatch -> combine recorded
once and replayed several times, with eager work and a poisoning of every output between the
replays; each replay must reproduce the eager results bit for bit.  The library's kernels take
all their sizes as arguments and clear nothing with memset, so a captured call is a faithful
replay of the eager one."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

POISON = 0x5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _buffers(moe, shape, dtype, routed):
    lay = moe.alloc_route(shape) if routed else moe.alloc_layout(shape)
    d = moe.alloc_dispatch(shape, dtype)
    out = torch.empty((shape.num_tokens, shape.hidden), dtype=torch.bfloat16, device="cuda")
    return lay, d, out


def _step(moe, shape, dtype, x, idx, w, logits, y, lay, d, out, gate):
    if logits is not None:
        moe.run_route(shape, logits, lay, gate)
        idx, w = lay["topk_idx"], lay["topk_w"]
    else:
        moe.run_layout(shape, idx, lay)
    moe.run_dispatch(shape, dtype, x, idx, w, lay, d)
    moe.moe_combine(shape, y, idx, w, d["send_row"], out)


def _results(lay, d, out):
    r = {k: v.clone() for k, v in d.items() if v is not None}
    r["out"] = out.clone()
    for k in ("tokens_per_rank", "tokens_per_expert", "is_token_in_rank", "topk_idx", "topk_w"):
        if k in lay:
            r[k] = lay[k].clone()
    return r


@pytest.mark.parametrize("name,T,routed", [("decode", 128, False), ("prefill", 2048, False), ("decode", 128, True),
                                           ("prefill", 2048, True), ("group_limited", 2048, False),
                                           ("skewed", 3000, False)])
def test_graph_replays_match_eager(name, T, routed):
    import combine_get_dispatch_07_amd as moe
    from tests.gpu_harness import to_dev_bf16

    cfg = W.with_tokens(W.CONFIG_BY_NAME[name], T)
    print(f"[case] graph {name} T={T} routed={routed}", flush=True)
    gate = "sigmoid" if cfg.routing == "sigmoid" else "softmax"
    dtype = cfg.dispatch_dtype
    shape = moe.MoeShape(cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks)
    inp = W.make_inputs(cfg)
    x = to_dev_bf16(inp["x"])
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    logits = torch.from_numpy(W.config_logits(cfg)).cuda() if routed else None
    y = to_dev_bf16(W.draw_expert_outputs(np.random.default_rng(3), shape.num_tokens * min(shape.num_topk,
                                                                                              shape.num_ranks),
                                          shape.hidden))

    lay, d, out = _buffers(moe, shape, dtype, routed)
    _step(moe, shape, dtype, x, idx, w, logits, y, lay, d, out, gate)
    torch.cuda.synchronize()
    eager = _results(lay, d, out)

    lay, d, out = _buffers(moe, shape, dtype, routed)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        _step(moe, shape, dtype, x, idx, w, logits, y, lay, d, out, gate)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            _step(moe, shape, dtype, x, idx, w, logits, y, lay, d, out, gate)
    # every output must be rewritten by the replay; the workspace keeps its state (its sync words
    # are zero between calls)
    bufs = [t for t in list(d.values()) + [v for k, v in lay.items() if k != "workspace"] + [out] if t is not None]
    for replay in range(3):
        for t in bufs:
            t.view(torch.uint8).fill_(POISON)
        scratch = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        got = _results(lay, d, out)
        n = int(eager["num_recv"].item())
        assert int(got["num_recv"].item()) == n, f"replay {replay}"
        for k, v in eager.items():
            a, b = v, got[k]
            if k in ("recv_x", "recv_scales", "recv_src_idx", "recv_topk_idx", "recv_topk_w"):
                a, b = a[:n], b[:n]  # rows at or beyond num_recv are not written
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {replay}: {k}"
    del g


def _replay_check(capture, outputs, label):
    """Eager run, then 3 graph replays with outputs poisoned before each; every replay must reproduce
    the eager bytes exactly."""
    capture()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        capture()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            capture()
    for replay in range(3):
        for t in outputs:
            t.view(torch.uint8).fill_(POISON)
        torch.randn(1 << 20, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, outputs)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{label} replay {replay}: output {i}"
    del g


def test_graph_replays_low_latency_path():
    """moe_dispatch_ll (one-launch form at decode size) + moe_combine_ll in a graph."""
    import combine_get_dispatch_07_amd as moe
    from tests.gpu_harness import to_dev_bf16

    cfg = W.CONFIG_BY_NAME["decode"]
    print("[case] graph low-latency decode", flush=True)
    shape = moe.MoeShape(cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks)
    inp = W.make_inputs(cfg)
    x = to_dev_bf16(inp["x"])
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    d = moe.alloc_dispatch_ll(shape, "fp8")
    y = to_dev_bf16(W.draw_expert_outputs(np.random.default_rng(4), cfg.num_experts * cfg.num_tokens,
                                          cfg.hidden)).view(cfg.num_experts, cfg.num_tokens, cfg.hidden)
    out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")

    def step():
        moe.run_dispatch_ll(shape, "fp8", x, idx, d)
        moe.moe_combine_ll(shape, y, idx, w, d["slot_pos"], out)

    # recv_x / recv_src_idx rows beyond each expert's count are not written: compare counts, positions,
    # the combine output, and the written rows through the combine (which reads only those)
    _replay_check(step, [d["recv_count"], d["slot_pos"], out], "low-latency")


def test_graph_replays_backward():
    """moe_combine_backward + moe_dispatch_backward in a graph, on the prefill shape with 512 tokens."""
    import combine_get_dispatch_07_amd as moe
    from tests.gpu_harness import to_dev_bf16

    cfg = W.with_tokens(W.CONFIG_BY_NAME["prefill"], 512)
    print("[case] graph backward T=512", flush=True)
    shape = moe.MoeShape(cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks)
    inp = W.make_inputs(cfg)
    x = to_dev_bf16(inp["x"])
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    lay, d = moe.alloc_layout(shape), moe.alloc_dispatch(shape, "bf16")
    moe.run_layout(shape, idx, lay)
    moe.run_dispatch(shape, "bf16", x, idx, w, lay, d)
    torch.cuda.synchronize()
    n = int(d["num_recv"].item())
    rng = np.random.default_rng(6)
    g = to_dev_bf16(W.draw_expert_outputs(rng, cfg.num_tokens, cfg.hidden))
    y = to_dev_bf16(W.draw_expert_outputs(rng, n, cfg.hidden))
    grad_recv_w = torch.from_numpy(rng.standard_normal((n, cfg.num_topk)).astype(np.float32)).cuda()
    grad_y = torch.empty((n, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    grad_w = torch.empty((cfg.num_tokens, cfg.num_topk), dtype=torch.float32, device="cuda")
    grad_x = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    grad_topk_w = torch.empty_like(grad_w)

    def step():
        moe.moe_combine_backward(shape, g, y, idx, w, d["send_row"], grad_y, grad_w)
        moe.moe_dispatch_backward(shape, y, idx, d["send_row"], grad_x, grad_recv_w, grad_topk_w)

    _replay_check(step, [grad_y, grad_w, grad_x, grad_topk_w], "backward")


def test_graph_replays_one_call_send_side():
    """moe_layout_dispatch (one kernel at decode size) + moe_combine in a graph."""
    import combine_get_dispatch_07_amd as moe
    from tests.gpu_harness import to_dev_bf16

    cfg = W.CONFIG_BY_NAME["decode"]
    print("[case] graph one-call send side, decode", flush=True)
    shape = moe.MoeShape(cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks)
    inp = W.make_inputs(cfg)
    x = to_dev_bf16(inp["x"])
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    lay, d, out = _buffers(moe, shape, "fp8", False)
    y = to_dev_bf16(W.draw_expert_outputs(np.random.default_rng(5), shape.num_tokens * min(shape.num_topk,
                                                                                              shape.num_ranks),
                                          shape.hidden))

    def step():
        moe.run_layout_dispatch(shape, "fp8", x, idx, w, lay, d)
        moe.moe_combine(shape, y, idx, w, d["send_row"], out)

    step()
    torch.cuda.synchronize()
    n = int(d["num_recv"].item())  # receive rows at or beyond n are not written
    outputs = [lay["tokens_per_rank"], lay["tokens_per_expert"], lay["is_token_in_rank"], d["rank_offsets"],
               d["send_row"], d["num_recv"], d["recv_src_idx"][:n], d["recv_x"][:n], d["recv_scales"][:n], out]
    _replay_check(step, outputs, "one-call send side")


@pytest.mark.parametrize("name,T", [("decode", 128), ("prefill", 2048)])
def test_graph_replays_route_dispatch(name, T):
    """moe_route_dispatch (one kernel at decode size: its sync words must come back to zero after every
    launch, graph replays included) + moe_combine in a graph; 2048 tokens take the two-launch form."""
    import combine_get_dispatch_07_amd as moe
    from tests.gpu_harness import to_dev_bf16

    cfg = W.with_tokens(W.CONFIG_BY_NAME[name], T)
    print(f"[case] graph route+dispatch {name} T={T}", flush=True)
    gate = "sigmoid" if cfg.routing == "sigmoid" else "softmax"
    dtype = cfg.dispatch_dtype
    shape = moe.MoeShape(cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks)
    logits = torch.from_numpy(W.config_logits(cfg)).cuda()
    x = to_dev_bf16(W.make_inputs(cfg)["x"])
    lay, d, out = _buffers(moe, shape, dtype, True)
    y = to_dev_bf16(W.draw_expert_outputs(np.random.default_rng(7), shape.num_tokens * min(shape.num_topk,
                                                                                              shape.num_ranks),
                                          shape.hidden))

    def step():
        moe.run_route_dispatch(shape, dtype, logits, x, lay, d, gate)
        moe.moe_combine(shape, y, lay["topk_idx"], lay["topk_w"], d["send_row"], out)

    step()
    torch.cuda.synchronize()
    n = int(d["num_recv"].item())
    outputs = [lay["topk_idx"], lay["topk_w"], lay["tokens_per_rank"], lay["tokens_per_expert"],
               lay["is_token_in_rank"], d["rank_offsets"], d["send_row"], d["num_recv"], d["recv_src_idx"][:n],
               d["recv_topk_idx"][:n], d["recv_topk_w"][:n], d["recv_x"][:n], out]
    if dtype == "fp8":
        outputs.append(d["recv_scales"][:n])
    _replay_check(step, outputs, f"route+dispatch {name}")


@pytest.mark.parametrize("name,T", [("decode", 128), ("prefill", 2048)])
def test_graph_replays_noalloc_send_side(name, T):
    """moe_layout_dispatch_noalloc -- for callers under graph capture, which cannot allocate -- + moe_combine
    in a graph, against the same eager calls."""
    import combine_get_dispatch_07_amd as moe
    from tests.gpu_harness import to_dev_bf16

    cfg = W.with_tokens(W.CONFIG_BY_NAME[name], T)
    print(f"[case] graph no-alloc send side {name} T={T}", flush=True)
    dtype = cfg.dispatch_dtype
    shape = moe.MoeShape(cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks)
    inp = W.make_inputs(cfg)
    x = to_dev_bf16(inp["x"])
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    lay, d, out = _buffers(moe, shape, dtype, False)
    y = to_dev_bf16(W.draw_expert_outputs(np.random.default_rng(8), shape.num_tokens * min(shape.num_topk,
                                                                                              shape.num_ranks),
                                          shape.hidden))

    def step():
        moe.moe_layout_dispatch_noalloc(shape, dtype, x, idx, w, lay["tokens_per_rank"], lay["tokens_per_expert"],
                                        lay["is_token_in_rank"], d["recv_x"], d["recv_scales"], d["recv_src_idx"],
                                        d["recv_topk_idx"], d["recv_topk_w"], d["rank_offsets"], d["send_row"],
                                        d["num_recv"])
        moe.moe_combine(shape, y, idx, w, d["send_row"], out)

    step()
    torch.cuda.synchronize()
    n = int(d["num_recv"].item())
    outputs = [lay["tokens_per_rank"], lay["tokens_per_expert"], lay["is_token_in_rank"], d["rank_offsets"],
               d["send_row"], d["num_recv"], d["recv_src_idx"][:n], d["recv_x"][:n], out]
    _replay_check(step, outputs, f"no-alloc send side {name}")
