"""moe_layout_dispatch_noalloc -- the dispatch plan in the library's static device array -- against
moe_layout_dispatch with a caller workspace, through the C ABI: bit-identical outputs on consecutive
calls, each smaller than the one before, across the multi-block path (above 1024 tokens) and the
one-kernel path (decode size, FP8)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

# (workload, tokens): consecutive calls on the shared array, each smaller than the one before
CALLS = [("prefill", 4096), ("prefill", 1500), ("decode", 128), ("tiny", 64)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs(lay, d, n):
    out = {k: lay[k].clone() for k in ("tokens_per_rank", "tokens_per_expert", "is_token_in_rank")}
    for k in ("rank_offsets", "send_row", "num_recv"):
        out[k] = d[k].clone()
    for k in ("recv_x", "recv_scales", "recv_src_idx", "recv_topk_idx", "recv_topk_w"):
        if d[k] is not None:
            out[k] = d[k][:n].clone()
    return out


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    import combine_get_dispatch_07_amd as moe
    from tests.gpu_harness import POISON, _poison, to_dev_bf16

    for name, T in CALLS:
        cfg = W.with_tokens(W.CONFIG_BY_NAME[name], T)
        dtype = cfg.dispatch_dtype
        print(f"[case] noalloc {name} T={T} {dtype}", flush=True)
        inp = W.make_inputs(cfg)
        shape = moe.MoeShape(cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_experts, cfg.num_ranks)
        x = to_dev_bf16(inp["x"])
        idx = torch.from_numpy(inp["topk_idx"]).cuda()
        w = torch.from_numpy(inp["topk_w"]).cuda()

        lay_a, d_a = moe.alloc_layout(shape), moe.alloc_dispatch(shape, dtype)
        _poison(lay_a)
        _poison(d_a)
        moe.run_layout_dispatch(shape, dtype, x, idx, w, lay_a, d_a)

        lay_b, d_b = moe.alloc_layout(shape), moe.alloc_dispatch(shape, dtype)
        _poison(lay_b)
        _poison(d_b)
        moe.moe_layout_dispatch_noalloc(shape, dtype, x, idx, w, lay_b["tokens_per_rank"], lay_b["tokens_per_expert"],
                                        lay_b["is_token_in_rank"], d_b["recv_x"], d_b["recv_scales"],
                                        d_b["recv_src_idx"], d_b["recv_topk_idx"], d_b["recv_topk_w"],
                                        d_b["rank_offsets"], d_b["send_row"], d_b["num_recv"])
        torch.cuda.synchronize()
        n = int(d_a["num_recv"].item())
        assert n > 0 and int(d_b["num_recv"].item()) == n
        a, b = _outputs(lay_a, d_a, n), _outputs(lay_b, d_b, n)
        for k in a:
            assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), f"{name} T={T}: {k}"
        # rows at or beyond num_recv stay untouched
        assert (d_b["recv_src_idx"][n:].view(torch.uint8) == POISON).all()
        assert (d_b["recv_x"][n:].view(torch.uint8) == POISON).all()
