"""CU-budget streams: results on a stream restricted to a subset of CUs match the oracle exactly."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("first_cu,num_cus", [(0, 8), (0, 32), (32, 224)])
def test_path_on_cu_limited_stream(first_cu, num_cus):
    import combine_get_dispatch_07_amd as moe
    from tests.gpu_harness import bf16_to_np, to_dev_bf16
    print(f"[case] cu budget first={first_cu} n={num_cus}", flush=True)
    cfg = W.with_tokens(W.CONFIG_BY_NAME["group_limited"], 600)
    d = W.make_inputs(cfg)
    x, idx, w = d["x"], d["topk_idx"], d["topk_w"]
    E, R, H, k = cfg.num_experts, cfg.num_ranks, cfg.hidden, cfg.num_topk
    shape = moe.MoeShape(cfg.num_tokens, H, k, E, R)
    xd, idx_d, w_d = to_dev_bf16(x), torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
    lay = moe.alloc_layout(shape)
    disp = moe.alloc_dispatch(shape, "fp8")
    ref = O.run_all(x, idx, w, E, R, "fp8")
    n = int(ref["num_recv"])
    y = W.draw_expert_outputs(np.random.default_rng(3), n, H)
    yd = to_dev_bf16(y)
    out = torch.empty((cfg.num_tokens, H), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    h = moe.stream_create_cu_range(first_cu, num_cus)
    try:
        moe.run_layout(shape, idx_d, lay, stream=h)
        moe.run_dispatch(shape, "fp8", xd, idx_d, w_d, lay, disp, stream=h)
        moe.moe_combine(shape, yd, idx_d, w_d, disp["send_row"], out, stream=h)
        torch.cuda.ExternalStream(h).synchronize()
    finally:
        moe.stream_destroy(h)
    assert np.array_equal(lay["is_token_in_rank"].cpu().numpy(), ref["is_token_in_rank"])
    assert np.array_equal(disp["send_row"].cpu().numpy(), ref["send_row"])
    assert np.array_equal(disp["recv_x"][:n].cpu().numpy(), ref["recv_x"])
    assert np.array_equal(disp["recv_scales"][:n].cpu().numpy().view(np.uint32), ref["recv_scales"].view(np.uint32))
    assert np.array_equal(bf16_to_np(out), O.combine(y, idx, w, ref["send_row"], E, R))


def test_cu_range_checks():
    import combine_get_dispatch_07_amd as moe
    for first, count in [(0, 12), (4, 8), (8, 10000), (-8, 16), (256, 8)]:
        with pytest.raises(moe.MoeError) as e:
            moe.stream_create_cu_range(first, count)
        assert e.value.code == 1, (first, count)
    h = moe.stream_create_cu_range(0, 0)  # unrestricted
    moe.stream_destroy(h)
    torch.zeros(1, device="cuda").sum().item()  # no error left behind
