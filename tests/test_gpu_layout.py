"""is_token_in_rank rows from moe_get_dispatch_layout at every alignment the ABI allows.

Rows are written by whole waves as 16-byte pieces when R is a power of two >= 4 and the buffer is
16-byte aligned, else one lane per token (as 32-bit words when R % 4 == 0 and the buffer is 4-byte
aligned, else bytes).  All three forms, in the one-block (T <= 1024) and multi-block layouts, with
ragged last waves: the rows equal the oracle's, and the bytes before and after them (poisoned) are
untouched.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

MASK_CASES = [  # (T, E, k, R): ragged last wave in each
    (130, 64, 4, 8),
    (1000, 256, 8, 64),
    (1023, 128, 6, 4),
    (4097, 512, 8, 16),
    (2500, 256, 8, 32),
    (3000, 96, 4, 12),
    (1500, 40, 3, 5),
]


@pytest.mark.parametrize("offset", [0, 4, 1], ids=["aligned16", "offset4", "offset1"])
@pytest.mark.parametrize("case", MASK_CASES, ids=[f"T{c[0]}_R{c[3]}" for c in MASK_CASES])
def test_mask_rows_any_alignment(case, offset):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_get_dispatch_07_amd as moe

    T, E, k, R = case
    print(f"[case] mask rows T={T} E={E} k={k} R={R} offset={offset}", flush=True)
    rng = np.random.default_rng(T * 131 + R * 7 + offset)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    shape = moe.MoeShape(T, 128, k, E, R)
    lay = moe.alloc_layout(shape)
    guard = 64
    flat = torch.full((offset + T * R + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    lay["is_token_in_rank"] = flat[offset:offset + T * R].view(T, R)
    moe.run_layout(shape, torch.from_numpy(idx).cuda(), lay)
    torch.cuda.synchronize()
    host = flat.cpu().numpy()
    tpr, tpe, mask = O.get_dispatch_layout(idx, E, R)
    assert np.array_equal(host[offset:offset + T * R].reshape(T, R), mask)
    assert np.all(host[:offset] == 0xA5) and np.all(host[offset + T * R:] == 0xA5), "guard bytes"
    assert np.array_equal(lay["tokens_per_rank"].cpu().numpy(), tpr)
    assert np.array_equal(lay["tokens_per_expert"].cpu().numpy(), tpe)
