"""The E4M3 rounding of the FP8 dispatch, on its own (moe_encode_e4m3: the device helper the
dispatch's quantiser uses), against the oracle's encoder over every fp32 magnitude below 464 --
the range that x / s reaches, since |x| <= amax and s = fl32(max(amax, 1e-4) / 448).

The argument, all of it checked here: the GPU encodes every non-negative fp32 bit pattern below
464.0f (about 1.14e9 values, in chunks); the codes must not decrease as the pattern grows (the
values grow with it), and at every place where they change the oracle must give the same code on
both sides.  A non-decreasing step function that agrees with the oracle's (monotone) rounding on
both sides of each of its steps and at both ends equals it everywhere.  Negative values: the code
of -v must be the code of v with the sign bit set, for every one of those patterns.
"""
import numpy as np
import pytest
import torch

from oracle import numerics as N

pytestmark = pytest.mark.gpu

LIMIT = 0x43E80000  # bit pattern of 464.0f
CHUNK = 1 << 28


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_encode_matches_oracle_everywhere_below_464():
    import combine_get_dispatch_07_amd as moe

    print(f"[case] e4m3 encode, {LIMIT} magnitudes x 2 signs", flush=True)
    left, right = [], []  # bit patterns on both sides of every change of code
    prev_last = None
    for lo in range(0, LIMIT, CHUNK):
        hi = min(lo + CHUNK, LIMIT)
        vals = torch.arange(lo, hi, dtype=torch.int32, device="cuda").view(torch.float32)
        codes = torch.empty(hi - lo, dtype=torch.uint8, device="cuda")
        moe.moe_encode_e4m3(vals, codes)
        neg_codes = torch.empty_like(codes)
        moe.moe_encode_e4m3(-vals, neg_codes)
        assert torch.equal(neg_codes, codes | 0x80), f"sign handling in [{lo:#x}, {hi:#x})"
        del neg_codes
        assert not bool((codes[1:] < codes[:-1]).any()), f"codes decrease in [{lo:#x}, {hi:#x})"
        if prev_last is not None:
            assert int(codes[0]) >= prev_last
            if int(codes[0]) != prev_last:
                left.append(lo - 1)
                right.append(lo)
        steps = torch.nonzero(codes[1:] != codes[:-1]).flatten().cpu().numpy().astype(np.int64) + lo
        left.extend(steps.tolist())
        right.extend((steps + 1).tolist())
        prev_last = int(codes[-1])
        if lo == 0:
            first_code = int(codes[0])
        del vals, codes
    torch.cuda.empty_cache()

    # 127 non-negative finite codes below 464 (0x00 .. 0x7E): 126 steps
    assert len(left) == 126, len(left)
    u = np.array([0] + left + right + [LIMIT - 1], dtype=np.uint32)
    got = moe_codes(u)
    want = N.e4m3_encode_rne(u.view(np.float32))
    assert np.array_equal(got, want), np.nonzero(got != want)
    assert first_code == int(want[0]) and prev_last == int(want[-1])


def moe_codes(patterns):
    """Codes of the given fp32 bit patterns through moe_encode_e4m3."""
    import combine_get_dispatch_07_amd as moe

    vals = torch.from_numpy(patterns.view(np.float32)).cuda()
    codes = torch.empty(vals.numel(), dtype=torch.uint8, device="cuda")
    moe.moe_encode_e4m3(vals, codes)
    return codes.cpu().numpy()


def test_encode_small_and_ragged_sizes():
    rng = np.random.default_rng(5)
    for n in (1, 2, 3, 5, 1023, 1025):
        v = (rng.standard_normal(n) * 100).astype(np.float32)
        v = np.clip(v, -463.0, 463.0)
        assert np.array_equal(moe_codes(v.view(np.uint32)), N.e4m3_encode_rne(v)), n
