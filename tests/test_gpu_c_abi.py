"""The C ABI used from plain C (tests/c_abi_client.c): no torch in the process, only the header,
libmoe_ep.so and the HIP runtime.  The client checks its results itself (per-rank counts by hand,
combine of the received rows returning x bit for bit); this test runs it as a child process."""
import os
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_client")


def test_c_client_layout_dispatch_combine():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(CLIENT), "tests/c_abi_client is missing: run __graft_entry__.build()"
    print("[case] c abi client", flush=True)
    r = subprocess.run([CLIENT], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "match" in r.stdout
    # the host cost of each entry point (enqueue only), for the record
    costs = [line for line in r.stdout.splitlines() if line.startswith("host_us_per_call")]
    assert len(costs) == 11, r.stdout
    print("\n".join(costs), flush=True)
