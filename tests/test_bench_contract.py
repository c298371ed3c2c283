"""bench.py's contract on the CPU: refusal of more than one GPU, and the algorithmic byte counts.

The byte counts are what a step must move once (distinct rows once): they are recomputed here from
the formulas written out, on the prefill workload with a fixed receive-row count.
"""
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_prefill():
    cfg = W.CONFIG_BY_NAME["prefill"]
    T, H, E, k, R, n = cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.num_topk, cfg.num_ranks, 21687
    b = bench.algorithmic_bytes(cfg, n)
    assert b["layout"] == T * k * 4 + T * R + 4 * (R + E)
    # bf16 rows: H * 2 bytes, no scales; per receive row 4 bytes of source index and 8k of ids and weights
    assert b["dispatch"] == T * H * 2 + T * k * 8 + T * R + n * (H * 2 + 4 + 8 * k) + T * R * 4
    assert b["combine"] == n * H * 2 + T * k * 8 + T * R * 4 + T * H * 2


def test_algorithmic_bytes_fp8_scales():
    cfg = W.CONFIG_BY_NAME["decode"]
    T, H, k, R, n = cfg.num_tokens, cfg.hidden, cfg.num_topk, cfg.num_ranks, 678
    b = bench.algorithmic_bytes(cfg, n)
    # FP8 rows: H bytes of codes plus one fp32 scale per 128 channels
    assert b["dispatch"] == T * H * 2 + T * k * 8 + T * R + n * (H + 4 * H // 128 + 4 + 8 * k) + T * R * 4


def test_rotation_keeps_source_rows_out_of_the_last_level_cache():
    llc = 256 << 20
    for cfg in W.CONFIGS:
        x_bytes = cfg.num_tokens * cfg.hidden * 2
        n = bench.rotation_sets(10 << 20, x_bytes)
        assert 3 <= n <= bench.MAX_SETS
        if n < bench.MAX_SETS:  # the other sets' source rows cover twice the cache
            assert (n - 1) * x_bytes >= 2 * llc, cfg.name
    assert bench.rotation_sets(900 << 20, 4096 * 7168 * 2) == 11  # prefill: 58.7 MB of rows per set
    assert bench.rotation_sets(3 << 30, 16384 * 7168 * 2) == 4    # 16384 tokens: 235 MB per set
    assert bench.rotation_sets(20 << 20, 128 * 7168 * 2) == bench.MAX_SETS  # decode
