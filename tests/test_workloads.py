"""The seeded input generator: determinism and routing recipes (no GPU).

Routing is input synthesis, not the hot path; beyond determinism and the
checks below its realism is parity unpinned.
"""
import numpy as np
import pytest

import workloads as W


def test_deterministic_per_seed():
    cfg = W.CONFIG_BY_NAME["tiny"]
    a, b = W.make_inputs(cfg), W.make_inputs(cfg)
    for key in a:
        assert np.array_equal(a[key], b[key])
    other = W.make_inputs(W.CONFIGS[1])
    assert not np.array_equal(a["topk_idx"][:4, :4], other["topk_idx"][:4, :4])


def _brute_topk(row, k):
    # repeatedly take the largest remaining score; on equal scores the lower id wins
    left = list(range(len(row)))
    out = []
    for _ in range(k):
        best = left[0]
        for e in left[1:]:
            if row[e] > row[best]:
                best = e
        out.append(best)
        left.remove(best)
    return out


def test_topk_ties_go_to_lower_id():
    scores = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, 0.5]], dtype=np.float32)
    assert W._stable_topk(scores, 4).tolist() == [[1, 2, 4, 3]]
    rng = np.random.default_rng(0)
    s = rng.integers(0, 4, size=(50, 12)).astype(np.float32)  # many ties
    got = W._stable_topk(s, 5)
    for t in range(50):
        assert got[t].tolist() == _brute_topk(s[t].tolist(), 5)


@pytest.mark.parametrize("cfg", W.CONFIGS, ids=lambda c: c.name)
def test_routing_shapes_and_weights(cfg):
    g = W.seed_streams(cfg.index)
    idx, w = W.route(cfg, g[1], g[3], num_tokens=min(cfg.num_tokens, 2048))
    assert idx.dtype == np.int32 and w.dtype == np.float32
    assert idx.shape == w.shape == (min(cfg.num_tokens, 2048), cfg.num_topk)
    assert ((idx >= 0) & (idx < cfg.num_experts)).all()
    srt = np.sort(idx, axis=1)
    assert (np.diff(srt, axis=1) > 0).all()  # distinct experts per token
    assert (w > 0).all()
    assert np.allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=cfg.num_topk * 2.0 ** -23)


def test_group_limited_stays_in_top_groups():
    cfg = W.CONFIG_BY_NAME["group_limited"]
    g = W.seed_streams(cfg.index)
    logits = np.random.default_rng(g[1].bit_generator.seed_seq).standard_normal((64, 256), dtype=np.float32)
    idx, _ = W.route(cfg, np.random.default_rng(g[1].bit_generator.seed_seq), g[3], num_tokens=64)
    per = cfg.num_experts // cfg.num_groups
    gmax = logits.reshape(64, cfg.num_groups, per).max(axis=2)
    for t in range(64):
        top_groups = set(np.argsort(-gmax[t], kind="stable")[:cfg.topk_groups].tolist())
        assert {int(e) // per for e in idx[t]} <= top_groups
        # the chosen experts are the best 8 among the allowed groups
        allowed = [e for e in range(256) if e // per in top_groups]
        best = sorted(allowed, key=lambda e: (-logits[t, e], e))[:cfg.num_topk]
        assert idx[t].tolist() == best


def test_zipf_first_pick_frequency():
    # Gumbel-top-k: the first pick is exactly Zipf(s) over the permuted popularity order
    cfg = W.with_tokens(W.CONFIG_BY_NAME["skewed"], 40000)
    g = W.seed_streams(cfg.index)
    perm_rng = np.random.default_rng(g[3].bit_generator.seed_seq)
    idx, _ = W.route(cfg, g[1], g[3])
    perm = perm_rng.permutation(cfg.num_experts)
    pos = np.empty(cfg.num_experts, dtype=np.int64)
    pos[perm] = np.arange(1, cfg.num_experts + 1)
    first = pos[idx[:, 0]]
    p = np.arange(1, cfg.num_experts + 1, dtype=np.float64) ** -cfg.zipf_s
    p /= p.sum()
    obs = np.bincount(first, minlength=cfg.num_experts + 1)[1:]
    # hottest expert: p1 = 0.2536; a 5-sigma band
    n = idx.shape[0]
    assert abs(obs[0] / n - p[0]) < 5 * np.sqrt(p[0] * (1 - p[0]) / n)
    # chi-square over the top 30 ranks plus a tail bin
    exp = np.concatenate([p[:30], [p[30:].sum()]]) * n
    o = np.concatenate([obs[:30], [obs[30:].sum()]])
    chi2 = ((o - exp) ** 2 / exp).sum()
    assert chi2 < 80  # 30 dof: 99.99th percentile is about 66


def test_hidden_values_are_bf16_normal():
    x = W.draw_hidden(np.random.default_rng(5), 256, 512)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(f.mean()) < 0.01 and abs(f.std() - 1.0) < 0.01
