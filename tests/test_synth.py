"""The synthetic workloads carry the structure the pages report (CPU only)."""

import numpy as np
import torch

from oracle import prhs_oracle as O
from sparse_top_kv_head_amd.synth import CONFIGS, N_SINKS, make_workload


def _small(name, **kw):
    c = CONFIGS[name]
    base = dict(ctx_len=min(c.ctx_len, 2048), batch=1, steps=min(c.steps, 12))
    base.update(kw)
    if c.n_clusters[1] > 32:
        base["n_clusters"] = (16, 32) if c.n_clusters[0] != c.n_clusters[1] else (24, 24)
    return c.replace(**base)


def test_shapes_dtypes_and_determinism():
    for name in CONFIGS:
        cfg = _small(name)
        w1 = make_workload(cfg)
        w2 = make_workload(cfg)
        assert w1.K.shape == (cfg.batch, cfg.n_kv_heads, cfg.ctx_len, cfg.head_dim)
        assert w1.V.shape == w1.K.shape and w1.K.dtype == cfg.torch_dtype
        assert w1.q.shape == (cfg.steps, cfg.batch, cfg.n_q_heads, cfg.head_dim)
        assert torch.equal(w1.K, w2.K) and torch.equal(w1.V, w2.V) and torch.equal(w1.q, w2.q)
        assert torch.isfinite(w1.K.float()).all() and torch.isfinite(w1.V.float()).all()


def test_adjacent_queries_are_similar():
    """Fig. 2 / Fig. 10: consecutive per-head queries have cosine above 0.8."""
    for name in ("toy", "llama2_4k", "mistral_gqa_32k"):
        q = make_workload(_small(name)).q.double().numpy()
        cos = (q[1:] * q[:-1]).sum(-1) / np.linalg.norm(q[1:], axis=-1) / np.linalg.norm(q[:-1], axis=-1)
        assert cos.min() > 0.8


def test_planted_clusters_rank_high_at_their_step():
    """Fig. 2 / Fig. 11: critical keys sit in contiguous clusters; the planted runs
    score well above the background at the step whose query they follow."""
    cfg = _small("llama2_4k")
    w = make_workload(cfg)
    q = w.q.double().numpy()
    K = w.K.double().numpy()
    hits, total, z = 0, 0, []
    for (b, g, start, L, owner, step) in w.clusters[:64]:
        s = O.attention_scores(q[step][b:b + 1, owner:owner + 1], K[b:b + 1, g:g + 1])[0, 0]
        hits += int((s[start:start + L] > np.median(s)).sum())
        total += L
        z.append((s[start:start + L].mean() - s.mean()) / s.std())
    # bias 1.5 along the unit query adds about 1.5 (the background std is about 1.05-1.2)
    assert hits / total > 0.85
    assert np.mean(z) > 0.75


def test_sinks_rank_at_top():
    cfg = _small("llama2_4k")
    w = make_workload(cfg)
    s = O.attention_scores(w.q[0].double().numpy(), w.K.double().numpy())
    inside, z = 0, []
    for h in range(cfg.n_q_heads):
        S = O.topn_select(s[0, h], 128)
        inside += len(set(range(N_SINKS)) & set(S.tolist()))
        z.append((s[0, h, :N_SINKS].mean() - s[0, h].mean()) / s[0, h].std())
    # sink bias 3.0 along the head's unit query: about 3 standard deviations at step 0
    assert inside / (N_SINKS * cfg.n_q_heads) > 0.6
    assert np.mean(z) > 2.0


def test_clusters_do_not_overlap_and_skip_sinks():
    cfg = _small("mistral_gqa_32k")
    w = make_workload(cfg)
    for b in range(cfg.batch):
        for g in range(cfg.n_kv_heads):
            runs = sorted((s, L) for (bb, gg, s, L, _, _) in w.clusters if bb == b and gg == g)
            for (s0, l0), (s1, _) in zip(runs, runs[1:]):
                assert s0 + l0 <= s1
            assert all(s >= N_SINKS and s + L <= cfg.ctx_len for s, L in runs)
            owners = {o for (bb, gg, _, _, o, _) in w.clusters if bb == b and gg == g}
            assert all(g * cfg.group <= o < (g + 1) * cfg.group for o in owners)
