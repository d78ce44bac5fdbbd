"""Host checks of the bench's diagnostics: the retained-mass gap beta_emp and
the overlap with the exact top-N that the CIS sweeps report (computed on the
device from the library's own outputs) against the oracle's definitions
(Tables VI/VII: beta_emp; Fig. 4: overlap), on CPU tensors."""

import types

import numpy as np
import torch

import bench
from oracle import prhs_oracle as O


def _fake_diag(s, M):
    """What DecodeEngine holds after score + TOPN select of M: the exact
    top-M indices ascending, their scores in that order, and lse_all."""
    B, H, t = s.shape
    idx = np.zeros((B, H, M), dtype=np.int32)
    sel = np.zeros((B, H, M), dtype=np.float32)
    lse = np.zeros((B, H), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            S = O.topn_select(s[b, h].astype(np.float64), M)
            idx[b, h] = S
            sel[b, h] = s[b, h, S]
            lse[b, h] = O.dense_softmax(s[b, h].astype(np.float64))[1]
    return types.SimpleNamespace(sel_scores=torch.from_numpy(sel), idx=torch.from_numpy(idx),
                                 lse_all=torch.from_numpy(lse),
                                 dims=types.SimpleNamespace(ctx_len=t))


def test_reuse_quality_matches_oracle():
    rng = np.random.default_rng(7)
    B, H, t, M, N, cap = 2, 3, 300, 120, 40, 130
    s = (rng.standard_normal((B, H, t)) * 2.0).astype(np.float32)
    diag = _fake_diag(s, M)
    S_idx = np.full((B, H, cap), -1, dtype=np.int32)
    S_cnt = np.zeros((B, H), dtype=np.int32)
    lse_sel = np.zeros((B, H), dtype=np.float32)
    sets = {}
    for b in range(B):
        for h in range(H):
            # a mix of the exact top keys and random ones, sizes up to M
            n = int(rng.integers(1, M + 1))
            top = O.topn_select(s[b, h].astype(np.float64), n)
            pool = np.union1d(top[: n // 2], rng.choice(t, size=n, replace=False))
            S = np.sort(pool[:n])
            sets[(b, h)] = S
            S_idx[b, h, :S.size] = S
            S_cnt[b, h] = S.size
            lse_sel[b, h] = O.sparse_attention(s[b, h].astype(np.float64),
                                               np.zeros((t, 1)), S)[1]
    beta, overlap = bench.reuse_quality(diag, M, N, torch.from_numpy(S_idx), torch.from_numpy(S_cnt),
                                        torch.from_numpy(lse_sel))
    for (b, h), S in sets.items():
        row = s[b, h].astype(np.float64)
        assert abs(float(beta[b, h]) - O.beta_emp(row, S)) < 1e-5, (b, h)
        assert float(overlap[b, h]) == O.overlap_with_oracle(S, O.topn_select(row, N)), (b, h)


def test_pages_context_quotes_the_abstract_and_picks_the_largest_ratio():
    """The context block carries the pages' A100 figures (Abstract) unchanged and
    this run's largest dense-over-CIS-16 ratio with its shape."""
    ctx = bench.pages_context()
    assert ctx["attention_operator_latency_speedup_over_dense"] == 9.9
    assert ctx["throughput_gain_over_dense"] == 2.8 and "this_run" not in ctx
    rows = [{"batch": 8, "ctx_len": 2048, "dense_over_cis16": 2.0, "dense_over_anchor": 1.3},
            {"batch": 16, "ctx_len": 16384, "dense_over_cis16": 9.0, "dense_over_anchor": 1.9},
            {"batch": 8, "ctx_len": 16384, "dense_over_cis16": 8.9, "dense_over_anchor": 2.0}]
    run = bench.pages_context({"rows": rows})["this_run"]
    assert run["dense_over_cis16_max"] == 9.0 and run["shape"] == "batch 16, t 16384"
    assert run["dense_over_anchor_same_shape"] == 1.9
