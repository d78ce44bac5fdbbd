"""Comparison rules between the HIP path and the fp64 oracle.

Tolerances:
* Scores: the kernel forms each score as an fp32 sum of d products (fp16
  products are exact in fp32; fp32 inputs are fused multiply-adds) and one
  fp32 scaling by the rounded 1/sqrt(d). Any summation order of d terms errs
  by at most (d - 1) u sum|q_c k_c| and the scaling adds 2u relative, so
  |s_gpu - s| <= (d + 2) u sum_c |q_c k_c| / sqrt(d) + 2u |s| with u = 2^-24.
* Dense log-sum-exp: the score error shifts it by at most max_i of the bound
  above; the fp32 exponentials (relative error <= 2e-6 over the score range
  used) and a summation tree of depth <= 64 add < 1e-5. Tolerance:
  max score bound + 2e-5.
* Index sets: equal except for keys whose oracle score lies within 1e-4 of
  the N-th oracle score; sparse outputs within 2e-3 max-abs; delta within
  1e-4 absolute (the stated acceptance rules of the method's hot path).
* Two decodes of one selection that add in a different order (the fused
  select-and-decode against the split decode and its merge): each fp32 sum
  of n non-negative-weighted terms lies within (n - 1)u of the exact sum, and
  the two paths' exponentials (exp(s - m) against exp(s - m_split) *
  exp(m_split - m)) differ by a few u. So the outputs differ by at most
  (4(n - 1) + 8) u max|v|, and lse_sel (hence delta) by (2(n - 1) + 8) u.
"""

import math

import numpy as np

from oracle import prhs_oracle as O

U32 = 2.0 ** -24
SET_BAND = 1e-4
OUT_TOL = 2e-3
DELTA_TOL = 1e-4


def reorder_tols(n, vmax):
    """(output, lse) tolerances between two summation orders of n weighted rows."""
    return (4 * (n - 1) + 8) * U32 * max(float(vmax), 1.0), (2 * (n - 1) + 8) * U32


def fused_anchor_decode(dtype_f16, head_dim, n_heads, mode_topn, n_budget):
    """Whether the anchor step decodes inside the select kernel (the library's
    rule, the same for top-N and for the delta budget, where n_budget is the
    cap: fp16 rows of 128 and n_budget <= 2048, at any head count). n_heads and
    mode_topn are accepted for the callers' clarity only."""
    del mode_topn, n_heads
    return dtype_f16 and head_dim == 128 and n_budget <= 2048


def score_bound(q, K):
    """Per-element bound on |s_gpu - s| for q [B,Hq,d], K [B,Hkv,t,d] (float64 arrays)."""
    B, Hq, d = q.shape
    G = Hq // K.shape[1]
    out = np.empty((B, Hq, K.shape[2]))
    for b in range(B):
        for h in range(Hq):
            out[b, h] = (np.abs(K[b, h // G]) @ np.abs(q[b, h])) / math.sqrt(d)
    s = O.attention_scores(q, K)
    return (d + 2) * U32 * out + 2 * U32 * np.abs(s) + 1e-30, s


def check_set_band(gpu_idx, s_row, N):
    """GPU set vs oracle top-N: identical outside the tie band around the N-th score."""
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    t = s_row.shape[0]
    assert gpu_idx.size == N, (gpu_idx.size, N)
    assert np.all(np.diff(gpu_idx) > 0), "indices not strictly ascending"
    assert gpu_idx.min() >= 0 and gpu_idx.max() < t
    ref = O.topn_select(s_row, N)
    sN = np.sort(s_row)[::-1][N - 1]
    band = np.abs(s_row - sN) <= SET_BAND
    g = np.zeros(t, bool)
    g[gpu_idx] = True
    r = np.zeros(t, bool)
    r[ref] = True
    bad = (g != r) & ~band
    assert not bad.any(), f"{bad.sum()} keys differ outside the band (first {np.flatnonzero(bad)[:5]})"
    return bool((g == r).all())


def check_delta_choice(gpu_idx, gpu_count, s_row, lse, cap, delta_star, cap_hit=None):
    """DELTA mode: N*_gpu is accepted if delta(N*) <= delta* + 1e-4 and
    delta(N* - 1) > delta* - 1e-4; when the cap binds, the oracle's dropped mass
    at the cap must also exceed delta* (within 1e-4). The set is then checked
    as the top-N* set within the tie band."""
    n = int(gpu_count)
    assert 1 <= n <= cap
    a_desc = np.sort(np.exp(np.asarray(s_row, np.float64) - lse))[::-1]
    tail = np.concatenate([np.cumsum(a_desc[::-1])[::-1], [0.0]])   # tail[n]: dropped mass of top-n
    capped = n == cap and tail[cap] > delta_star + DELTA_TOL
    if not capped:
        assert tail[n] <= delta_star + DELTA_TOL, (n, tail[n], delta_star)
        if n > 1:
            assert tail[n - 1] > delta_star - DELTA_TOL, (n, tail[n - 1], delta_star)
    if cap_hit is not None:
        expect_hit = tail[cap] > delta_star
        if bool(cap_hit) != expect_hit:
            assert abs(tail[cap] - delta_star) <= DELTA_TOL
        if cap_hit:
            assert n == cap
    return check_set_band(gpu_idx, s_row, n)
