"""fp64 reference semantics of the PrHS decode hot path (test infrastructure only).

Citations name the page "Near-Oracle KV Selection via Pre-hoc Sparsity for
Long-Context Inference" (its thelatestinai.com card) and the passage on it.
Where the pages leave a step open, the reading taken is stated in place.

Conventions shared by every function:

* ``q``: [B, H_q, d]; ``K``, ``V``: [B, H_kv, t, d]; query head ``h`` reads KV
  head ``h // G`` with ``G = H_q // H_kv`` (grouped-query attention).
* All arithmetic is float64 on the stored input values (fp16 or fp32 inputs
  are widened exactly).
* Index sets are returned as ascending int64 arrays of unique indices.
"""

from __future__ import annotations

import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Scores and dense attention weights
# ---------------------------------------------------------------------------

def attention_scores(q, K):
    """Scaled dot-product score of a decode query against every cached key.

    Table I names the query q, the per-head dimension d and the KV cache K; the
    attention weights A(.) it lists are the softmax of these scores. The scale
    1/sqrt(d) is the standard scaled dot product (the pages cite "Attention is
    all you need" for it and print no other scale).

    q: [B, H_q, d]; K: [B, H_kv, t, d]  ->  s: [B, H_q, t] float64.
    """
    q = _f64(q)
    K = _f64(K)
    B, Hq, d = q.shape
    Bk, Hkv, t, dk = K.shape
    if Bk != B or dk != d or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    s = np.empty((B, Hq, t), dtype=np.float64)
    inv = 1.0 / math.sqrt(d)
    for b in range(B):
        for h in range(Hq):
            s[b, h] = (K[b, h // G] @ q[b, h]) * inv
    return s


def dense_softmax(s):
    """Dense attention weights over all t keys and their log-sum-exp.

    Table I: A(.) is the attention weight; the retained and dropped masses
    tau(.) and delta(.) are fractions of it, so its normaliser is the dense
    softmax over every key of the step (reading: per query head, per step).

    Returns (A, lse) with A = exp(s - lse) along the last axis.
    """
    s = _f64(s)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    A = e / z
    lse = (m + np.log(z))[..., 0]
    return A, lse


# ---------------------------------------------------------------------------
# Selectors
# ---------------------------------------------------------------------------

def _descending_order(s_row):
    """Key order of the top-k oracle: score descending, lower index first on ties.

    The pages do not say how ties at the N-th score are broken; the lower index
    wins here. Softmax is monotone, so ranking by score equals ranking by
    attention weight (Fig. 2 and Fig. 9 rank by the top-k oracle).
    """
    s_row = _f64(s_row)
    idx = np.arange(s_row.shape[0])
    return np.lexsort((idx, -s_row))


def topn_select(s_row, N):
    """Top-k oracle: the N keys of highest attention weight (Fig. 1, Fig. 2, Fig. 9).

    Table I: the selector S returns a subset of indices; S_t is the set chosen
    at step t within the KV budget N. The oracle keeps the N largest weights,
    which minimises the dropped mass delta over all subsets of size N.
    Returned in ascending index order.
    """
    t = len(s_row)
    if not (1 <= N <= t):
        raise ValueError("budget N must lie in [1, t]")
    order = _descending_order(s_row)
    return np.sort(order[:N])


def delta_budget_select(s_row, lse, N_cap, delta_star):
    """Dropped-mass-controlled selection (Abstract: control delta in advance).

    Reading: the smallest N >= 1 whose top-N set leaves dropped mass
    delta <= delta_star (inclusive), capped at N_cap. The dropped mass of the
    top-n set is the sum of the weights not taken, accumulated from the
    smallest weight upward (a direct tail sum, no 1 - sum cancellation).

    Returns (idx ascending, N_star, cap_hit).
    """
    s_row = _f64(s_row)
    t = len(s_row)
    if not (1 <= N_cap <= t):
        raise ValueError("cap must lie in [1, t]")
    order = _descending_order(s_row)
    a_sorted = np.exp(s_row[order] - float(lse))
    # tail[n] = sum_{j >= n} a_sorted[j]: dropped mass after keeping the first n.
    tail = np.concatenate([np.cumsum(a_sorted[::-1])[::-1], [0.0]])
    N_star = None
    for n in range(1, N_cap + 1):
        if tail[n] <= delta_star:
            N_star = n
            break
    cap_hit = N_star is None
    if cap_hit:
        N_star = N_cap
    return np.sort(order[:N_star]), N_star, cap_hit


# ---------------------------------------------------------------------------
# Critical-index-set (CIS) sharing across adjacent decode steps
# ---------------------------------------------------------------------------

def cis_dilate(anchor_idx, r, t):
    """Dilate a critical-index set for reuse by later queries (Fig. 4, Table VIII).

    Fig. 4 shares the critical tokens of one query with the next two and grows
    the shared set around its clusters; Table VIII tunes a radius r in {1, 2}.
    Reading: every anchor index i contributes the window [i - r, i + r] clipped
    to [0, t); the shared set is the union of these windows (r = 0 is the
    DirectReuse control of Table VI).
    """
    if r < 0:
        raise ValueError("radius must be >= 0")
    mask = np.zeros(t, dtype=bool)
    for i in np.asarray(anchor_idx, dtype=np.int64):
        lo = max(0, int(i) - r)
        hi = min(t - 1, int(i) + r)
        mask[lo:hi + 1] = True
    return np.flatnonzero(mask)


def random_expansion(anchor_idx, draws, m):
    """The RandomExpansion control of Table VI (Panel A): the anchor's set grown
    to a matched size m with keys chosen at random instead of by dilation.

    Reading (the pages give the control's name and its matched budget only):
    the random choice is made by per-key draws passed in as an input, so that
    any implementation makes the same choice: the m - |S_a| keys outside the
    anchor set with the smallest draws, the lower index winning equal draws.
    Draws are used as 23-bit integers (draws & 0x7FFFFF).

    anchor_idx: ascending anchor set; draws: [t] non-negative integers; m:
    target size, |S_a| <= m <= t. Returns the ascending expanded set.
    """
    S = np.asarray(anchor_idx, dtype=np.int64)
    d = np.asarray(draws, dtype=np.int64) & 0x7FFFFF
    t = d.size
    if not S.size <= m <= t:
        raise ValueError("m outside [|S_a|, t]")
    member = np.zeros(t, dtype=bool)
    member[S] = True
    outside = np.flatnonzero(~member)
    order = np.lexsort((outside, d[outside]))     # by draw, then by index
    extra = outside[order[:m - S.size]]
    return np.sort(np.concatenate([S, extra]))


def cis_schedule(n_steps, period, q_steps=None, sim_tau=None):
    """Which decode steps run exact retrieval, and which anchor each step reuses.

    Table IV/VIII: the CIS block size s; reading: one exact top-k retrieval per
    block of ``period`` steps, the rest reuse the most recent anchor's exact set
    (Fig. 4 shares query 405's set with both 406 and 407: it is not chained).
    Fig. 8 / Fig. 9(c): sharing is allowed only while sim(q, q') >= tau; when
    ``sim_tau`` is given (per-head cosine of the current and anchor query), a
    step whose cosine falls below it becomes an anchor as well.

    q_steps: optional [n_steps, d] queries of one head (needed for the gate).
    Returns a list of (is_anchor, anchor_step) per step.
    """
    out = []
    anchor = None
    for s in range(n_steps):
        make_anchor = (s % period == 0) or anchor is None
        if not make_anchor and sim_tau is not None:
            a = _f64(q_steps[anchor])
            b = _f64(q_steps[s])
            cos = float(a @ b) / (np.linalg.norm(a) * np.linalg.norm(b))
            make_anchor = cos < sim_tau
        if make_anchor:
            anchor = s
        out.append((make_anchor, anchor))
    return out


# ---------------------------------------------------------------------------
# Sparse attention and the mass bookkeeping
# ---------------------------------------------------------------------------

def sparse_attention(s_row, V_head, S):
    """Attention restricted to the selected entries (Abstract; Table V caption).

    Reading: the softmax is renormalised over S, so
    o_S = sum_{i in S} exp(s_i - m_S) v_i / sum_{i in S} exp(s_i - m_S)
    with m_S = max_{i in S} s_i, and lse_S = m_S + log sum_{i in S} exp(s_i - m_S).

    Returns (o_S [d], lse_S).
    """
    s_row = _f64(s_row)
    S = np.asarray(S, dtype=np.int64)
    if S.size == 0:
        raise ValueError("empty selection")
    sv = s_row[S]
    m = sv.max()
    w = np.exp(sv - m)
    l = w.sum()
    o = (w @ _f64(V_head)[S]) / l
    return o, m + math.log(l)


def dropped_mass(s_row, S):
    """Dropped and retained attention mass of a selection (Table I: delta(.), tau(.)).

    delta(S) is the dense attention mass of the keys not in S, summed directly;
    tau(S) = 1 - delta(S).
    """
    A, _ = dense_softmax(s_row)
    keep = np.zeros(A.shape[-1], dtype=bool)
    keep[np.asarray(S, dtype=np.int64)] = True
    delta = float(A[~keep].sum())
    return delta, 1.0 - delta


def overlap_with_oracle(D, S_star):
    """Share of the oracle's critical set found in a reused set (Fig. 4 overlap)."""
    S_star = np.asarray(S_star)
    return np.intersect1d(np.asarray(D), S_star).size / S_star.size


def beta_emp(s_row, S):
    """Retained-mass gap to the oracle at equal size (Tables VI and VII: beta_emp).

    beta_emp(S) = tau(TopK_|S|) - tau(S), non-negative since the oracle set of
    that size keeps the most mass.
    """
    S = np.asarray(S)
    d_sel, _ = dropped_mass(s_row, S)
    d_top, _ = dropped_mass(s_row, topn_select(s_row, S.size))
    return d_sel - d_top


# ---------------------------------------------------------------------------
# One decode step over all (or sampled) heads
# ---------------------------------------------------------------------------

def decode_step(q, K, V, mode, N=None, delta_star=None, sets=None, heads=None):
    """One pass of the hot path: score, select, sparse attention, delta/tau.

    mode: "topn" (budget N), "delta" (cap N, target delta_star) or "given"
    (``sets[(b, h)]`` supplies the index set, e.g. a dilated CIS).
    heads: optional list of (b, h) pairs to evaluate (sampling at full size);
    default all heads.

    Returns a dict keyed by (b, h) with idx, count, cap_hit, out, lse_sel,
    lse_all, delta, tau.
    """
    q = _f64(q)
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    res = {}
    for (b, h) in heads:
        s = attention_scores(q[b:b + 1, h:h + 1], K[b:b + 1, h // G:h // G + 1])[0, 0]
        _, lse_all = dense_softmax(s)
        cap_hit = False
        if mode == "topn":
            S = topn_select(s, N)
        elif mode == "delta":
            S, _, cap_hit = delta_budget_select(s, lse_all, N, delta_star)
        elif mode == "given":
            S = np.asarray(sets[(b, h)], dtype=np.int64)
        else:
            raise ValueError(mode)
        o, lse_S = sparse_attention(s, V[b, h // G], S)
        delta, tau = dropped_mass(s, S)
        res[(b, h)] = dict(idx=S, count=int(S.size), cap_hit=cap_hit, out=o,
                           lse_sel=lse_S, lse_all=float(lse_all), delta=delta,
                           tau=tau, scores=s)
    return res
