"""Pins of the fp64 oracle against things other than itself.

Each ``check_*`` helper encodes one pin: a closed form, a brute force over
subsets, an independent library routine (torch's scaled_dot_product_attention,
scipy's logsumexp) or the index example of Fig. 4 of "Near-Oracle KV Selection
via Pre-hoc Sparsity for Long-Context Inference". The mutation tests at the end
plant plausible mistakes in copies of the oracle functions and show that some
pin fails for each.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import prhs_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# Scores
# ---------------------------------------------------------------------------

def check_scores_unit_query(scores_fn):
    """q = sqrt(d) e_c makes q.k/sqrt(d) equal to column c of that head's K.

    Distinct K per KV head and G = 4 also pin the grouped-head mapping h -> h // G.
    """
    B, Hq, Hkv, t, d = 2, 8, 2, 37, 16
    K = _rand((B, Hkv, t, d), 1)
    G = Hq // Hkv
    q = np.zeros((B, Hq, d))
    cols = {}
    for b in range(B):
        for h in range(Hq):
            c = (3 * h + 5 * b) % d
            cols[(b, h)] = c
            q[b, h, c] = math.sqrt(d)
    s = scores_fn(q, K)
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(s[b, h], K[b, h // G, :, cols[(b, h)]], rtol=0, atol=1e-12)


def check_dense_matches_sdpa(scores_fn, attn_fn):
    """With S = all keys, the sparse output is dense attention (torch SDPA, fp64)."""
    B, Hq, Hkv, t, d = 2, 8, 2, 29, 16
    q = _rand((B, Hq, d), 2)
    K = _rand((B, Hkv, t, d), 3)
    V = _rand((B, Hkv, t, d), 4)
    s = scores_fn(q, K)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[:, :, None, :], torch.tensor(K), torch.tensor(V), enable_gqa=True)[:, :, 0, :].numpy()
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            o, lse = attn_fn(s[b, h], V[b, h // G], np.arange(t))
            np.testing.assert_allclose(o, ref[b, h], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, scipy.special.logsumexp(s[b, h]), rtol=0, atol=1e-12)


def test_scores_unit_query():
    check_scores_unit_query(O.attention_scores)


def test_dense_output_matches_sdpa():
    check_dense_matches_sdpa(O.attention_scores, O.sparse_attention)


# ---------------------------------------------------------------------------
# Softmax
# ---------------------------------------------------------------------------

def test_softmax_sums_to_one_shift_invariant_and_lse():
    s = _rand((3, 5, 101), 5, 4.0)
    A, lse = O.dense_softmax(s)
    assert np.max(np.abs(A.sum(-1) - 1.0)) <= 1e-12
    A2, lse2 = O.dense_softmax(s + 17.25)
    np.testing.assert_allclose(A2, A, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse2, lse + 17.25, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Top-N oracle
# ---------------------------------------------------------------------------

def check_topn_brute_force(topn_fn):
    """Top-N minimises delta over every size-N subset; unique sets match."""
    for t in (1, 2, 5, 9, 12):
        s = _rand(t, 100 + t, 2.0)
        A, _ = O.dense_softmax(s)
        for N in range(1, t + 1):
            best, best_set = None, None
            for sub in itertools.combinations(range(t), N):
                d = 1.0 - A[list(sub)].sum()
                if best is None or d < best - 1e-15:
                    best, best_set = d, sub
            S = topn_fn(s, N)
            assert S.size == N
            d_top = A[np.setdiff1d(np.arange(t), S)].sum()
            assert abs(d_top - best) <= 1e-12
            assert tuple(S) == tuple(sorted(best_set))


def check_topn_ties(topn_fn):
    """Ties go to the lower index; all-equal scores give delta = 1 - N/t exactly."""
    s = np.array([1.0, 3.0, 2.0, 3.0, 3.0, -1.0])
    assert list(topn_fn(s, 1)) == [1]
    assert list(topn_fn(s, 2)) == [1, 3]
    assert list(topn_fn(s, 3)) == [1, 3, 4]
    assert list(topn_fn(s, 4)) == [1, 2, 3, 4]
    t = 16
    flat = np.full(t, 0.75)
    for N in range(1, t + 1):
        S = topn_fn(flat, N)
        assert list(S) == list(range(N))
        d, tau = O.dropped_mass(flat, S)
        assert abs(d - (1 - N / t)) <= 1e-15


def test_topn_brute_force():
    check_topn_brute_force(O.topn_select)


def test_topn_ties():
    check_topn_ties(O.topn_select)


def test_topn_rejects_bad_budget():
    with pytest.raises(ValueError):
        O.topn_select(np.zeros(4), 0)
    with pytest.raises(ValueError):
        O.topn_select(np.zeros(4), 5)


# ---------------------------------------------------------------------------
# Dropped mass, sparse output identities
# ---------------------------------------------------------------------------

def check_delta_properties(delta_fn):
    rng = np.random.default_rng(7)
    t = 200
    s = rng.standard_normal(t) * 2.0
    prev = 2.0
    for N in range(1, t + 1):
        d, tau = delta_fn(s, O.topn_select(s, N))
        assert d <= prev + 1e-15          # non-increasing in N
        assert abs(d + tau - 1.0) <= 1e-15
        prev = d
        if N % 37 == 0:
            for _ in range(5):             # top-N beats random subsets of equal size
                R = rng.choice(t, N, replace=False)
                assert d <= delta_fn(s, R)[0] + 1e-15
    assert delta_fn(s, np.arange(t))[0] == 0.0


def test_delta_properties():
    check_delta_properties(O.dropped_mass)


def check_tau_vs_lse(attn_fn, delta_fn):
    """tau(S) = exp(lse_S - lse_all): ties the sparse lse to the dense normaliser."""
    s = _rand(300, 9, 3.0)
    V = _rand((300, 8), 10)
    lse_all = scipy.special.logsumexp(s)
    for N in (1, 7, 64, 299):
        S = O.topn_select(s, N)
        _, lse_S = attn_fn(s, V, S)
        d, tau = delta_fn(s, S)
        assert abs(tau - math.exp(lse_S - lse_all)) <= 1e-12


def test_tau_vs_lse():
    check_tau_vs_lse(O.sparse_attention, O.dropped_mass)


def check_decomposition_and_bound(attn_fn, delta_fn):
    """o_dense = tau o_S + delta o_{S^c} (o_dense from torch SDPA) and
    |o_dense - o_S|_inf <= delta * max_c (max_i v_ic - min_i v_ic)."""
    t, d = 257, 32
    q = _rand((1, 1, d), 11, 1.5)
    K = _rand((1, 1, t, d), 12)
    V = _rand((1, 1, t, d), 13)
    s = O.attention_scores(q, K)[0, 0]
    dense = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[:, :, None, :], torch.tensor(K), torch.tensor(V))[0, 0, 0].numpy()
    span = (V[0, 0].max(0) - V[0, 0].min(0)).max()
    for N in (1, 16, 100, 256):
        S = O.topn_select(s, N)
        Sc = np.setdiff1d(np.arange(t), S)
        oS, _ = attn_fn(s, V[0, 0], S)
        oC, _ = attn_fn(s, V[0, 0], Sc)
        delta, tau = delta_fn(s, S)
        np.testing.assert_allclose(tau * oS + delta * oC, dense, rtol=0, atol=1e-12)
        assert np.max(np.abs(dense - oS)) <= delta * span + 1e-12


def test_decomposition_and_bound():
    check_decomposition_and_bound(O.sparse_attention, O.dropped_mass)


# ---------------------------------------------------------------------------
# Delta-budget selection
# ---------------------------------------------------------------------------

def check_delta_budget(budget_fn):
    rng = np.random.default_rng(21)
    for trial in range(40):
        t = int(rng.integers(1, 300))
        s = rng.standard_normal(t) * rng.uniform(0.5, 6.0)
        lse = scipy.special.logsumexp(s)
        A = np.exp(s - lse)
        cap = int(rng.integers(1, t + 1))
        prev_n = None
        for ds in (0.5, 0.2, 0.05, 0.01, 0.0):
            S, n, cap_hit = budget_fn(s, lse, cap, ds)
            assert S.size == n and 1 <= n <= cap
            assert list(S) == list(O.topn_select(s, n))
            drop = lambda k: 1.0 - A[O.topn_select(s, k)].sum() if k < t else 0.0
            if not cap_hit:
                assert drop(n) <= ds + 1e-12
                if n > 1:
                    assert drop(n - 1) > ds - 1e-12
            else:
                assert n == cap and drop(cap) > ds - 1e-12
            if prev_n is not None:
                assert n >= prev_n            # non-increasing in delta*
            prev_n = n


def check_delta_budget_brute_force(budget_fn):
    """N* is the size of the smallest subset of any kind whose dropped mass is <= delta*."""
    for t in (3, 6, 10):
        s = _rand(t, 300 + t, 2.5)
        lse = scipy.special.logsumexp(s)
        A = np.exp(s - lse)
        for ds in (0.3, 0.1, 0.02):
            need = None
            for n in range(1, t + 1):
                if any(1.0 - A[list(c)].sum() <= ds for c in itertools.combinations(range(t), n)):
                    need = n
                    break
            _, n, cap_hit = budget_fn(s, lse, t, ds)
            assert not cap_hit and n == need


def test_delta_budget():
    check_delta_budget(O.delta_budget_select)


def test_delta_budget_brute_force():
    check_delta_budget_brute_force(O.delta_budget_select)


# ---------------------------------------------------------------------------
# CIS dilation and schedule
# ---------------------------------------------------------------------------

def _runs_to_set(runs):
    return [i for a, b in runs for i in range(a, b + 1)]


def check_cis_fig4(dilate_fn):
    g = json.load(open(os.path.join(GOLDEN, "cis_fig4.json")))
    anchor = _runs_to_set(g["anchor"])
    for case in g["cases"]:
        D = dilate_fn(anchor, case["r"], g["t"])
        assert list(D) == _runs_to_set(case["expect_runs"])
        assert len(D) == case["size"]


def check_cis_properties(dilate_fn):
    rng = np.random.default_rng(31)
    for trial in range(60):
        t = int(rng.integers(1, 200))
        n = int(rng.integers(1, t + 1))
        S = np.sort(rng.choice(t, n, replace=False))
        r = int(rng.integers(0, 6)) if trial % 7 else int(rng.integers(0, 400))
        D = dilate_fn(S, r, t)
        assert np.all(np.diff(D) > 0) and (D.size == 0 or (D[0] >= 0 and D[-1] < t))
        assert np.isin(S, D).all()
        assert D.size <= min(t, (2 * r + 1) * n)
        # brute-force membership by distance to the nearest anchor index
        pos = np.searchsorted(S, np.arange(t))
        left = np.abs(np.arange(t) - S[np.clip(pos - 1, 0, n - 1)])
        right = np.abs(S[np.clip(pos, 0, n - 1)] - np.arange(t))
        member = np.minimum(left, right) <= r
        assert list(D) == list(np.flatnonzero(member))
        if r == 0:
            assert list(D) == list(S)
    # single run
    D = dilate_fn(np.arange(40, 51), 3, 60)
    assert list(D) == list(range(37, 54))


def check_random_expansion(expand_fn):
    """Random expansion: against a sequential argmin draw (a different procedure),
    an optimality certificate, and the special cases."""
    rng = np.random.default_rng(41)
    for trial in range(50):
        t = int(rng.integers(1, 120))
        n = int(rng.integers(1, t + 1))
        S = np.sort(rng.choice(t, n, replace=False))
        m = int(rng.integers(n, t + 1))
        hi = 1 << 23 if trial % 3 else 8            # some trials with many equal draws
        draws = rng.integers(0, hi, t) | (rng.integers(0, 2, t) << 30)   # bits above 23 are ignored
        E = expand_fn(S, draws, m)
        # sequential draw: repeatedly take the outsider with the smallest
        # 23-bit draw, the lowest index among equal ones
        low = [int(x) & 0x7FFFFF for x in draws]
        taken = set(int(i) for i in S)
        while len(taken) < m:
            best = min((i for i in range(t) if i not in taken), key=lambda i: (low[i], i))
            taken.add(best)
        assert list(E) == sorted(taken)
        assert np.all(np.diff(E) > 0) and np.isin(S, E).all() and E.size == m
        chosen = np.setdiff1d(E, S)
        rest = np.setdiff1d(np.arange(t), E)
        if chosen.size and rest.size:
            worst = max((low[i], i) for i in chosen)
            assert all((low[j], j) > worst for j in rest)
    S = np.array([3, 9, 10])
    assert list(expand_fn(S, np.arange(20), 3)) == [3, 9, 10]
    assert list(expand_fn(S, np.arange(20)[::-1], 20)) == list(range(20))
    assert list(expand_fn(S, np.zeros(20, dtype=np.int64), 6)) == [0, 1, 2, 3, 9, 10]


def test_random_expansion_pins():
    check_random_expansion(O.random_expansion)


def test_cis_fig4_golden():
    check_cis_fig4(O.cis_dilate)


def test_cis_properties():
    check_cis_properties(O.cis_dilate)


def test_cis_schedule_period_and_not_chained():
    sched = O.cis_schedule(10, 4)
    assert [a for a, _ in sched] == [True, False, False, False, True, False, False, False, True, False]
    assert [s for _, s in sched] == [0, 0, 0, 0, 4, 4, 4, 4, 8, 8]


def test_cis_schedule_gate():
    d = 8
    q = np.zeros((6, d))
    q[:, 0] = 1.0
    q[3, 1] = 5.0           # step 3 turns away from the anchor query
    sched = O.cis_schedule(6, 100, q, sim_tau=0.8)
    assert [a for a, _ in sched] == [True, False, False, True, True, False]
    assert [s for _, s in sched] == [0, 0, 0, 3, 4, 4]
    sched = O.cis_schedule(6, 100, q, sim_tau=None)
    assert [a for a, _ in sched] == [True] + [False] * 5


def test_beta_emp():
    rng = np.random.default_rng(41)
    s = rng.standard_normal(120) * 2
    for N in (1, 10, 60):
        assert abs(O.beta_emp(s, O.topn_select(s, N))) <= 1e-15
        R = rng.choice(120, N, replace=False)
        assert O.beta_emp(s, R) >= -1e-15
    S = O.topn_select(s, 10)
    assert O.overlap_with_oracle(O.cis_dilate(S, 2, 120), S) == 1.0


def test_decode_step_consistency():
    """decode_step composes the pinned pieces (GQA, all three modes)."""
    B, Hq, Hkv, t, d = 1, 4, 2, 64, 16
    q = _rand((B, Hq, d), 51)
    K = _rand((B, Hkv, t, d), 52)
    V = _rand((B, Hkv, t, d), 53)
    r = O.decode_step(q, K, V, "topn", N=8)
    s = O.attention_scores(q, K)
    for (b, h), v in r.items():
        assert list(v["idx"]) == list(O.topn_select(s[b, h], 8))
        o, lse = O.sparse_attention(s[b, h], V[b, h // 2], v["idx"])
        np.testing.assert_allclose(v["out"], o, atol=1e-15)
    r = O.decode_step(q, K, V, "delta", N=t, delta_star=0.1)
    for v in r.values():
        assert v["delta"] <= 0.1 + 1e-12
    sets = {(0, h): np.arange(h, t, 3) for h in range(Hq)}
    r = O.decode_step(q, K, V, "given", sets=sets)
    assert all(list(v["idx"]) == list(sets[k]) for k, v in r.items())


# ---------------------------------------------------------------------------
# Planted mistakes: every one must trip a pin above.
# ---------------------------------------------------------------------------

def _scores_wrong_scale(q, K):
    return O.attention_scores(q, K) * math.sqrt(q.shape[-1]) / q.shape[-1]


def _scores_wrong_group(q, K):
    q = np.asarray(q, float)
    K = np.asarray(K, float)
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    return np.stack([np.stack([K[b, h % Hkv] @ q[b, h] / math.sqrt(d) for h in range(Hq)]) for b in range(B)])


def _topn_high_index_ties(s, N):
    s = np.asarray(s, float)
    order = np.lexsort((-np.arange(len(s)), -s))
    return np.sort(order[:N])


def _topn_off_by_one(s, N):
    return O.topn_select(s, max(1, N - 1)) if N > 1 else O.topn_select(s, N)


def _attn_unnormalised_max(s, V, S):
    o, lse = O.sparse_attention(s, V, S)
    S = np.asarray(S)
    return o * np.exp(np.asarray(s)[S]).sum() / np.exp(np.asarray(s)[S] - np.max(np.asarray(s)[S])).sum(), lse


def _delta_budget_strict(s, lse, cap, ds):
    S, n, hit = O.delta_budget_select(s, lse, cap, ds)
    if n < cap:
        n += 1
    return O.topn_select(s, n), n, hit


def _dilate_shrunk(S, r, t):
    return O.cis_dilate(S, max(0, r - 1), t)


def _dilate_unclipped_left(S, r, t):
    D = O.cis_dilate(S, r, t)
    return D[D >= r] if r > 0 else D


def _expand_high_index_ties(S, draws, m):
    d = np.asarray(draws, dtype=np.int64) & 0x7FFFFF
    t = d.size
    out = np.setdiff1d(np.arange(t), S)
    order = np.lexsort((-out, d[out]))
    return np.sort(np.concatenate([S, out[order[:m - len(S)]]]))


def _expand_unmasked(S, draws, m):
    d = np.asarray(draws, dtype=np.int64)
    out = np.setdiff1d(np.arange(d.size), S)
    order = np.lexsort((out, d[out]))
    return np.sort(np.concatenate([S, out[order[:m - len(S)]]]))


def _expand_ignoring_members(S, draws, m):
    d = np.asarray(draws, dtype=np.int64) & 0x7FFFFF
    order = np.lexsort((np.arange(d.size), d))
    return np.union1d(S, order[:m - len(S)])


def _delta_via_kept_count(s, S):
    d, tau = O.dropped_mass(s, S)
    t = len(s)
    return 1.0 - len(S) / t, len(S) / t


def _delta_swapped(s, S):
    d, tau = O.dropped_mass(s, S)
    return tau, d


@pytest.mark.parametrize("check,args", [
    (check_scores_unit_query, (_scores_wrong_scale,)),
    (check_scores_unit_query, (_scores_wrong_group,)),
    (check_dense_matches_sdpa, (_scores_wrong_scale, O.sparse_attention)),
    (check_dense_matches_sdpa, (O.attention_scores, _attn_unnormalised_max)),
    (check_topn_ties, (_topn_high_index_ties,)),
    (check_topn_brute_force, (_topn_off_by_one,)),
    (check_delta_budget, (_delta_budget_strict,)),
    (check_delta_budget_brute_force, (_delta_budget_strict,)),
    (check_cis_fig4, (_dilate_shrunk,)),
    (check_cis_properties, (_dilate_unclipped_left,)),
    (check_tau_vs_lse, (O.sparse_attention, _delta_via_kept_count)),
    (check_delta_properties, (_delta_swapped,)),
    (check_decomposition_and_bound, (O.sparse_attention, _delta_via_kept_count)),
    (check_random_expansion, (_expand_high_index_ties,)),
    (check_random_expansion, (_expand_unmasked,)),
    (check_random_expansion, (_expand_ignoring_members,)),
])
def test_planted_mistake_is_caught(check, args):
    with pytest.raises((AssertionError, ValueError, IndexError)):
        check(*args)
