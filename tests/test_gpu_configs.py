"""End-to-end parity of the decode hot path on the configured workloads.

Every workload runs at its full configured size in the launch configuration
the benchmark uses (DecodeEngine.anchor_step / reuse_step); the oracle checks
a sample of heads and steps (each oracle head costs one fp64 pass over its
KV head). Inputs are the seeded synthetic workloads; expected values come only
from the oracle.
"""

import numpy as np
import pytest
import torch

from oracle import prhs_oracle as O
from sparse_top_kv_head_amd import prhs as P
from sparse_top_kv_head_amd.engine import AdaptiveEngine, DecodeEngine
from sparse_top_kv_head_amd.synth import CONFIGS, layer_draws, make_workload
from tests.parity_util import (DELTA_TOL, OUT_TOL, check_delta_choice, check_set_band,
                               reorder_tols)

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()
    return torch.device("cuda:0")


def _np(x):
    return x.detach().double().cpu().numpy()


def _sample_heads(cfg, n, seed):
    rng = np.random.default_rng(seed)
    allh = [(b, h) for b in range(cfg.batch) for h in range(cfg.n_q_heads)]
    pick = rng.choice(len(allh), size=min(n, len(allh)), replace=False)
    return sorted(allh[i] for i in pick)


class _KVCache:
    """fp64 host copies of the KV heads the oracle needs, fetched on demand."""

    def __init__(self, w):
        self.w = w
        self.k = {}
        self.v = {}

    def kv(self, b, g):
        if (b, g) not in self.k:
            self.k[(b, g)] = _np(self.w.K[b, g])
            self.v[(b, g)] = _np(self.w.V[b, g])
        return self.k[(b, g)], self.v[(b, g)]


def _oracle_scores(cache, q64, b, h, G):
    K, V = cache.kv(b, h // G)
    s = O.attention_scores(q64[b:b + 1, h:h + 1], K[None, None])[0, 0]
    return s, V


def _check_topn_heads(eng, w, cfg, step, heads, cache):
    q64 = _np(w.q[step])
    G = cfg.group
    exact_heads = 0
    for (b, h) in heads:
        s, V = _oracle_scores(cache, q64, b, h, G)
        n = int(eng.count[b, h])
        gidx = eng.idx[b, h, :n].cpu().numpy()
        exact = check_set_band(gidx, s, cfg.budget)
        exact_heads += exact
        S_ref = O.topn_select(s, cfg.budget) if exact else gidx
        o_ref, lse_ref = O.sparse_attention(s, V, S_ref)
        d_ref, _ = O.dropped_mass(s, S_ref)
        assert np.max(np.abs(_np(eng.out[b, h]) - o_ref)) <= OUT_TOL
        assert abs(eng.delta[b, h].item() - d_ref) <= DELTA_TOL
        assert abs(eng.tau[b, h].item() - (1 - d_ref)) <= DELTA_TOL
        _, lse_all = O.dense_softmax(s)
        assert abs(eng.lse_all[b, h].item() - lse_all) <= 1e-3
    return exact_heads


def test_llama2_4k_full():
    """LLaMA2-7B-shaped layer: every head of three of the 64 steps."""
    dev = _dev()
    cfg = CONFIGS["llama2_4k"]
    w = make_workload(cfg, device=dev)
    eng = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    cache = _KVCache(w)
    heads = [(0, h) for h in range(cfg.n_q_heads)]
    for step in (0, 31, cfg.steps - 1):
        eng.topn_step(w.q[step], w.K, w.V, cfg.budget)
        torch.cuda.synchronize()
        assert _check_topn_heads(eng, w, cfg, step, heads, cache) >= len(heads) - 2


@pytest.mark.parametrize("name", ["mistral_gqa_32k", "gqa16_32k", "mistral_gqa_128k"])
def test_mistral_gqa_32k_sampled(name):
    """GQA layers at 32K (Mistral-7B-shaped, 4 query heads per KV head; and 16
    per KV head, one scan launch per group) and at 128K (selection streams the
    rows past 64K keys): 16 sampled heads at three steps, plus run-to-run
    determinism of every head's indices and outputs."""
    dev = _dev()
    cfg = CONFIGS[name]
    w = make_workload(cfg, device=dev)
    eng = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    cache = _KVCache(w)
    for step in (0, 13, cfg.steps - 1):
        eng.topn_step(w.q[step], w.K, w.V, cfg.budget)
        torch.cuda.synchronize()
        heads = _sample_heads(cfg, 16, step)
        assert _check_topn_heads(eng, w, cfg, step, heads, cache) >= len(heads) - 2
        assert torch.all(eng.count == cfg.budget)
    first = (eng.idx.clone(), eng.count.clone(), eng.out.clone(), eng.delta.clone())
    eng.topn_step(w.q[cfg.steps - 1], w.K, w.V, cfg.budget)
    torch.cuda.synchronize()
    for a, b in zip(first, (eng.idx, eng.count, eng.out, eng.delta)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["mistral_gqa_32k", "llama2_4k"])
def test_fused_decode_matches_decode_kernel(name):
    """At full size, the attention the selection kernel computes for its own
    head (the anchor step) and the one prhs_sparse_decode computes over the
    same selection from the same score rows differ only by the order of their
    fp32 sums: outputs within (4(n - 1) + 8) u max|v|, lse_sel, delta and tau
    within (2(n - 1) + 8) u."""
    dev = _dev()
    cfg = CONFIGS[name]
    w = make_workload(cfg, device=dev)
    a = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    b = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    q = w.q[cfg.steps // 2]
    a.anchor_step(q, w.K, w.V, P.PRHS_TOPN, cfg.budget, hint=False)   # every score row written
    P.prhs_sparse_decode(a.dims, q, w.K, w.V, a.idx, a.cap, a.count, a.scores, a.lse_all, b.out,
                         b.lse_sel, b.delta, b.tau, b.ws)
    torch.cuda.synchronize()
    otol, ltol = reorder_tols(cfg.budget, w.V.abs().max().item())
    assert (a.out - b.out).abs().max().item() <= otol
    for n in ("lse_sel", "delta", "tau"):
        assert (getattr(a, n) - getattr(b, n)).abs().max().item() <= ltol, n


@pytest.mark.parametrize("name", ["llama2_cis_8k", "llama2_cis_8k_sharp"])
def test_llama2_cis_8k_schedule(name):
    """CIS reuse at full size: exact retrieval every 4th step, +-2 dilation of the
    anchor's set otherwise (not chained), attention over the reused set with
    gathered K and V rows; delta of the reused set against the oracle. Also at
    query scale 3, where the exact top-512 keeps most of the mass."""
    dev = _dev()
    cfg = CONFIGS[name]
    w = make_workload(cfg, device=dev)
    r = cfg.radius
    dil_cap = min(cfg.ctx_len, (2 * r + 1) * cfg.budget)
    anchor = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    reuse = DecodeEngine(w.K, cfg.n_q_heads, dil_cap)
    cache = _KVCache(w)
    heads = _sample_heads(cfg, 12, 3)
    sched = O.cis_schedule(8, cfg.refresh_period)
    anchor_sets = {}
    for step, (is_anchor, a_step) in enumerate(sched):
        q64 = _np(w.q[step])
        if is_anchor:
            anchor.topn_step(w.q[step], w.K, w.V, cfg.budget)
            torch.cuda.synchronize()
            _check_topn_heads(anchor, w, cfg, step, heads, cache)
            anchor_sets = {bh: anchor.idx[bh[0], bh[1], :int(anchor.count[bh])].cpu().numpy() for bh in heads}
            a_idx, a_cnt = anchor.idx.clone(), anchor.count.clone()
            continue
        reuse.reuse_step(w.q[step], w.K, w.V, a_idx, a_cnt, cfg.budget, r)
        # diagnostic pass: dense lse of this step for the reused set's delta
        reuse.score(w.q[step], w.K)
        reuse.dropped_mass()
        torch.cuda.synchronize()
        for (b, h) in heads:
            s, V = _oracle_scores(cache, q64, b, h, cfg.group)
            D_ref = O.cis_dilate(anchor_sets[(b, h)], r, cfg.ctx_len)
            n = int(reuse.count[b, h])
            assert np.array_equal(reuse.idx[b, h, :n].cpu().numpy(), D_ref)
            o_ref, lse_ref = O.sparse_attention(s, V, D_ref)
            d_ref, _ = O.dropped_mass(s, D_ref)
            assert np.max(np.abs(_np(reuse.out[b, h]) - o_ref)) <= OUT_TOL
            assert abs(reuse.lse_sel[b, h].item() - lse_ref) <= 1e-3
            assert abs(reuse.delta[b, h].item() - d_ref) <= DELTA_TOL
            # the reused set keeps at most the oracle's mass at its own size
            assert O.beta_emp(s, D_ref) >= -1e-12


def _delta_layer(cfg, which):
    """The layer of lowest, median or highest drawn cluster bias (sharp
    variant: of lowest, median or highest drawn query scale) among the 32."""
    draws = [layer_draws(cfg, l) for l in range(cfg.n_layers)]
    key = (lambda l: draws[l][0]) if cfg.q_scale[0] != cfg.q_scale[1] else (lambda l: draws[l][1])
    order = sorted(range(cfg.n_layers), key=key)
    return order[{"low": 0, "mid": cfg.n_layers // 2, "high": -1}[which]]


@pytest.mark.parametrize("which", ["low", "mid", "high"])
@pytest.mark.parametrize("variant", ["literal", "sharp"])
def test_delta_16k_layer_sampled(variant, which):
    """Delta-budgeted layers at full size (each of the 32 layers is an
    independent KV cache with its own drawn cluster count and bias in
    [0.5, 2]): smallest N with delta <= 0.05, capped at 2048, on the layers of
    lowest, median and highest bias. The "sharp" variant draws a per-layer
    query scale in [1, 4] so that N* varies; there the layers are picked by
    that scale."""
    dev = _dev()
    cfg = CONFIGS["delta_16k"]
    if variant == "sharp":
        cfg = cfg.replace(q_scale=(1.0, 4.0))
    layer = _delta_layer(cfg, which)
    print(f"delta_16k {variant} layer {layer} draws {layer_draws(cfg, layer)}", flush=True)
    w = make_workload(cfg, device=dev, layer=layer)
    eng = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    cache = _KVCache(w)
    for step in (0, cfg.steps - 1):
        eng.delta_step(w.q[step], w.K, w.V, cfg.budget, cfg.delta_star)
        torch.cuda.synchronize()
        q64 = _np(w.q[step])
        for (b, h) in _sample_heads(cfg, 12, 100 * layer + step):
            s, V = _oracle_scores(cache, q64, b, h, cfg.group)
            _, lse = O.dense_softmax(s)
            n = int(eng.count[b, h])
            gidx = eng.idx[b, h, :n].cpu().numpy()
            exact = check_delta_choice(gidx, n, s, float(lse), cfg.budget, cfg.delta_star,
                                       cap_hit=int(eng.cap_hit[b, h]))
            S_ref = O.topn_select(s, n) if exact else gidx
            o_ref, _ = O.sparse_attention(s, V, S_ref)
            d_ref, _ = O.dropped_mass(s, S_ref)
            assert np.max(np.abs(_np(eng.out[b, h]) - o_ref)) <= OUT_TOL
            assert abs(eng.delta[b, h].item() - d_ref) <= DELTA_TOL
            if not int(eng.cap_hit[b, h]):
                assert eng.delta[b, h].item() <= cfg.delta_star + DELTA_TOL


def test_growing_cache_cis_schedule():
    """Growing cache (t = t0 + step: one more key visible each step) with the
    CIS schedule of the LLaMA2 reuse workload: exact top-N at anchor steps (the
    threshold hint carried across the growth) and the anchor's set dilated and
    clipped to the current t at reuse steps. Each step first appends its key
    and value rows (prhs_append_kv) to a cache whose rows from t0 - 1 on start
    zeroed. Sets, outputs and delta against the oracle on the first t keys of
    every step."""
    dev = _dev()
    t0, steps = 3000, 10
    cfg = CONFIGS["llama2_cis_8k"].replace(batch=1, ctx_len=t0 + steps, steps=steps)
    w = make_workload(cfg, device=dev)
    N, r, Pd = cfg.budget, cfg.radius, cfg.refresh_period
    Kc, Vc = w.K.clone(), w.V.clone()
    Kc[:, :, t0 - 1:] = 0
    Vc[:, :, t0 - 1:] = 0
    anchor = DecodeEngine(Kc, cfg.n_q_heads, N)
    reuse = DecodeEngine(Kc, cfg.n_q_heads, min(cfg.ctx_len, (2 * r + 1) * N))
    cache = _KVCache(w)
    heads = _sample_heads(cfg, 8, 5)
    anchor_sets = {}
    for step in range(steps):
        t = t0 + step
        anchor.set_ctx_len(t)
        reuse.set_ctx_len(t)
        anchor.append_kv(w.K[:, :, t - 1].contiguous(), w.V[:, :, t - 1].contiguous(), Kc, Vc, t - 1)
        q64 = _np(w.q[step])
        if step % Pd == 0:
            anchor.topn_step(w.q[step], Kc, Vc, N)
            torch.cuda.synchronize()
            for (b, h) in heads:
                s_full, V = _oracle_scores(cache, q64, b, h, cfg.group)
                s, V = s_full[:t], V[:t]
                n = int(anchor.count[b, h])
                gidx = anchor.idx[b, h, :n].cpu().numpy()
                assert n == N and gidx.max() < t
                exact = check_set_band(gidx, s, N)
                S_ref = O.topn_select(s, N) if exact else gidx
                o_ref, _ = O.sparse_attention(s, V, S_ref)
                d_ref, _ = O.dropped_mass(s, S_ref)
                assert np.max(np.abs(_np(anchor.out[b, h]) - o_ref)) <= OUT_TOL
                assert abs(anchor.delta[b, h].item() - d_ref) <= DELTA_TOL
                anchor_sets[(b, h)] = gidx
            continue
        reuse.reuse_step(w.q[step], Kc, Vc, anchor.idx, anchor.count, N, r)
        reuse.score(w.q[step], Kc)
        reuse.dropped_mass()
        torch.cuda.synchronize()
        for (b, h) in heads:
            s_full, V = _oracle_scores(cache, q64, b, h, cfg.group)
            s, V = s_full[:t], V[:t]
            D_ref = O.cis_dilate(anchor_sets[(b, h)], r, t)
            n = int(reuse.count[b, h])
            assert np.array_equal(reuse.idx[b, h, :n].cpu().numpy(), D_ref)
            o_ref, lse_ref = O.sparse_attention(s, V, D_ref)
            d_ref, _ = O.dropped_mass(s, D_ref)
            assert np.max(np.abs(_np(reuse.out[b, h]) - o_ref)) <= OUT_TOL
            assert abs(reuse.lse_sel[b, h].item() - lse_ref) <= 1e-3
            assert abs(reuse.delta[b, h].item() - d_ref) <= DELTA_TOL


@pytest.mark.parametrize("period,sim_tau", [(4, 0.7), (8, 0.97), (16, 0.95), (4, 0.99)])
def test_adaptive_cis_gate(period, sim_tau):
    """Per-head gated CIS (one exact retrieval per `period` steps, and in between
    whenever the cosine of a head's query with its anchor query falls below
    sim_tau) on the LLaMA2 reuse workload's head shape. Every gate decision is
    checked against the fp64 cosine wherever that cosine is more than 1e-4 from
    the threshold; refreshed heads' exact sets, reused heads' dilated sets,
    outputs and delta against the oracle on sampled heads."""
    dev = _dev()
    cfg = CONFIGS["llama2_cis_8k"].replace(batch=1, steps=12)
    w = make_workload(cfg, device=dev)
    N, r, t, H = cfg.budget, cfg.radius, cfg.ctx_len, cfg.n_q_heads
    eng = AdaptiveEngine(w.K, H, N, r, period, sim_tau)
    cache = _KVCache(w)
    heads = _sample_heads(cfg, 8, 11)
    anchor_q, anchor_set = {}, {}
    refreshes = 0
    for step in range(cfg.steps):
        eng.step(w.q[step], w.K, w.V)
        torch.cuda.synchronize()
        q64 = _np(w.q[step])
        ref = eng.refresh.cpu().numpy()
        sim = eng.sim.cpu().numpy()
        refreshes += int(ref.sum())
        for h in range(H):
            force = step % period == 0
            if h in anchor_q:
                a, x = anchor_q[h], q64[0, h]
                cos = float(a @ x) / (np.linalg.norm(a) * np.linalg.norm(x))
                assert abs(sim[0, h] - cos) <= 1e-5
                if not force and abs(cos - sim_tau) > 1e-4:
                    assert ref[0, h] == int(cos < sim_tau), (step, h, cos)
            else:
                assert ref[0, h] == 1
            if force:
                assert ref[0, h] == 1
            if ref[0, h]:
                anchor_q[h] = q64[0, h].copy()
        for (b, h) in heads:
            s, V = _oracle_scores(cache, q64, b, h, cfg.group)
            if ref[b, h]:
                n = int(eng.anchor_count[b, h])
                gidx = eng.anchor_idx[b, h, :n].cpu().numpy()
                assert n == N
                exact = check_set_band(gidx, s, N)
                S = O.topn_select(s, N) if exact else gidx
                anchor_set[(b, h)] = gidx
                d_ref, _ = O.dropped_mass(s, S)
                assert abs(eng.delta[b, h].item() - d_ref) <= DELTA_TOL
            else:
                S = O.cis_dilate(anchor_set[(b, h)], r, t)
                n = int(eng.dil_count[b, h])
                assert np.array_equal(eng.dil_idx[b, h, :n].cpu().numpy(), S)
            o_ref, lse_ref = O.sparse_attention(s, V, S)
            assert np.max(np.abs(_np(eng.out[b, h]) - o_ref)) <= OUT_TOL
            assert abs(eng.lse_sel[b, h].item() - lse_ref) <= 1e-3
    # forced refreshes on steps 0, period, ...; the gate adds some in between.
    # Adjacent queries of this walk have cosine ~0.98, so a threshold of 0.99
    # refreshes every head at every step, one of 0.7 never fires in 4 steps.
    forced = H * len(range(0, cfg.steps, period))
    if sim_tau >= 0.99:
        assert refreshes == H * cfg.steps
    elif sim_tau <= 0.7:
        assert refreshes == forced
    else:
        assert forced < refreshes < H * cfg.steps
