"""Anchor steps with the carried threshold hint, at the shapes where the
selection also decodes its head (fp16 rows of 128, budgets up to 2048): the
scan hands the selection only the keys at or above each head's hint, and heads
whose hinted keys miss the answer take the full search.

The results must not depend on the hint: every case compares hinted steps
with unhinted ones bit for bit -- the selected sets, the dense log-sum-exp,
the attention outputs and masses -- over consecutive steps, with hints forced
to miss both ways and mixed across heads, and under graph replay; sampled
heads are checked against the fp64 oracle. Inputs are seeded synthetic
layers; expected values come only from the oracle.
"""


import numpy as np
import pytest
import torch

from oracle import prhs_oracle as O
from sparse_top_kv_head_amd import prhs as P
from sparse_top_kv_head_amd.engine import DecodeEngine
from sparse_top_kv_head_amd.synth import CONFIGS, make_workload
from tests.parity_util import DELTA_TOL, OUT_TOL, check_set_band

pytestmark = pytest.mark.gpu

NAMES = ("count", "lse_all", "out", "lse_sel", "delta", "tau")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()
    return torch.device("cuda:0")


def _np(x):
    return x.detach().double().cpu().numpy()


def _same(hinted, plain, tag):
    for n in NAMES:
        assert torch.equal(getattr(hinted, n), getattr(plain, n)), (tag, n)
    B, H = plain.count.shape
    for b in range(B):
        for h in range(H):
            c = int(plain.count[b, h])
            assert torch.equal(hinted.idx[b, h, :c], plain.idx[b, h, :c]), (tag, b, h)


def _oracle_heads(eng, w, q, heads, N):
    q64 = _np(q)
    G = eng.dims.n_q_heads // eng.dims.n_kv_heads
    for (b, h) in heads:
        K, V = _np(w.K[b, h // G]), _np(w.V[b, h // G])
        s = O.attention_scores(q64[b:b + 1, h:h + 1], K[None, None])[0, 0]
        gidx = eng.idx[b, h, :N].cpu().numpy()
        exact = check_set_band(gidx, s, N)
        S = O.topn_select(s, N) if exact else gidx
        o_ref, _ = O.sparse_attention(s, V, S)
        d_ref, _ = O.dropped_mass(s, S)
        assert np.max(np.abs(_np(eng.out[b, h]) - o_ref)) <= OUT_TOL, (b, h)
        assert abs(eng.delta[b, h].item() - d_ref) <= DELTA_TOL, (b, h)
        assert abs(eng.tau[b, h].item() - (1.0 - d_ref)) <= DELTA_TOL, (b, h)
        _, lse = O.dense_softmax(s)
        assert abs(eng.lse_all[b, h].item() - lse) <= 1e-3, (b, h)


HINT_CASES = [
    # B, Hq, Hkv, t, N, n_clusters
    (4, 32, 8, 32768, 2048, (256, 256)),   # the Mistral-7B-shaped GQA layer at 32K
    (1, 32, 32, 4096, 256, (32, 32)),      # LLaMA2-7B-shaped, one split per head
    (8, 32, 32, 8192, 512, (32, 32)),      # the CIS workload's anchor steps (two splits)
    (2, 64, 8, 5000, 700, (64, 64)),       # G = 8, ragged t, a short last split
    (1, 16, 8, 300, 100, (4, 4)),          # G = 2, two chunks, the last one partial
    (2, 48, 8, 3001, 192, (16, 16)),       # G = 6 (sub-groups of 4 and 2), ragged t
    (2, 32, 2, 8192, 512, (64, 64)),       # G = 16: one scan launch per KV head
    (1, 28, 4, 6000, 256, (32, 32)),       # G = 7 (Qwen2.5-7B grouping), ragged t
    (1, 128, 64, 65536, 256, (128, 128)),  # the largest context the registers hold
    (1, 8, 2, 131072, 2048, (512, 512)),   # 512 candidate chunks per head; streamed when unhinted
    (1, 4, 1, 262144, 1024, (256, 256)),   # the largest context the selection takes
]


@pytest.mark.parametrize("B,Hq,Hkv,t,N,ncl", HINT_CASES)
def test_hinted_steps_match_unhinted(B, Hq, Hkv, t, N, ncl):
    dev = _dev()
    cfg = CONFIGS["mistral_gqa_32k"].replace(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, ctx_len=t,
                                             budget=N, steps=4, n_clusters=ncl)
    w = make_workload(cfg, device=dev)
    hinted = DecodeEngine(w.K, Hq, N)
    plain = DecodeEngine(w.K, Hq, N)
    rng = np.random.default_rng(t)
    for step in range(cfg.steps):
        print(f"[hint] B={B} Hq={Hq} Hkv={Hkv} t={t} N={N} step={step}", flush=True)
        hinted.anchor_step(w.q[step], w.K, w.V, P.PRHS_TOPN, N)
        plain.anchor_step(w.q[step], w.K, w.V, P.PRHS_TOPN, N, hint=False)
        torch.cuda.synchronize()
        assert torch.isfinite(hinted.theta).all()
        _same(hinted, plain, step)
        if step == cfg.steps - 1:
            allh = [(b, h) for b in range(B) for h in range(Hq)]
            pick = rng.choice(len(allh), size=min(6, len(allh)), replace=False)
            _oracle_heads(hinted, w, w.q[step], [allh[i] for i in sorted(pick)], N)


def test_forced_misses_and_mixed_hints():
    """Hints that list no key (fewer than N candidates), that list every key
    (more than the selection's LDS list holds), and a mix of hinted and
    unhinted heads in one step: the missed heads go through the full
    selection and every output still equals the unhinted step's."""
    dev = _dev()
    cfg = CONFIGS["mistral_gqa_32k"].replace(batch=4, ctx_len=16384, budget=1024, steps=3,
                                             n_clusters=(128, 128))
    w = make_workload(cfg, device=dev)
    hinted = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    plain = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    q = w.q[1]
    plain.anchor_step(q, w.K, w.V, P.PRHS_TOPN, cfg.budget, hint=False)
    hinted.anchor_step(w.q[0], w.K, w.V, P.PRHS_TOPN, cfg.budget)
    torch.cuda.synchronize()
    good = hinted.theta.clone()
    mixed = good.clone()
    mixed[:, ::3] = float("nan")
    mixed[:, 1::5] = 1e30
    mixed[:, 2::7] = -1e30
    for tag, th in (("none listed", torch.full_like(good, 1e30)),
                    ("all listed", torch.full_like(good, -1e30)), ("mixed", mixed)):
        print(f"[hint] forced hints: {tag}", flush=True)
        hinted.theta.copy_(th)
        hinted.anchor_step(q, w.K, w.V, P.PRHS_TOPN, cfg.budget)
        torch.cuda.synchronize()
        assert torch.isfinite(hinted.theta).all()
        _same(hinted, plain, tag)


def test_hinted_step_graph_replay():
    """The 32K GQA step captured once replays, replay after replay, to the
    eager results, with eager work and synchronisations between replays."""
    dev = _dev()
    cfg = CONFIGS["mistral_gqa_32k"]
    w = make_workload(cfg, device=dev)
    eng = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    other = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    names = ("lse_all", "idx", "count", "out", "lse_sel", "delta", "tau")
    eng.anchor_step(w.q[2], w.K, w.V, P.PRHS_TOPN, cfg.budget)
    eng.anchor_step(w.q[2], w.K, w.V, P.PRHS_TOPN, cfg.budget)
    torch.cuda.synchronize()
    ref = {n: getattr(eng, n).clone() for n in names}
    g = eng.capture([(w.q[2], w.K, w.V)], P.PRHS_TOPN, cfg.budget)
    for r in range(4):
        print(f"[hint] replay {r}", flush=True)
        other.anchor_step(w.q[r], w.K, w.V, P.PRHS_TOPN, cfg.budget)
        for n in names:
            getattr(eng, n).fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(eng, n), ref[n]), (r, n)
