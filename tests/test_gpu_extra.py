"""More GPU parity: the fused anchor step over shapes (grouped heads in
sub-groups, ragged contexts, fp32 at d=64, DELTA), graph replay of the gated
CIS step and of the dense decode, determinism, and the gate's extremes."""

import numpy as np
import pytest
import torch

from oracle import prhs_oracle as O
from sparse_top_kv_head_amd import prhs as P
from sparse_top_kv_head_amd.engine import AdaptiveEngine, DecodeEngine
from sparse_top_kv_head_amd.synth import CONFIGS, make_workload
from tests.parity_util import (DELTA_TOL, OUT_TOL, check_delta_choice, check_set_band,
                               fused_anchor_decode, reorder_tols)

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()
    return torch.device("cuda:0")


def _np(x):
    return x.detach().double().cpu().numpy()


ANCHOR_CASES = [
    # B, Hq, Hkv, d, t, dtype, N, mode, delta*
    (2, 6, 2, 128, 1001, torch.float16, 100, P.PRHS_TOPN, 0.0),     # G = 3, ragged t
    (1, 4, 4, 64, 777, torch.float32, 50, P.PRHS_TOPN, 0.0),        # fp32, d = 64
    (1, 8, 1, 128, 5000, torch.float16, 4096, P.PRHS_TOPN, 0.0),    # G = 8, N close to t
    (2, 4, 2, 64, 3001, torch.float16, 600, P.PRHS_DELTA, 0.2),     # DELTA, d = 64
    (1, 2, 2, 128, 1, torch.float16, 1, P.PRHS_TOPN, 0.0),          # one key
    (1, 4, 4, 128, 300, torch.float16, 300, P.PRHS_TOPN, 0.0),      # N = t
    (1, 4, 1, 128, 9000, torch.float16, 700, P.PRHS_DELTA, 0.05),   # DELTA, scan candidates off
    (1, 16, 1, 128, 2500, torch.float16, 256, P.PRHS_TOPN, 0.0),    # G = 16: one scan launch
    (1, 24, 2, 128, 1800, torch.float16, 200, P.PRHS_DELTA, 0.1),   # G = 12: one launch, DELTA
]


@pytest.mark.parametrize("B,Hq,Hkv,d,t,dtype,N,mode,ds", ANCHOR_CASES)
def test_anchor_step_shapes(B, Hq, Hkv, d, t, dtype, N, mode, ds):
    """Two anchor steps (the second with the carried hint) against the oracle."""
    dev = _dev()
    g = torch.Generator().manual_seed(B * 1000 + t)
    K = torch.randn((B, Hkv, t, d), generator=g).to(dtype).to(dev)
    V = torch.randn((B, Hkv, t, d), generator=g).to(dtype).to(dev)
    K64, V64 = _np(K), _np(V)
    eng = DecodeEngine(K, Hq, N)
    G = Hq // Hkv
    for step in range(2):
        q = (torch.randn((B, Hq, d), generator=g) * 2.5).to(dtype).to(dev)
        eng.anchor_step(q, K, V, mode, N, ds)
        torch.cuda.synchronize()
        s_all = O.attention_scores(_np(q), K64)
        for b in range(B):
            for h in range(Hq):
                s = s_all[b, h]
                _, lse = O.dense_softmax(s)
                n = int(eng.count[b, h])
                gidx = eng.idx[b, h, :n].cpu().numpy()
                assert np.all(np.diff(gidx) > 0) and gidx.min() >= 0 and gidx.max() < t
                if mode == P.PRHS_TOPN:
                    assert n == N
                    exact = check_set_band(gidx, s, N)
                    S = O.topn_select(s, N) if exact else gidx
                else:
                    exact = check_delta_choice(gidx, n, s, float(lse), N, ds,
                                               cap_hit=int(eng.cap_hit[b, h]))
                    S = O.topn_select(s, n) if exact else gidx
                o_ref, _ = O.sparse_attention(s, V64[b, h // G], S)
                d_ref, _ = O.dropped_mass(s, S)
                assert np.max(np.abs(_np(eng.out[b, h]) - o_ref)) <= OUT_TOL, (step, b, h)
                assert abs(eng.delta[b, h].item() - d_ref) <= DELTA_TOL
                assert abs(eng.lse_all[b, h].item() - lse) <= 1e-3


FUSED_CASES = [
    # kind, B, Hq, Hkv, t, N: every case decodes inside the select kernel
    ("random", 2, 64, 8, 5003, 1000),    # 128 heads, ragged t
    ("random", 1, 128, 32, 2048, 2048),  # N = t: every key
    ("flat", 1, 128, 16, 10000, 2048),   # equal scores, t past the LDS list: streamed emission
    ("ties", 2, 64, 16, 3000, 700),      # few distinct scores: boundary ties
    ("random", 1, 8, 2, 2000, 256),      # one-split budget on few heads
    ("random", 1, 128, 32, 1500, 1),     # N = 1
    ("random", 1, 128, 16, 40000, 2048), # past 32K keys: the 64-keys-per-thread select
]


def _fused_inputs(kind, B, Hq, Hkv, t, g):
    d = 128
    if kind == "flat":
        K = torch.randn((B, Hkv, 1, d), generator=g).expand(B, Hkv, t, d).contiguous()
        q = torch.randn((B, Hq, d), generator=g)
    elif kind == "ties":
        K = torch.randint(-1, 2, (B, Hkv, t, d), generator=g).float()
        q = torch.randint(-1, 2, (B, Hq, d), generator=g).float()
    else:
        K = torch.randn((B, Hkv, t, d), generator=g)
        q = torch.randn((B, Hq, d), generator=g) * 2.5
    V = torch.randn((B, Hkv, t, d), generator=g) * 3.0
    return q.half(), K.half(), V.half()


@pytest.mark.parametrize("kind,B,Hq,Hkv,t,N", FUSED_CASES)
def test_fused_select_decode(kind, B, Hq, Hkv, t, N):
    """Anchor steps that decode inside the select kernel, through each emission
    (scan candidates with the carried hint, the sampled list, the streamed
    row), against the oracle: the exact top-N, the attention output and delta."""
    assert fused_anchor_decode(True, 128, B * Hq, True, N)
    dev = _dev()
    g = torch.Generator().manual_seed(7 * t + N)
    q, K, V = _fused_inputs(kind, B, Hq, Hkv, t, g)
    K, V = K.to(dev), V.to(dev)
    K64, V64 = _np(K), _np(V)
    eng = DecodeEngine(K, Hq, N)
    G = Hq // Hkv
    for step in range(2):
        qs = (q if step == 0 else q.roll(1, dims=1)).to(dev)
        eng.anchor_step(qs, K, V, P.PRHS_TOPN, N)
        torch.cuda.synchronize()
        s_all = O.attention_scores(_np(qs), K64)
        for b in range(B):
            for h in range(Hq):
                s = s_all[b, h]
                assert int(eng.count[b, h]) == N
                gidx = eng.idx[b, h, :N].cpu().numpy()
                assert np.all(np.diff(gidx) > 0) and gidx.min() >= 0 and gidx.max() < t
                S = O.topn_select(s, N) if check_set_band(gidx, s, N) else gidx
                o_ref, lse_ref = O.sparse_attention(s, V64[b, h // G], S)
                d_ref, _ = O.dropped_mass(s, S)
                assert np.max(np.abs(_np(eng.out[b, h]) - o_ref)) <= OUT_TOL, (step, b, h)
                assert abs(eng.lse_sel[b, h].item() - lse_ref) <= 1e-3, (step, b, h)
                assert abs(eng.delta[b, h].item() - d_ref) <= DELTA_TOL, (step, b, h)
                assert abs(eng.tau[b, h].item() - (1.0 - d_ref)) <= DELTA_TOL


REUSE_CASES = [
    # B, Hq, Hkv, d, t, dtype, anchor cap, radius, anchor lists
    (2, 64, 8, 128, 5000, torch.float16, 512, 2, "sorted"),    # 128 heads: one kernel
    (1, 128, 32, 64, 3001, torch.float16, 300, 0, "sorted"),   # radius 0, d = 64
    (1, 128, 16, 128, 2000, torch.float32, 200, 31, "sorted"), # 2r + 1 = 63, fp32
    (1, 128, 16, 128, 2000, torch.float16, 100, 40, "sorted"), # 2r + 1 = 81: dilation kernel first
    (1, 8, 2, 128, 3000, torch.float16, 256, 2, "sorted"),     # 8 heads: split decode and merge
    (1, 128, 32, 128, 4000, torch.float16, 700, 2, "edges"),   # empty, clamped, ends, unsorted
]


def _anchor_lists(kind, B, H, t, cap, g):
    idx = torch.zeros((B, H, cap), dtype=torch.int32)
    cnt = torch.zeros((B, H), dtype=torch.int32)
    for b in range(B):
        for h in range(H):
            n = int(torch.randint(cap // 2, cap + 1, (1,), generator=g))
            sel = torch.randperm(t, generator=g)[:n].sort().values.to(torch.int32)
            idx[b, h, :n] = sel
            cnt[b, h] = n
    if kind == "edges":
        cnt[0, 0] = 0                                   # empty
        idx[0, 1] = torch.randperm(t, generator=g)[:cap].sort().values.to(torch.int32)
        cnt[0, 1] = cap + 50                            # clamped to cap
        idx[0, 2, :3] = torch.tensor([0, 1, t - 1], dtype=torch.int32)
        cnt[0, 2] = 3                                   # both ends of the context
        idx[0, 3, :6] = torch.tensor([40, 10, 10, 900, 5, t + 7], dtype=torch.int32)
        cnt[0, 3] = 6                                   # unsorted, repeated, out of range
    return idx, cnt


@pytest.mark.parametrize("B,Hq,Hkv,d,t,dtype,cap,r,kind", REUSE_CASES)
def test_reuse_step_matches_two_calls(B, Hq, Hkv, d, t, dtype, cap, r, kind):
    """The one-call reuse step equals prhs_cis_reuse followed by a gathered-K
    prhs_sparse_decode, bit for bit, and the oracle on well-formed heads."""
    dev = _dev()
    g = torch.Generator().manual_seed(t + cap + r)
    K = torch.randn((B, Hkv, t, d), generator=g).to(dtype).to(dev)
    V = torch.randn((B, Hkv, t, d), generator=g).to(dtype).to(dev)
    q = (torch.randn((B, Hq, d), generator=g) * 2.0).to(dtype).to(dev)
    aidx, acnt = _anchor_lists(kind, B, Hq, t, cap, g)
    aidx, acnt = aidx.to(dev), acnt.to(dev)
    dims = P.make_dims(K, Hq)
    ocap = min(t, (2 * r + 1) * cap)
    res = []
    for one_call in (True, False):
        o_idx = torch.full((B, Hq, ocap), -7, dtype=torch.int32, device=dev)
        o_cnt = torch.full((B, Hq), -7, dtype=torch.int32, device=dev)
        out = torch.full((B, Hq, d), 7.0, device=dev)
        lse = torch.full((B, Hq), 7.0, device=dev)
        ws = P.alloc_workspace(dims, P.PRHS_OP_DECODE, ocap, device=dev)
        if one_call:
            P.prhs_reuse_step(dims, aidx, cap, acnt, r, q, K, V, o_idx, ocap, o_cnt, out, lse, ws)
        else:
            P.prhs_cis_reuse(dims, aidx, cap, acnt, r, None, None, 0.0, o_idx, ocap, o_cnt)
            P.prhs_sparse_decode(dims, q, K, V, o_idx, ocap, o_cnt, None, None, out, lse, ws=ws)
        torch.cuda.synchronize()
        res.append((o_idx, o_cnt, out, lse))
    (i1, c1, o1, l1), (i2, c2, o2, l2) = res
    assert torch.equal(c1, c2)
    for b in range(B):
        for h in range(Hq):
            n = int(c1[b, h])
            assert torch.equal(i1[b, h, :n], i2[b, h, :n]), (b, h)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # the oracle on well-formed heads
    s_all = O.attention_scores(_np(q), _np(K))
    V64 = _np(V)
    G = Hq // Hkv
    a_cpu, n_cpu = aidx.cpu().numpy(), acnt.cpu().numpy()
    for b in range(B):
        for h in range(0, Hq, 7):
            if kind == "edges" and b == 0 and h in (0, 1, 3):
                continue
            n = int(min(n_cpu[b, h], cap))
            D_ref = O.cis_dilate(a_cpu[b, h, :n], r, t)
            assert int(c1[b, h]) == len(D_ref)
            assert np.array_equal(i1[b, h, :len(D_ref)].cpu().numpy(), D_ref)
            if len(D_ref):
                o_ref, l_ref = O.sparse_attention(s_all[b, h], V64[b, h // G], D_ref)
                assert np.max(np.abs(_np(o1[b, h]) - o_ref)) <= OUT_TOL
                assert abs(l1[b, h].item() - l_ref) <= 1e-3
    if kind == "edges":
        assert int(c1[0, 0]) == 0 and o1[0, 0].abs().max().item() == 0.0
        assert l1[0, 0].item() == -float("inf")
        D1 = O.cis_dilate(a_cpu[0, 1, :cap], r, t)
        assert int(c1[0, 1]) == len(D1) and np.array_equal(i1[0, 1, :len(D1)].cpu().numpy(), D1)
        # unsorted input: strictly ascending output inside [0, t)
        n3 = int(c1[0, 3])
        got = i1[0, 3, :n3].cpu().numpy()
        assert n3 > 0 and np.all(np.diff(got) > 0) and got.min() >= 0 and got.max() < t


@pytest.mark.parametrize("q_scale", [(1.0, 1.0), (1.0, 4.0)])
def test_delta_consecutive_steps(q_scale):
    """Consecutive DELTA anchor steps over a drifting query: every head of every
    step matches the oracle (smallest N with delta <= target, capped), and a
    call given a threshold hint selects exactly what a call without one does."""
    dev = _dev()
    cfg = CONFIGS["delta_16k"].replace(batch=2, n_q_heads=8, n_kv_heads=8, ctx_len=8192,
                                       budget=1024, steps=4, q_scale=q_scale)
    w = make_workload(cfg, device=dev, layer=3)
    hinted = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    plain = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    K64, V64 = _np(w.K), _np(w.V)
    for step in range(cfg.steps):
        hinted.anchor_step(w.q[step], w.K, w.V, P.PRHS_DELTA, cfg.budget, cfg.delta_star)
        plain.anchor_step(w.q[step], w.K, w.V, P.PRHS_DELTA, cfg.budget, cfg.delta_star,
                          hint=False)
        torch.cuda.synchronize()
        assert torch.equal(hinted.count, plain.count) and torch.equal(hinted.cap_hit, plain.cap_hit)
        s_all = O.attention_scores(_np(w.q[step]), K64)
        for b in range(cfg.batch):
            for h in range(cfg.n_q_heads):
                n = int(hinted.count[b, h])
                gidx = hinted.idx[b, h, :n].cpu().numpy()
                assert np.array_equal(gidx, plain.idx[b, h, :n].cpu().numpy()), (step, b, h)
                s = s_all[b, h]
                _, lse = O.dense_softmax(s)
                exact = check_delta_choice(gidx, n, s, float(lse), cfg.budget, cfg.delta_star,
                                           cap_hit=int(hinted.cap_hit[b, h]))
                S = O.topn_select(s, n) if exact else gidx
                o_ref, _ = O.sparse_attention(s, V64[b, h], S)
                d_ref, _ = O.dropped_mass(s, S)
                assert np.max(np.abs(_np(hinted.out[b, h]) - o_ref)) <= OUT_TOL, (step, b, h)
                assert abs(hinted.delta[b, h].item() - d_ref) <= DELTA_TOL


def _small_cis(dev, batch=1, heads=8, ctx=4096, steps=8):
    cfg = CONFIGS["llama2_cis_8k"].replace(batch=batch, n_q_heads=heads, n_kv_heads=heads,
                                           ctx_len=ctx, budget=256, steps=steps)
    return cfg, make_workload(cfg, device=dev)


def _same_decode(a, b, n, vmax, names=("out", "lse_sel", "delta", "tau")):
    """Outputs of one selection decoded by two paths: bit-equal when both split
    and merge, else equal up to summation order."""
    fused = fused_anchor_decode(True, a.out.shape[-1], a.out.shape[0] * a.out.shape[1], True, n)
    otol, ltol = reorder_tols(n, vmax) if fused else (0.0, 0.0)
    for name in names:
        x, y = getattr(a, name), getattr(b, name)
        tol = otol if name == "out" else ltol
        assert (x - y).abs().max().item() <= tol, name


def test_adaptive_all_refresh_equals_anchor_steps():
    """A threshold above 1 refreshes every head at every step: the gated step then
    selects exactly what plain anchor steps select, and decodes to the same
    outputs (bit-equal, or up to summation order where the anchor step decodes
    inside its select kernel)."""
    dev = _dev()
    cfg, w = _small_cis(dev)
    ad = AdaptiveEngine(w.K, cfg.n_q_heads, cfg.budget, cfg.radius, 4, 2.0)
    an = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    vmax = w.V.abs().max().item()
    for step in range(cfg.steps):
        ad.step(w.q[step], w.K, w.V)
        an.anchor_step(w.q[step], w.K, w.V, P.PRHS_TOPN, cfg.budget)
        torch.cuda.synchronize()
        assert torch.all(ad.refresh == 1)
        assert torch.equal(ad.lse_all, an.lse_all), step
        _same_decode(ad, an, cfg.budget, vmax)
        assert torch.equal(ad.anchor_idx, an.idx) and torch.equal(ad.anchor_count, an.count)


@pytest.mark.parametrize("batch", [1, 16])
def test_adaptive_never_gated_follows_period(batch):
    """A threshold below -1 never fires: heads refresh exactly on the forced steps,
    and the shared steps equal the plain CIS reuse step bit for bit (8 heads:
    dilation, then split decode; 128 heads: dilation inside the decode kernel)."""
    dev = _dev()
    cfg, w = _small_cis(dev, batch=batch)
    period = 3
    ad = AdaptiveEngine(w.K, cfg.n_q_heads, cfg.budget, cfg.radius, period, -2.0)
    anchor = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    reuse = DecodeEngine(w.K, cfg.n_q_heads, ad.dil_cap)
    for step in range(cfg.steps):
        ad.step(w.q[step], w.K, w.V)
        if step % period == 0:
            anchor.anchor_step(w.q[step], w.K, w.V, P.PRHS_TOPN, cfg.budget)
        else:
            reuse.reuse_step(w.q[step], w.K, w.V, anchor.idx, anchor.count, cfg.budget, cfg.radius)
        torch.cuda.synchronize()
        assert torch.all(ad.refresh == int(step % period == 0))
        if step % period == 0:
            _same_decode(ad, anchor, cfg.budget, w.V.abs().max().item(), ("out", "lse_sel"))
        else:
            assert torch.equal(ad.out, reuse.out) and torch.equal(ad.lse_sel, reuse.lse_sel), step
        if step % period:
            assert torch.equal(ad.dil_count, reuse.count)
            for b in range(cfg.batch):
                for h in range(cfg.n_q_heads):
                    c = int(reuse.count[b, h])
                    assert torch.equal(ad.dil_idx[b, h, :c], reuse.idx[b, h, :c]), (step, b, h)


@pytest.mark.parametrize("batch", [2, 16])
def test_adaptive_graph_replay(batch):
    """The gated step captured as a HIP graph replays to the eager results, replay
    after replay, with the state reset and eager work in between (16 heads:
    split decode and merge; 128 heads: one workgroup per head)."""
    dev = _dev()
    cfg, w = _small_cis(dev, batch=batch)
    steps = 6

    def fresh():
        return AdaptiveEngine(w.K, cfg.n_q_heads, cfg.budget, cfg.radius, 4, 0.97)

    eager = fresh()
    for step in range(steps):
        eager.step(w.q[step], w.K, w.V)
    torch.cuda.synchronize()
    names = ("out", "lse_sel", "anchor_idx", "anchor_count", "dil_count", "refresh", "anchor_q")
    ref = {n: getattr(eager, n).clone() for n in names}
    eng = fresh()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for step in range(steps):
            eng.step(w.q[step], w.K, w.V)
    other = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    for r in range(3):
        other.anchor_step(w.q[r], w.K, w.V, P.PRHS_TOPN, cfg.budget)   # eager work in between
        eng.anchor_count.zero_()
        eng.anchor_q.zero_()
        eng.theta.fill_(float("nan"))
        eng.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(eng, n), ref[n]), (r, n)


@pytest.mark.parametrize("batch", [1, 16])
def test_reuse_step_graph_replay(batch):
    """A captured CIS reuse step (dilation, then decode over gathered K and V
    rows) replays to the eager results; at 128 heads the decode runs one
    workgroup per head."""
    dev = _dev()
    cfg, w = _small_cis(dev, batch=batch)
    H, N = cfg.n_q_heads, cfg.budget
    anchor = DecodeEngine(w.K, H, N)
    anchor.anchor_step(w.q[0], w.K, w.V, P.PRHS_TOPN, N)
    cap = (2 * cfg.radius + 1) * N
    eng = DecodeEngine(w.K, H, cap)
    eng.reuse_step(w.q[1], w.K, w.V, anchor.idx, anchor.count, N, cfg.radius)
    torch.cuda.synchronize()
    names = ("idx", "count", "out", "lse_sel")
    ref = {n: getattr(eng, n).clone() for n in names}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        eng.reuse_step(w.q[1], w.K, w.V, anchor.idx, anchor.count, N, cfg.radius)
    other = DecodeEngine(w.K, H, cap)
    for r in range(3):
        other.reuse_step(w.q[2 + r], w.K, w.V, anchor.idx, anchor.count, N, cfg.radius)
        for n in names:
            getattr(eng, n).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in ("count", "out", "lse_sel"):
            assert torch.equal(getattr(eng, n), ref[n]), (r, n)
        # the dilation writes the first count entries of each row
        for b in range(cfg.batch):
            for h in range(H):
                c = int(ref["count"][b, h])
                assert torch.equal(eng.idx[b, h, :c], ref["idx"][b, h, :c]), (r, b, h)


def test_dense_decode_deterministic_and_graph():
    dev = _dev()
    cfg, w = _small_cis(dev, batch=2, ctx=5000)
    eng = DecodeEngine(w.K, cfg.n_q_heads, 1, dense=True)
    eng.dense_step(w.q[0], w.K, w.V)
    torch.cuda.synchronize()
    out, lse = eng.out.clone(), eng.lse_all.clone()
    eng.dense_step(w.q[0], w.K, w.V)
    torch.cuda.synchronize()
    assert torch.equal(out, eng.out) and torch.equal(lse, eng.lse_all)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        eng.dense_step(w.q[0], w.K, w.V)
    for _ in range(3):
        eng.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eng.out)


def test_most_heads_one_call():
    """The largest head count a call takes (B * H_q = 65535: the scan's grid
    has one row of workgroups per KV head): an anchor step and a CIS reuse step
    over 65535 MHA heads, with sampled heads against the oracle."""
    dev = _dev()
    B, H, d, t, N, r = 3, 21845, 64, 160, 8, 1
    assert B * H == 65535
    g = torch.Generator().manual_seed(65535)
    K = torch.randn((B, H, t, d), generator=g).half().to(dev)
    V = torch.randn((B, H, t, d), generator=g).half().to(dev)
    q = (torch.randn((B, H, d), generator=g) * 2.0).half().to(dev)
    anchor = DecodeEngine(K, H, N)
    reuse = DecodeEngine(K, H, min(t, (2 * r + 1) * N))
    anchor.anchor_step(q, K, V, P.PRHS_TOPN, N)
    reuse.reuse_step(q, K, V, anchor.idx, anchor.count, N, r)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    heads = [(0, 0), (B - 1, H - 1)] + [(int(b), int(h)) for b, h in
                                        zip(rng.integers(0, B, 40), rng.integers(0, H, 40))]
    for (b, h) in heads:
        q64 = _np(q[b, h])[None, None]
        K64, V64 = _np(K[b, h]), _np(V[b, h])
        s = O.attention_scores(q64, K64[None, None])[0, 0]
        n = int(anchor.count[b, h])
        assert n == N
        gidx = anchor.idx[b, h, :n].cpu().numpy()
        exact = check_set_band(gidx, s, N)
        S = O.topn_select(s, N) if exact else gidx
        o_ref, lse_ref = O.sparse_attention(s, V64, S)
        assert np.max(np.abs(_np(anchor.out[b, h]) - o_ref)) <= OUT_TOL, (b, h)
        assert abs(anchor.lse_sel[b, h].item() - lse_ref) <= 1e-3, (b, h)
        D = O.cis_dilate(gidx, r, t)
        nd = int(reuse.count[b, h])
        assert np.array_equal(reuse.idx[b, h, :nd].cpu().numpy(), D), (b, h)
        o_ref, lse_ref = O.sparse_attention(s, V64, D)
        assert np.max(np.abs(_np(reuse.out[b, h]) - o_ref)) <= OUT_TOL, (b, h)
    del K, V, anchor, reuse
    torch.cuda.empty_cache()
