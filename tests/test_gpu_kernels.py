"""Per-call parity of the HIP path (through the C ABI) against the fp64 oracle.

Inputs come from seeded generators on the host (or the synthetic workload
module); expected values come only from the oracle.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import prhs_oracle as O
from sparse_top_kv_head_amd import prhs as P
from sparse_top_kv_head_amd.engine import DecodeEngine
from tests.parity_util import (DELTA_TOL, OUT_TOL, check_delta_choice, check_set_band,
                               fused_anchor_decode, reorder_tols,
                               score_bound)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()
    return torch.device("cuda:0")


def _kv(B, Hkv, t, d, dtype, seed, pad_t=0, dev="cuda"):
    """Random K or V, optionally padded along the row stride (a strided view)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((B, Hkv, t, d + pad_t), generator=g, dtype=torch.float32).to(dtype)
    return x.to(dev)[..., :d]


def _np(x):
    return x.detach().double().cpu().numpy()


# ---------------------------------------------------------------------------
# prhs_score
# ---------------------------------------------------------------------------

SCORE_CASES = [
    # B, Hq, Hkv, d, t, dtype, pad
    (1, 4, 4, 64, 512, torch.float32, 0),     # toy shape
    (1, 8, 2, 128, 3000, torch.float16, 0),   # ragged t, G = 4
    (2, 8, 1, 64, 1537, torch.float16, 0),    # G = 8
    (1, 6, 2, 128, 1025, torch.float16, 8),   # G = 3 (2 + 1 sub-groups), strided rows
    (1, 4, 4, 128, 1, torch.float16, 0),      # t = 1
    (2, 4, 2, 128, 2048, torch.float32, 4),   # fp32, d = 128, strided rows
    (1, 16, 2, 128, 700, torch.float16, 0),   # G = 8, one partial chunk
    (1, 16, 1, 128, 3000, torch.float16, 0),  # G = 16: one matrix-core launch reads K once
    (2, 24, 1, 128, 1000, torch.float16, 8),  # G = 24: sub-groups of 16 and 8, strided rows
    (1, 16, 1, 64, 900, torch.float16, 0),    # G = 16 on the dot-product path: 8 + 8
    (1, 28, 4, 128, 2000, torch.float16, 0),  # G = 7 (Qwen2.5-7B grouping): one launch, 8-row operand
    (1, 24, 2, 128, 1500, torch.float16, 0),  # G = 12: one launch, 16-row operand
]


@pytest.mark.parametrize("B,Hq,Hkv,d,t,dtype,pad", SCORE_CASES)
def test_score_and_lse(B, Hq, Hkv, d, t, dtype, pad):
    dev = _dev()
    K = _kv(B, Hkv, t, d, dtype, 11, pad)
    g = torch.Generator().manual_seed(12)
    q = (torch.randn((B, Hq, d), generator=g) * 1.3).to(dtype).to(dev)
    dims = P.make_dims(K, Hq)
    scores = torch.full((B, Hq, dims.scores_ld), float("nan"), device=dev)
    lse = torch.empty((B, Hq), device=dev)
    ws = P.alloc_workspace(dims, P.PRHS_OP_SCORE, device=dev)
    P.prhs_score(dims, q, K, scores, lse, ws)
    torch.cuda.synchronize()
    bound, s_ref = score_bound(_np(q), _np(K))
    s_gpu = _np(scores)[..., :t]
    err = np.abs(s_gpu - s_ref)
    assert np.all(err <= bound), float((err / bound).max())
    _, lse_ref = O.dense_softmax(s_ref)
    lse_tol = bound.max(axis=-1) + 2e-5
    assert np.all(np.abs(_np(lse) - lse_ref) <= lse_tol)
    # scores only (no lse, no workspace)
    scores2 = torch.zeros_like(scores)
    P.prhs_score(dims, q, K, scores2, None, None)
    torch.cuda.synchronize()
    assert torch.equal(scores2[..., :t], scores[..., :t])


# ---------------------------------------------------------------------------
# prhs_select_topk, TOPN: the decision is taken on the same fp32 values on
# both sides, so the result must be bit-identical.
# ---------------------------------------------------------------------------

def _score_rows(kind, H, t, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        s = rng.standard_normal((H, t)) * 1.7
    elif kind == "ties":
        s = np.round(rng.standard_normal((H, t)) * 4) / 4
    elif kind == "flat":
        s = np.full((H, t), 0.5)
    elif kind == "signed_zero":
        s = rng.choice([-0.0, 0.0, 1.0, -1.0], size=(H, t))
    elif kind == "neg_inf":
        s = rng.standard_normal((H, t))
        s[rng.random((H, t)) < 0.5] = -np.inf
    elif kind == "wide":
        s = rng.standard_normal((H, t)) * 1e3 + rng.choice([-1e30, 1e30, 0], size=(H, t))
    else:
        raise ValueError(kind)
    return s.astype(np.float32)


SELECT_CASES = [
    ("normal", 3, 1), ("normal", 3, 2), ("normal", 5, 7), ("normal", 4, 1000), ("normal", 2, 1025),
    ("normal", 2, 4097), ("normal", 2, 32768), ("normal", 1, 65536), ("ties", 3, 5000),
    # the last length of the 512-thread workgroup (4096) and short rows of it with
    # ties, flat scores and -inf
    ("normal", 2, 4096), ("ties", 2, 4096), ("flat", 2, 2048), ("neg_inf", 2, 4000),
    ("flat", 2, 3000), ("signed_zero", 2, 777), ("neg_inf", 2, 2049), ("wide", 2, 16384),
    # sampled threshold and its streamed fallback at larger t
    ("flat", 2, 16384), ("ties", 2, 8192), ("neg_inf", 2, 32768), ("wide", 1, 65536),
    ("signed_zero", 2, 20000),
    # past the keys the registers hold: streamed search, emission in 64K tiles
    ("normal", 2, 65537), ("ties", 2, 100000), ("flat", 1, 131072), ("neg_inf", 1, 200000),
    ("signed_zero", 1, 140000), ("normal", 1, 262144),
]


@pytest.mark.parametrize("kind,H,t", SELECT_CASES)
def test_select_topn_exact(kind, H, t):
    dev = _dev()
    s = _score_rows(kind, H, t, 100 + t)
    ld = (t + 3) // 4 * 4
    buf = torch.zeros((1, H, ld), dtype=torch.float32)
    buf[0, :, :t] = torch.from_numpy(s)
    scores = buf.to(dev)
    dims = P.PrhsDims(1, H, H, 128, t, P.PRHS_F16, H * t * 128, t * 128, 128, ld)
    Ns = sorted({1, max(1, t // 3), max(1, t - 1), t, min(t, 2048)})
    if kind == "neg_inf":
        Ns.append(min(t, int((s[0] > -np.inf).sum()) + 3))
    for N in Ns:
        cap = N + 5
        idx = torch.full((1, H, cap), -7, dtype=torch.int32, device=dev)
        cnt = torch.full((1, H), -7, dtype=torch.int32, device=dev)
        P.prhs_select_topk(dims, scores, None, P.PRHS_TOPN, N, 0.0, idx, cap, cnt)
        torch.cuda.synchronize()
        gi = idx.cpu().numpy()[0]
        gc = cnt.cpu().numpy()[0]
        for h in range(H):
            assert gc[h] == N
            ref = O.topn_select(s[h].astype(np.float64), N)
            assert np.array_equal(gi[h, :N], ref), (kind, t, N, h)
            assert np.all(gi[h, N:] == -7)   # nothing written past the count


def test_select_deterministic_and_in_place():
    dev = _dev()
    H, t, N = 4, 32768, 2048
    s = _score_rows("ties", H, t, 5)
    scores = torch.from_numpy(s).reshape(1, H, t).to(dev)
    dims = P.PrhsDims(1, H, H, 128, t, P.PRHS_F16, H * t * 128, t * 128, 128, t)
    outs = []
    for _ in range(3):
        idx = torch.empty((1, H, N), dtype=torch.int32, device=dev)
        cnt = torch.empty((1, H), dtype=torch.int32, device=dev)
        P.prhs_select_topk(dims, scores, None, P.PRHS_TOPN, N, 0.0, idx, N, cnt)
        outs.append((idx.cpu(), cnt.cpu()))
    for i, c in outs[1:]:
        assert torch.equal(i, outs[0][0]) and torch.equal(c, outs[0][1])


# ---------------------------------------------------------------------------
# prhs_select_topk, DELTA
# ---------------------------------------------------------------------------

DELTA_CASES = [
    # scale of the scores, t, cap, delta*, quantum (0: continuous scores)
    (4.0, 4096, 2048, 0.05, 0), (8.0, 16384, 2048, 0.05, 0), (1.0, 16384, 2048, 0.05, 0),
    (3.0, 1000, 1000, 0.0, 0), (3.0, 1000, 1000, 1.0, 0), (6.0, 777, 50, 0.2, 0),
    (2.0, 32768, 4096, 0.1, 0), (12.0, 65536, 512, 0.01, 0), (3.0, 8192, 1024, 0.3, 0),
    # coarse score grids: many keys tie with the boundary key
    (4.0, 16384, 2048, 0.05, 0.5), (1.0, 6000, 3000, 0.2, 0.25), (6.0, 20000, 800, 0.1, 1.0),
    # past 64K keys: streamed searches, tiled emission
    (4.0, 131072, 2048, 0.05, 0), (12.0, 100000, 512, 0.01, 0), (2.0, 262144, 4096, 0.1, 0.5),
]


@pytest.mark.parametrize("scale,t,cap,ds,quant", DELTA_CASES)
def test_select_delta(scale, t, cap, ds, quant):
    dev = _dev()
    H = 4
    rng = np.random.default_rng(int(scale * 100) + t)
    s = (rng.standard_normal((H, t)) * scale).astype(np.float32)
    s[:, rng.integers(0, t, 5)] += 3 * scale   # a few sinks
    if quant:
        s = (np.round(s / quant) * quant).astype(np.float32)
    _, lse = O.dense_softmax(s.astype(np.float64))
    ld = (t + 3) // 4 * 4
    buf = torch.zeros((1, H, ld), dtype=torch.float32)
    buf[0, :, :t] = torch.from_numpy(s)
    scores = buf.to(dev)
    lse_t = torch.from_numpy(lse.astype(np.float32)).reshape(1, H).to(dev)
    dims = P.PrhsDims(1, H, H, 128, t, P.PRHS_F16, H * t * 128, t * 128, 128, ld)
    idx = torch.full((1, H, cap), -7, dtype=torch.int32, device=dev)
    cnt = torch.empty((1, H), dtype=torch.int32, device=dev)
    hit = torch.full((1, H), -1, dtype=torch.int32, device=dev)
    P.prhs_select_topk(dims, scores, lse_t, P.PRHS_DELTA, cap, ds, idx, cap, cnt, hit)
    torch.cuda.synchronize()
    gi, gc, gh = idx.cpu().numpy()[0], cnt.cpu().numpy()[0], hit.cpu().numpy()[0]
    s64 = s.astype(np.float64)
    for h in range(H):
        n = int(gc[h])
        check_delta_choice(gi[h, :n], n, s64[h], float(lse[h]), cap, ds, cap_hit=gh[h])


# ---------------------------------------------------------------------------
# prhs_cis_reuse
# ---------------------------------------------------------------------------

def _run_cis(anchor_sets, t, r, q_cur=None, q_anc=None, tau=0.0):
    dev = _dev()
    H = len(anchor_sets)
    acap = max(1, max(len(a) for a in anchor_sets))
    aidx = torch.full((1, H, acap), -1, dtype=torch.int32)
    acnt = torch.zeros((1, H), dtype=torch.int32)
    for h, a in enumerate(anchor_sets):
        aidx[0, h, :len(a)] = torch.as_tensor(a, dtype=torch.int32)
        acnt[0, h] = len(a)
    ocap = min(t, (2 * r + 1) * acap)
    out = torch.full((1, H, ocap), -7, dtype=torch.int32, device=dev)
    ocnt = torch.full((1, H), -7, dtype=torch.int32, device=dev)
    ok = torch.full((1, H), -7, dtype=torch.int32, device=dev) if q_cur is not None else None
    dims = P.PrhsDims(1, H, H, 128, t, P.PRHS_F16, H * t * 128, t * 128, 128, (t + 3) // 4 * 4)
    P.prhs_cis_reuse(dims, aidx.to(dev), acap, acnt.to(dev), r, q_cur, q_anc, tau, out, ocap, ocnt, ok)
    torch.cuda.synchronize()
    res = []
    for h in range(H):
        n = int(ocnt[0, h])
        res.append(out[0, h, :n].cpu().numpy())
    return res, (ok.cpu().numpy()[0] if ok is not None else None)


def test_cis_fig4_golden():
    g = json.load(open(os.path.join(GOLDEN, "cis_fig4.json")))
    anchor = [i for a, b in g["anchor"] for i in range(a, b + 1)]
    for case in g["cases"]:
        (D,), _ = _run_cis([anchor], g["t"], case["r"])
        expect = [i for a, b in case["expect_runs"] for i in range(a, b + 1)]
        assert D.tolist() == expect


@pytest.mark.parametrize("t,n,r", [(8192, 512, 2), (8192, 512, 0), (1000, 300, 1), (300, 300, 3),
                                   (5000, 700, 40), (64, 10, 100), (20000, 1, 5), (70000, 3000, 2)])
def test_cis_random_sets(t, n, r):
    rng = np.random.default_rng(t + n + r)
    sets = [np.sort(rng.choice(t, size=min(n, t), replace=False)) for _ in range(5)]
    sets.append(np.arange(min(n, t)))                       # one contiguous run at the start
    sets.append(np.arange(t - min(n, t), t))                # ... and at the end
    got, _ = _run_cis(sets, t, r)
    for a, D in zip(sets, got):
        assert np.array_equal(D, O.cis_dilate(a, r, t))


def test_cis_empty_and_gate():
    dev = _dev()
    t, d, H = 4096, 128, 6
    rng = np.random.default_rng(9)
    q_anc = rng.standard_normal((H, d))
    # current queries at chosen cosines to the anchor
    cos_target = np.array([0.99, 0.85, 0.79, 0.5, -0.2, 0.81])
    q_cur = np.empty_like(q_anc)
    for h in range(H):
        a = q_anc[h] / np.linalg.norm(q_anc[h])
        o = rng.standard_normal(d)
        o -= (o @ a) * a
        o /= np.linalg.norm(o)
        q_cur[h] = (cos_target[h] * a + math.sqrt(1 - cos_target[h] ** 2) * o) * 7.0
    qa = torch.from_numpy(q_anc).to(torch.float16).reshape(1, H, d).to(dev)
    qc = torch.from_numpy(q_cur).to(torch.float16).reshape(1, H, d).to(dev)
    sets = [np.array([5, 6, 7]), np.array([], dtype=np.int64), np.array([0]), np.array([4095]),
            np.array([10, 4000]), np.array([1, 2, 3, 4])]
    got, ok = _run_cis(sets, t, 2, qc, qa, 0.8)
    for a, D in zip(sets, got):
        assert np.array_equal(D, O.cis_dilate(a, 2, t))
    qa64, qc64 = _np(qa)[0], _np(qc)[0]
    for h in range(H):
        c = qa64[h] @ qc64[h] / np.linalg.norm(qa64[h]) / np.linalg.norm(qc64[h])
        assert abs(c - 0.8) > 1e-3
        assert ok[h] == int(c >= 0.8)


# ---------------------------------------------------------------------------
# prhs_sparse_decode (+ fused delta) and prhs_dropped_mass
# ---------------------------------------------------------------------------

DECODE_CASES = [
    # B, Hq, Hkv, d, t, dtype, N
    (1, 4, 4, 64, 512, torch.float32, 64),
    (1, 8, 2, 128, 3000, torch.float16, 300),
    (2, 8, 1, 64, 1537, torch.float16, 1537),
    (1, 4, 4, 128, 4096, torch.float16, 1),
    (1, 8, 4, 128, 9000, torch.float16, 2048),
    # >= 128 heads: one workgroup per head, no merge
    (2, 64, 8, 128, 5000, torch.float16, 2048),
    (1, 128, 32, 64, 3001, torch.float16, 700),
    (1, 128, 16, 128, 2000, torch.float32, 500),
    (4, 32, 8, 128, 9000, torch.float16, 8000),    # capacity 8003, near the per-head limit
    (1, 128, 16, 128, 9000, torch.float16, 8190),  # capacity 8193: past it, split and merge
]


@pytest.mark.parametrize("B,Hq,Hkv,d,t,dtype,N", DECODE_CASES)
@pytest.mark.parametrize("with_scores", [True, False])
def test_sparse_decode(B, Hq, Hkv, d, t, dtype, N, with_scores):
    dev = _dev()
    K = _kv(B, Hkv, t, d, dtype, 21)
    V = _kv(B, Hkv, t, d, dtype, 22)
    g = torch.Generator().manual_seed(23)
    q = (torch.randn((B, Hq, d), generator=g) * 2.0).to(dtype).to(dev)
    q64, K64, V64 = _np(q), _np(K), _np(V)
    s = O.attention_scores(q64, K64)
    _, lse = O.dense_softmax(s)
    G = Hq // Hkv
    cap = N + 3
    idx = torch.full((B, Hq, cap), -1, dtype=torch.int32)
    cnt = torch.zeros((B, Hq), dtype=torch.int32)
    sets = {}
    for b in range(B):
        for h in range(Hq):
            S = O.topn_select(s[b, h], N)
            sets[(b, h)] = S
            idx[b, h, :N] = torch.from_numpy(S.astype(np.int32))
            cnt[b, h] = N
    dims = P.make_dims(K, Hq)
    scores = torch.zeros((B, Hq, dims.scores_ld), dtype=torch.float32)
    scores[..., :t] = torch.from_numpy(s.astype(np.float32))
    out = torch.empty((B, Hq, d), device=dev)
    lse_sel = torch.empty((B, Hq), device=dev)
    delta = torch.empty((B, Hq), device=dev)
    tau = torch.empty((B, Hq), device=dev)
    lse_all = torch.from_numpy(lse.astype(np.float32)).to(dev)
    ws = P.alloc_workspace(dims, P.PRHS_OP_DECODE, cap, device=dev)
    P.prhs_sparse_decode(dims, q, K, V, idx.to(dev), cap, cnt.to(dev),
                         scores.to(dev) if with_scores else None, lse_all, out, lse_sel, delta, tau, ws)
    torch.cuda.synchronize()
    o_g, l_g, d_g, t_g = _np(out), _np(lse_sel), _np(delta), _np(tau)
    for b in range(B):
        for h in range(Hq):
            o_ref, lse_ref = O.sparse_attention(s[b, h], V64[b, h // G], sets[(b, h)])
            d_ref, tau_ref = O.dropped_mass(s[b, h], sets[(b, h)])
            assert np.max(np.abs(o_g[b, h] - o_ref)) <= OUT_TOL
            assert abs(l_g[b, h] - lse_ref) <= 1e-4
            assert abs(d_g[b, h] - d_ref) <= DELTA_TOL
            assert abs(t_g[b, h] - tau_ref) <= DELTA_TOL
    # standalone dropped mass agrees with the fused epilogue
    d2 = torch.empty_like(delta)
    P.prhs_dropped_mass(dims, lse_sel, lse_all, d2)
    torch.cuda.synchronize()
    assert torch.equal(d2, delta)


# ---------------------------------------------------------------------------
# prhs_dense_decode: the dense baseline (N = t)
# ---------------------------------------------------------------------------

DENSE_CASES = [
    # B, Hq, Hkv, d, t, dtype, row padding (strided K/V)
    (1, 4, 4, 64, 512, torch.float32, 0),
    (1, 8, 2, 128, 3000, torch.float16, 0),
    (2, 8, 1, 64, 1537, torch.float16, 8),
    (1, 6, 2, 128, 700, torch.float16, 0),      # G = 3: sub-groups of 2 and 1
    (2, 32, 32, 128, 4096, torch.float16, 0),   # LLaMA2-7B-shaped layer
    (1, 32, 8, 128, 9000, torch.float16, 0),    # Mistral-7B-shaped GQA layer
    (1, 16, 2, 128, 255, torch.float16, 0),     # G = 8, a single partial chunk
    (1, 2, 1, 128, 1, torch.float32, 0),        # one key
    (1, 16, 1, 128, 3000, torch.float16, 0),    # G = 16: one launch reads K and V once
    (1, 32, 2, 128, 600, torch.float32, 4),     # G = 16, fp32, strided rows
    (1, 16, 1, 64, 700, torch.float32, 0),      # G = 16, fp32, d = 64
    (1, 16, 1, 64, 300, torch.float16, 0),      # G = 16, fp16, d = 64: sub-groups of 8 and 8
]


@pytest.mark.parametrize("B,Hq,Hkv,d,t,dtype,pad", DENSE_CASES)
def test_dense_decode(B, Hq, Hkv, d, t, dtype, pad):
    dev = _dev()
    K = _kv(B, Hkv, t, d, dtype, 31, pad)
    V = _kv(B, Hkv, t, d, dtype, 32, pad)
    g = torch.Generator().manual_seed(33)
    q = (torch.randn((B, Hq, d), generator=g) * 2.0).to(dtype).to(dev)
    q64, K64, V64 = _np(q), _np(K), _np(V)
    s = O.attention_scores(q64, K64)
    _, lse = O.dense_softmax(s)
    G = Hq // Hkv
    dims = P.make_dims(K, Hq)
    out = torch.full((B, Hq, d), float("nan"), device=dev)
    lse_g = torch.full((B, Hq), float("nan"), device=dev)
    ws = P.alloc_workspace(dims, P.PRHS_OP_DENSE, device=dev)
    P.prhs_dense_decode(dims, q, K, V, out, lse_g, ws)
    torch.cuda.synchronize()
    o_g, l_g = _np(out), _np(lse_g)
    every = np.arange(t)
    for b in range(B):
        for h in range(Hq):
            o_ref, lse_ref = O.sparse_attention(s[b, h], V64[b, h // G], every)
            assert np.max(np.abs(o_g[b, h] - o_ref)) <= OUT_TOL, (b, h)
            assert abs(l_g[b, h] - lse[b, h]) <= 1e-4, (b, h)
            assert abs(lse_ref - lse[b, h]) <= 1e-12


# ---------------------------------------------------------------------------
# prhs_random_expand: the budget-matched random control of dilation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("t,n,m,bits", [(8192, 512, 2139, 23), (1000, 300, 1000, 23),
                                         (5000, 64, 64, 23), (3000, 200, 900, 3),
                                         (20000, 512, 2000, 23), (150000, 512, 2500, 23)])
def test_random_expand_exact(t, n, m, bits):
    """Bit-exact against the oracle: anchor sets from a clustered workload and
    random ones, draws from the seeded generator (bits=3: many equal draws, so
    the index tie rule decides)."""
    from sparse_top_kv_head_amd.synth import expansion_draws
    dev = _dev()
    H = 6
    rng = np.random.default_rng(t + n)
    acap = n
    aidx = torch.full((1, H, acap), -1, dtype=torch.int32)
    acnt = torch.zeros((1, H), dtype=torch.int32)
    sets = []
    for h in range(H):
        k = n if h % 3 else max(1, n // 2)        # some heads with fewer anchors
        S = np.sort(rng.choice(t, k, replace=False))
        if h == 1:
            S = np.arange(min(k, t))             # one contiguous run
        sets.append(S)
        aidx[0, h, :S.size] = torch.from_numpy(S.astype(np.int32))
        acnt[0, h] = S.size
    draws = expansion_draws(1, H, t, seed=7 + t, device=dev, bits=bits)
    dims = P.PrhsDims(1, H, H, 128, t, P.PRHS_F16, H * t * 128, t * 128, 128, (t + 3) // 4 * 4)
    out = torch.full((1, H, m), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((1, H), -7, dtype=torch.int32, device=dev)
    ws = P.alloc_workspace(dims, P.PRHS_OP_EXPAND, device=dev)
    P.prhs_random_expand(dims, aidx.to(dev), acap, acnt.to(dev), draws, m, out, m, cnt, ws)
    torch.cuda.synchronize()
    dr = draws.cpu().numpy()
    for h in range(H):
        ref = O.random_expansion(sets[h], dr[0, h], m)
        assert int(cnt[0, h]) == m
        assert np.array_equal(out[0, h].cpu().numpy(), ref), h


@pytest.mark.parametrize("H,cap", [(4, 300), (4, 256), (128, 300)])
def test_sparse_decode_edge_counts(H, cap):
    """Empty sets, counts above the capacity, out-of-range indices; split and
    merge (4 heads, 300 rows) and one workgroup per head (a one-split
    capacity, or 128 heads)."""
    dev = _dev()
    B, d, t = 1, 128, 600
    K = _kv(B, H, t, d, torch.float16, 31)
    V = _kv(B, H, t, d, torch.float16, 32)
    q = torch.randn((B, H, d), generator=torch.Generator().manual_seed(33)).half().to(dev)
    idx = torch.arange(cap, dtype=torch.int32).repeat(B, H, 1)
    idx[0, 2, 5] = -3        # skipped
    idx[0, 2, 6] = t + 10    # skipped
    cnt = torch.full((B, H), cap, dtype=torch.int32)
    cnt[0, :4] = torch.tensor([0, 1000, 10, cap], dtype=torch.int32)   # empty, clamped, bad ids, full
    dims = P.make_dims(K, H)
    out = torch.empty((B, H, d), device=dev)
    lse_sel = torch.empty((B, H), device=dev)
    ws = P.alloc_workspace(dims, P.PRHS_OP_DECODE, cap, device=dev)
    P.prhs_sparse_decode(dims, q, K, V, idx.to(dev), cap, cnt.to(dev), None, None, out, lse_sel,
                         None, None, ws)
    torch.cuda.synchronize()
    s = O.attention_scores(_np(q), _np(K))[0]
    V64 = _np(V)[0]
    assert torch.all(out[0, 0] == 0) and lse_sel[0, 0].item() == -math.inf
    for h, S in ((1, np.arange(cap)), (2, np.array([0, 1, 2, 3, 4, 7, 8, 9])), (3, np.arange(cap))):
        o_ref, l_ref = O.sparse_attention(s[h], V64[h], S)
        assert np.max(np.abs(_np(out)[0, h] - o_ref)) <= OUT_TOL
        assert abs(lse_sel[0, h].item() - l_ref) <= 1e-4


# ---------------------------------------------------------------------------
# The engine's anchor step on a small workload, compared in full.
# ---------------------------------------------------------------------------

def test_engine_topn_step_small():
    dev = _dev()
    from sparse_top_kv_head_amd.synth import CONFIGS, make_workload
    cfg = CONFIGS["toy"]
    w = make_workload(cfg, device=dev)
    eng = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    K64, V64 = _np(w.K), _np(w.V)
    for step in range(cfg.steps):
        q = w.q[step]
        eng.topn_step(q, w.K, w.V, cfg.budget)
        torch.cuda.synchronize()
        ref = O.decode_step(_np(q), K64, V64, "topn", N=cfg.budget)
        for (b, h), r in ref.items():
            gidx = eng.idx[b, h, :int(eng.count[b, h])].cpu().numpy()
            exact = check_set_band(gidx, r["scores"], cfg.budget)
            o_ref = r["out"] if exact else O.sparse_attention(r["scores"], V64[b, h], gidx)[0]
            assert np.max(np.abs(_np(eng.out[b, h]) - o_ref)) <= OUT_TOL
            assert abs(eng.delta[b, h].item() - r["delta"]) <= DELTA_TOL


# ---------------------------------------------------------------------------
# prhs_anchor_step: one call, same results as the three calls in sequence.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode,budget,heads", [
    (P.PRHS_TOPN, 256, 8),     # one-split budget: decoded inside the select kernel
    (P.PRHS_TOPN, 512, 8),     # decoded inside the select kernel at any head count
    (P.PRHS_TOPN, 2560, 8),    # budget over 2048: split decode and merge
    (P.PRHS_TOPN, 512, 128),
    (P.PRHS_DELTA, 256, 8),
    (P.PRHS_DELTA, 2560, 8),   # cap over 2048: split decode and merge
])
def test_anchor_step_matches_separate_calls(mode, budget, heads):
    """The one-call step selects exactly what the separate calls select; its
    outputs are bit-equal when it decodes the same way (split and merge) and
    equal up to summation order when the select kernel decodes too."""
    dev = _dev()
    from sparse_top_kv_head_amd.synth import CONFIGS, make_workload
    cfg = CONFIGS["llama2_4k"].replace(steps=2, n_q_heads=heads, n_kv_heads=heads // 4,
                                       budget=budget)
    w = make_workload(cfg, device=dev)
    a = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    b = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    q = w.q[1]
    ds = 0.3
    a.anchor_step(q, w.K, w.V, mode, cfg.budget, ds)
    b.score(q, w.K)
    b.select(mode, cfg.budget, ds)
    b.decode(q, w.K, w.V, True)
    torch.cuda.synchronize()
    assert torch.equal(a.scores[..., :cfg.ctx_len], b.scores[..., :cfg.ctx_len])
    assert torch.equal(a.lse_all, b.lse_all)
    assert torch.equal(a.count, b.count)
    for h in range(cfg.n_q_heads):
        n = int(a.count[0, h])
        assert torch.equal(a.idx[0, h, :n], b.idx[0, h, :n])
    fused = fused_anchor_decode(True, cfg.head_dim, heads, mode == P.PRHS_TOPN, budget)
    if fused:
        otol, ltol = reorder_tols(budget, w.V.abs().max().item())
        assert (a.out - b.out).abs().max().item() <= otol
        for name in ("lse_sel", "delta", "tau"):
            assert (getattr(a, name) - getattr(b, name)).abs().max().item() <= ltol, name
    else:
        for name in ("out", "lse_sel", "delta", "tau"):
            assert torch.equal(getattr(a, name), getattr(b, name)), name
    if mode == P.PRHS_DELTA:
        assert torch.equal(a.cap_hit, b.cap_hit)


@pytest.mark.parametrize("batch,budget", [(1, 512), (4, 512), (1, 2560)])
def test_anchor_step_graph_replay_matches_eager(batch, budget):
    """A captured step replays to the eager results, replay after replay, with
    eager work and synchronisations between the replays (budget 512: decoded
    inside the select kernel; 2560: split decode and merge)."""
    dev = _dev()
    from sparse_top_kv_head_amd.synth import CONFIGS, make_workload
    cfg = CONFIGS["mistral_gqa_32k"].replace(batch=batch, ctx_len=8192, budget=budget, steps=3,
                                             n_clusters=(64, 64))
    w = make_workload(cfg, device=dev)
    eng = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    other = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    # scores are not compared: the captured step carries a finite threshold
    # hint, and a hinted head whose candidates hold its answer gets no score row
    names = ("lse_all", "idx", "count", "out", "lse_sel", "delta", "tau")
    eng.anchor_step(w.q[1], w.K, w.V, P.PRHS_TOPN, cfg.budget)
    torch.cuda.synchronize()
    ref = {n: getattr(eng, n).clone() for n in names}
    eng.anchor_step(w.q[0], w.K, w.V, P.PRHS_TOPN, cfg.budget)      # overwrite before capture
    g = eng.capture([(w.q[1], w.K, w.V)], P.PRHS_TOPN, cfg.budget)
    for r in range(4):
        other.anchor_step(w.q[r % 3], w.K, w.V, P.PRHS_TOPN, cfg.budget)   # eager work in between
        for n in names:
            getattr(eng, n).fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(eng, n), ref[n]), (r, n)


# ---------------------------------------------------------------------------
# Threshold hints: results never depend on the hint.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ctx", [32768, 4096])
def test_anchor_step_hint_exact(ctx):
    """Steps with the carried hint, and with hints forced too high, too low and
    absent, give the same indices and outputs as steps without a hint. Where a
    forced hint misses on every head, the selection recomputes each skipped
    score row: the rows must be bit-identical to the scan's."""
    dev = _dev()
    from sparse_top_kv_head_amd.synth import CONFIGS, make_workload
    cfg = CONFIGS["mistral_gqa_32k"].replace(batch=1, ctx_len=ctx, budget=min(2048, ctx // 8),
                                             steps=4, n_clusters=(64, 64))
    w = make_workload(cfg, device=dev)
    hinted = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    plain = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    names = ("idx", "count", "out", "lse_sel", "delta", "tau", "lse_all")
    forced = {2: 1e30, 3: -1e30}
    for step in range(cfg.steps):
        if step in forced:
            hinted.theta.fill_(forced[step])
        hinted.anchor_step(w.q[step], w.K, w.V, P.PRHS_TOPN, cfg.budget)
        plain.anchor_step(w.q[step], w.K, w.V, P.PRHS_TOPN, cfg.budget, hint=False)
        torch.cuda.synchronize()
        assert torch.isfinite(hinted.theta).all()
        for n in names:
            a, b = getattr(hinted, n), getattr(plain, n)
            if n == "idx":
                for h in range(cfg.n_q_heads):
                    c = int(plain.count[0, h])
                    assert torch.equal(a[0, h, :c], b[0, h, :c]), (step, h)
            else:
                assert torch.equal(a, b), (step, n)
        # a hint of 1e30 lists no key; one of -1e30 lists every key, more
        # than the selection's 8192-entry list beyond 8K keys
        if step == 2 or (step == 3 and cfg.ctx_len > 8192):
            t = cfg.ctx_len
            assert torch.equal(hinted.scores[..., :t], plain.scores[..., :t]), step


@pytest.mark.parametrize("B,Hq,Hkv,t,pad,N", [
    (1, 6, 2, 3001, 0, 128),     # G = 3: sub-groups of 2 and 1, ragged t
    (2, 12, 2, 2048, 8, 256),    # G = 6: sub-groups of 4 and 2, strided rows
    (1, 16, 1, 1537, 0, 64),     # G = 16: one sub-group
    (1, 24, 1, 2500, 0, 128),    # G = 24: sub-groups of 16 and 8
    (1, 12, 1, 2000, 0, 128),    # G = 12: one sub-group, 16-row operand
    (1, 4, 4, 9000, 0, 512),     # MHA, t past the selection's 8192-entry list
    (1, 4, 1, 65536, 0, 1024),   # G = 4 at the largest context the registers hold
    (1, 4, 1, 262144, 0, 1024),  # the largest context the selection takes (streamed)
])
def test_anchor_step_recomputed_rows(B, Hq, Hkv, t, pad, N):
    """A hinted anchor step whose hints miss (too high: no key listed; too low:
    every key listed, beyond 8K keys more than the list holds) recomputes each
    skipped score row inside the selection. The rows, and everything selected
    and attended from them, equal those of an unhinted step bit for bit, for
    every query sub-group shape the scan launches."""
    dev = _dev()
    K = _kv(B, Hkv, t, 128, torch.float16, 11, pad_t=pad)
    V = _kv(B, Hkv, t, 128, torch.float16, 12, pad_t=pad)
    g = torch.Generator().manual_seed(13)
    q = torch.randn((B, Hq, 128), generator=g).to(torch.float16).to(dev)
    hinted = DecodeEngine(K, Hq, N)
    plain = DecodeEngine(K, Hq, N)
    plain.anchor_step(q, K, V, P.PRHS_TOPN, N, hint=False)
    lows = (-1e30,) if t > 8192 else ()
    for th in (1e30,) + lows:
        hinted.scores.fill_(float("nan"))
        hinted.theta.fill_(th)
        hinted.anchor_step(q, K, V, P.PRHS_TOPN, N)
        torch.cuda.synchronize()
        assert torch.equal(hinted.scores[..., :t], plain.scores[..., :t]), th
        for n in ("count", "lse_all", "out", "lse_sel", "delta", "tau"):
            assert torch.equal(getattr(hinted, n), getattr(plain, n)), (th, n)
        for b in range(B):
            for h in range(Hq):
                assert torch.equal(hinted.idx[b, h, :N], plain.idx[b, h, :N]), (th, b, h)


def test_scan_wide_rows_fall_back():
    """A KV head whose rows span 4 GiB or more (here a row stride of 2^20 + 128
    fp16 elements over 2048 keys) is scanned by the dot-product kernel, since
    the matrix-core kernel addresses a head's rows with 32-bit offsets; the
    scores still meet the rounding bound against the fp64 oracle, and a hinted
    anchor step still writes every score row (no row is skipped)."""
    dev = _dev()
    B, Hq, Hkv, d, t, N = 1, 4, 1, 128, 2048, 64
    st = (1 << 20) + 128
    assert t * st * 2 >= 1 << 32
    base = torch.empty((B, Hkv, t, st), dtype=torch.float16, device=dev)
    K = base[..., :d]
    g = torch.Generator().manual_seed(21)
    K.copy_(torch.randn((B, Hkv, t, d), generator=g).to(torch.float16))
    V = base[..., d:2 * d]
    V.copy_(torch.randn((B, Hkv, t, d), generator=g).to(torch.float16))
    q = torch.randn((B, Hq, d), generator=g).to(torch.float16).to(dev)
    eng = DecodeEngine(K, Hq, N)
    assert eng.dims.kv_stride_t == st
    eng.scores.fill_(float("nan"))
    eng.theta.fill_(-1e30)          # a finite hint on every head
    eng.anchor_step(q, K, V, P.PRHS_TOPN, N)
    torch.cuda.synchronize()
    bound, s_ref = score_bound(_np(q), _np(K))
    err = np.abs(_np(eng.scores)[..., :t] - s_ref)
    assert np.all(err <= bound), float(np.nanmax(err / bound))
    for h in range(Hq):
        sN = np.sort(s_ref[0, h])[::-1][N - 1]
        gidx = eng.idx[0, h, :N].cpu().numpy()
        ref = np.sort(np.argsort(-s_ref[0, h], kind="stable")[:N])
        diff = np.setxor1d(gidx, ref)
        assert np.all(np.abs(s_ref[0, h][diff] - sN) <= 1e-4), h
    del base, K, V, eng
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,d,pad,pos", [
    (torch.float16, 128, 8, 0), (torch.float16, 128, 0, 999), (torch.float32, 64, 4, 517),
    (torch.float32, 128, 0, 3), (torch.float16, 64, 0, 1000),
])
def test_append_kv(dtype, d, pad, pos):
    """prhs_append_kv writes exactly row pos of every (b, KV head) of K and V,
    bit for bit, and nothing else."""
    dev = _dev()
    B, Hkv, t = 3, 5, 1001
    K = _kv(B, Hkv, t, d, dtype, 31, pad_t=pad)
    V = _kv(B, Hkv, t, d, dtype, 32, pad_t=pad)
    g = torch.Generator().manual_seed(33)
    kn = torch.randn((B, Hkv, d), generator=g).to(dtype).to(dev)
    vn = torch.randn((B, Hkv, d), generator=g).to(dtype).to(dev)
    K_ref, V_ref = K.clone(), V.clone()
    K_ref[:, :, pos] = kn
    V_ref[:, :, pos] = vn
    P.prhs_append_kv(P.make_dims(K, Hkv), kn, vn, K, V, pos)
    torch.cuda.synchronize()
    assert torch.equal(K, K_ref) and torch.equal(V, V_ref)
