"""A seeded sweep of shapes through the one-call steps against the oracle:
48 cases drawn once from a fixed seed over batch, KV heads, query heads per KV
head (1-20, so one matrix-core launch, padded operands and runs of 16 all
occur), head_dim, dtype, context length (1 to 20 000, log-uniform), budget,
selection mode and dilation radius. Each case runs two anchor steps (the second
with the carried threshold hint) and a CIS reuse step of the second step's
set, and checks every head: the set against the oracle's (up to the tie band),
the attention output, the dropped mass and the dilated set (bit-exact)."""

import numpy as np
import pytest
import torch

from oracle import prhs_oracle as O
from sparse_top_kv_head_amd import prhs as P
from sparse_top_kv_head_amd.engine import DecodeEngine
from tests.parity_util import (DELTA_TOL, OUT_TOL, check_delta_choice, check_set_band)

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()
    return torch.device("cuda:0")


def _np(x):
    return x.detach().double().cpu().numpy()


def _cases(n=48, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 20]))
        d = int(rng.choice([64, 128]))
        f16 = bool(rng.random() < 0.75)
        t = int(np.exp(rng.uniform(0.0, np.log(20000.0))))
        t = max(t, 1)
        N = int(max(1, min(t, np.exp(rng.uniform(0.0, np.log(min(t, 4096) + 1))))))
        delta = bool(rng.random() < 0.3)
        ds = float(rng.choice([0.0, 0.02, 0.1, 0.4])) if delta else 0.0
        r = int(rng.choice([0, 1, 2, 3]))
        out.append((i, B, Hkv * G, Hkv, d, f16, t, N, delta, ds, r))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "case%02d" % c[0])
def test_sweep_steps_against_oracle(case):
    i, B, Hq, Hkv, d, f16, t, N, delta, ds, r = case
    print(f"sweep case {i}: B={B} Hq={Hq} Hkv={Hkv} d={d} f16={f16} t={t} N={N} "
          f"delta={delta} ds={ds} r={r}", flush=True)
    dev = _dev()
    dtype = torch.float16 if f16 else torch.float32
    g = torch.Generator().manual_seed(1000 + i)
    K = torch.randn((B, Hkv, t, d), generator=g).to(dtype).to(dev)
    V = torch.randn((B, Hkv, t, d), generator=g).to(dtype).to(dev)
    K64, V64 = _np(K), _np(V)
    G = Hq // Hkv
    mode = P.PRHS_DELTA if delta else P.PRHS_TOPN
    eng = DecodeEngine(K, Hq, N)
    cap = min(t, (2 * r + 1) * N)
    reuse = DecodeEngine(K, Hq, cap)
    for step in range(2):
        q = (torch.randn((B, Hq, d), generator=g) * 2.0).to(dtype).to(dev)
        eng.anchor_step(q, K, V, mode, N, ds)
        torch.cuda.synchronize()
        s_all = O.attention_scores(_np(q), K64)
        idx, cnt = eng.idx.cpu().numpy(), eng.count.cpu().numpy()
        out, dl, hit = _np(eng.out), _np(eng.delta), eng.cap_hit.cpu().numpy()
        for b in range(B):
            for h in range(Hq):
                s = s_all[b, h]
                _, lse = O.dense_softmax(s)
                n = int(cnt[b, h])
                gidx = idx[b, h, :n]
                assert n >= 1 and np.all(np.diff(gidx) > 0) and gidx.min() >= 0 and gidx.max() < t
                if mode == P.PRHS_TOPN:
                    assert n == N
                    exact = check_set_band(gidx, s, N)
                    S = O.topn_select(s, N) if exact else gidx
                else:
                    exact = check_delta_choice(gidx, n, s, float(lse), N, ds, cap_hit=int(hit[b, h]))
                    S = O.topn_select(s, n) if exact else gidx
                o_ref, _ = O.sparse_attention(s, V64[b, h // G], S)
                d_ref, _ = O.dropped_mass(s, S)
                assert np.max(np.abs(out[b, h] - o_ref)) <= OUT_TOL, (step, b, h)
                assert abs(dl[b, h] - d_ref) <= DELTA_TOL, (step, b, h)
    # reuse of the second step's sets for the same query, dilated by r
    reuse.reuse_step(q, K, V, eng.idx, eng.count, N, r)
    torch.cuda.synchronize()
    ridx, rcnt = reuse.idx.cpu().numpy(), reuse.count.cpu().numpy()
    rout, rlse = _np(reuse.out), _np(reuse.lse_sel)
    for b in range(B):
        for h in range(Hq):
            s = s_all[b, h]
            D = O.cis_dilate(idx[b, h, :int(cnt[b, h])], r, t)
            assert np.array_equal(ridx[b, h, :int(rcnt[b, h])], D), (b, h)
            o_ref, lse_ref = O.sparse_attention(s, V64[b, h // G], D)
            assert np.max(np.abs(rout[b, h] - o_ref)) <= OUT_TOL, (b, h)
            assert abs(rlse[b, h] - lse_ref) <= 1e-3, (b, h)
