"""GPU test of prhs_sparse_decode_noalloc, the sparse decode that keeps its
split partials in the library's per-device scratch array instead of a caller
workspace. Each case makes two calls in a row, the second on a smaller input
(so the scratch still holds the first call's partials), and compares every
output with prhs_sparse_decode on the same inputs: both run the same kernels in
the same order, so the results must be bit-identical."""

import pytest
import torch

from sparse_top_kv_head_amd import prhs as P

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()
    return torch.device("cuda:0")


def _inputs(B, Hq, Hkv, d, t, cap, dtype, seed, dev):
    g = torch.Generator().manual_seed(seed)
    K = torch.randn((B, Hkv, t, d), generator=g).to(dtype).to(dev)
    V = torch.randn((B, Hkv, t, d), generator=g).to(dtype).to(dev)
    q = (torch.randn((B, Hq, d), generator=g) * 1.5).to(dtype).to(dev)
    dims = P.make_dims(K, Hq)
    scores = torch.full((B, Hq, dims.scores_ld), float("-inf"))
    scores[..., :t] = torch.randn((B, Hq, t), generator=g) * 3.0
    lse_all = torch.logsumexp(scores[..., :t].double(), dim=-1).float()
    # one set per head: a random count in [0, cap] (head 0 empty, head 1 full),
    # then that many distinct keys, ascending
    idx = torch.full((B, Hq, cap), -1, dtype=torch.int32)
    cnt = torch.randint(0, cap + 1, (B, Hq), generator=g, dtype=torch.int32)
    cnt.view(-1)[0] = 0
    cnt.view(-1)[min(1, B * Hq - 1)] = cap
    for b in range(B):
        for h in range(Hq):
            n = int(cnt[b, h])
            keys = torch.randperm(t, generator=g)[:n].sort().values
            idx[b, h, :n] = keys.to(torch.int32)
    return dict(dims=dims, q=q, K=K, V=V, idx=idx.to(dev), cap=cap, cnt=cnt.to(dev),
                scores=scores.to(dev), lse_all=lse_all.to(dev))


def _outputs(x, dev):
    B, Hq, d = x["q"].shape
    return dict(out=torch.full((B, Hq, d), float("nan"), device=dev),
                lse_sel=torch.full((B, Hq), float("nan"), device=dev),
                delta=torch.full((B, Hq), float("nan"), device=dev),
                tau=torch.full((B, Hq), float("nan"), device=dev))


def _run(x, dev, noalloc, with_scores):
    o = _outputs(x, dev)
    scores = x["scores"] if with_scores else None
    if noalloc:
        P.prhs_sparse_decode_noalloc(x["dims"], x["q"], x["K"], x["V"], x["idx"], x["cap"], x["cnt"],
                                     scores, x["lse_all"], o["out"], o["lse_sel"], o["delta"],
                                     o["tau"])
    else:
        ws = P.alloc_workspace(x["dims"], P.PRHS_OP_DECODE, x["cap"], device=dev)
        P.prhs_sparse_decode(x["dims"], x["q"], x["K"], x["V"], x["idx"], x["cap"], x["cnt"],
                             scores, x["lse_all"], o["out"], o["lse_sel"], o["delta"], o["tau"], ws)
    return o


# (B, H_q, H_kv, d, t, cap, dtype, with_scores) of the first and the second call
CASES = [
    # both split (fewer than 128 heads, sets over 256 rows)
    ((2, 32, 8, 128, 16384, 4096, torch.float16, True),
     (1, 8, 2, 64, 3001, 700, torch.float32, False)),
    # one workgroup per head (128 heads), then a split decode
    ((4, 32, 8, 128, 8192, 2048, torch.float16, True),
     (1, 4, 4, 128, 600, 300, torch.float16, True)),
    # the largest split a 16-head decode fits in the scratch, then a small one
    ((1, 16, 4, 128, 131072, 129024, torch.float16, True),
     (1, 16, 4, 128, 4096, 1000, torch.float16, False)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_decode(first, second):
    dev = _dev()
    for seed, (B, Hq, Hkv, d, t, cap, dtype, with_scores) in zip((101, 202), (first, second)):
        print(f"case B={B} Hq={Hq} Hkv={Hkv} d={d} t={t} cap={cap} {dtype} scores={with_scores}",
              flush=True)
        x = _inputs(B, Hq, Hkv, d, t, cap, dtype, seed, dev)
        need = P.prhs_workspace_bytes(x["dims"], P.PRHS_OP_DECODE, cap)
        assert need <= P.PRHS_NOALLOC_SCRATCH_BYTES
        got = _run(x, dev, True, with_scores)
        ref = _run(x, dev, False, with_scores)
        torch.cuda.synchronize()
        for k in ("out", "lse_sel", "delta", "tau"):
            assert torch.equal(got[k].isnan(), ref[k].isnan()), k
            assert torch.equal(torch.nan_to_num(got[k]), torch.nan_to_num(ref[k])), k
        # every head but the first (the empty set) has finite outputs
        assert torch.isfinite(got["out"].view(-1, d)[1:]).all()


def test_noalloc_rejects_oversize_on_device():
    """A split decode beyond the scratch is refused and leaves the outputs untouched."""
    dev = _dev()
    x = _inputs(1, 16, 4, 128, 131072, 129025, torch.float16, 303, dev)
    o = _outputs(x, dev)
    with pytest.raises(P.PrhsError, match="allocation-free"):
        P.prhs_sparse_decode_noalloc(x["dims"], x["q"], x["K"], x["V"], x["idx"], x["cap"], x["cnt"],
                                     x["scores"], x["lse_all"], o["out"], o["lse_sel"], o["delta"],
                                     o["tau"])
    torch.cuda.synchronize()
    assert o["out"].isnan().all() and o["lse_sel"].isnan().all()
