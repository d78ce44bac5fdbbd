"""GPU test of the device-checked library (libprhs_checked.so, built with
PRHS_DEVICE_CHECKS): clean calls succeed; a call whose inputs break the
documented contract (an index of a given set outside [0, t); an anchor set that
is not strictly ascending) returns PRHS_E_HIP naming the broken check, after
the kernels have run to completion exactly as in the unchecked build (they skip
such entries; nothing traps); the next clean call succeeds again. The checked
library is loaded in a child process, so this process keeps the product one."""

import os
import subprocess
import sys

import pytest
import torch

from sparse_top_kv_head_amd import build as B

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys, torch
sys.path.insert(0, sys.argv[1])
from sparse_top_kv_head_amd import prhs as P
from sparse_top_kv_head_amd.engine import DecodeEngine
assert P._LIB_PATH.endswith("libprhs_checked.so"), P._LIB_PATH
dev = torch.device("cuda:0")
g = torch.Generator().manual_seed(3)
B_, Hq, Hkv, d, t, N, r = 1, 8, 2, 128, 3000, 64, 2
K = torch.randn((B_, Hkv, t, d), generator=g).half().to(dev)
V = torch.randn((B_, Hkv, t, d), generator=g).half().to(dev)
q = torch.randn((B_, Hq, d), generator=g).half().to(dev)

def expect_check(fn, text):
    try:
        fn()
    except P.PrhsError as e:
        assert e.code == P.PRHS_E_HIP and "device check failed" in str(e) and text in str(e), str(e)
        print("caught:", str(e), flush=True)
        return
    raise AssertionError("no device check reported: " + text)

# clean calls: anchor step (scan, candidates, select, decode), reuse step (dilation + decode)
eng = DecodeEngine(K, Hq, N)
eng.anchor_step(q, K, V, P.PRHS_TOPN, N)
eng.anchor_step(q, K, V, P.PRHS_TOPN, N)          # with the carried hint
reuse = DecodeEngine(K, Hq, min(t, (2 * r + 1) * N))
reuse.reuse_step(q, K, V, eng.idx, eng.count, N, r)
torch.cuda.synchronize()

# a decode over a set holding an index past t
bad = eng.idx.clone()
bad[0, 3, 5] = t + 10
out = torch.empty((B_, Hq, d), device=dev)
lse = torch.empty((B_, Hq), device=dev)
ws = P.alloc_workspace(eng.dims, P.PRHS_OP_DECODE, N, device=dev)
expect_check(lambda: P.prhs_sparse_decode(eng.dims, q, K, V, bad, N, eng.count, None, None, out, lse,
                                          ws=ws), "an index outside [0, t)")
# the same set is fine again once the index is in range
P.prhs_sparse_decode(eng.dims, q, K, V, eng.idx, N, eng.count, None, None, out, lse, ws=ws)

# a dilation of an anchor set out of order
swapped = eng.idx.clone()
swapped[0, 2, 10], swapped[0, 2, 11] = eng.idx[0, 2, 11], eng.idx[0, 2, 10]
cap = min(t, (2 * r + 1) * N)
oidx = torch.empty((B_, Hq, cap), dtype=torch.int32, device=dev)
ocnt = torch.empty((B_, Hq), dtype=torch.int32, device=dev)
expect_check(lambda: P.prhs_cis_reuse(eng.dims, swapped, N, eng.count, r, None, None, 0.0, oidx, cap,
                                      ocnt), "not strictly ascending")
P.prhs_cis_reuse(eng.dims, eng.idx, N, eng.count, r, None, None, 0.0, oidx, cap, ocnt)
torch.cuda.synchronize()
print("CHECKS-OK", flush=True)
'''


def test_checked_library_reports_broken_contracts():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(B.CHECKED_LIB), \
        f"{B.CHECKED_LIB} is missing: build it with `python -m sparse_top_kv_head_amd.build --checked`"
    env = dict(os.environ, PRHS_LIB=B.CHECKED_LIB)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, env=env,
                       timeout=240)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "CHECKS-OK" in r.stdout
    assert r.stdout.count("caught:") == 2
