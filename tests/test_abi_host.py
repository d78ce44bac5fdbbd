"""The C-ABI library loads, exports every symbol include/*.h declares, and rejects
invalid arguments on the host before any HIP call (CPU only: every call here
fails validation, so nothing is ever launched)."""

import ctypes
import math
import os
import re

import pytest

from sparse_top_kv_head_amd import prhs as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prhs.h")
PROBE_HEADER = os.path.join(ROOT, "include", "prhs_probe.h")

FAKE = 0x100000          # 16-byte aligned, never dereferenced: every call below is invalid
FAKE_MIS = 0x100008      # 8-byte aligned only


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(P._LIB_PATH):
        from sparse_top_kv_head_amd import build
        build.build()
    return P.lib()


def _dims(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, ctx_len=1000, dtype=P.PRHS_F16,
                kv_stride_b=2 * 1000 * 128, kv_stride_h=1000 * 128, kv_stride_t=128, scores_ld=1000)
    base.update(kw)
    return P.PrhsDims(**base)


def _declared(path):
    return set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(prhs_\w+)\s*\(", open(path).read(), re.M))


def test_header_symbols_are_exported(L):
    text = open(HEADER).read()
    declared = _declared(HEADER)
    assert declared == set(P.EXPORTED)
    assert _declared(PROBE_HEADER) == set(P.PROBE_EXPORTED)
    for name in declared | _declared(PROBE_HEADER):
        assert hasattr(L, name), name
    assert P.PRHS_MAX_SELECT_CTX == int(re.search(r"PRHS_MAX_SELECT_CTX\s+(\d+)", text).group(1))
    assert P.PRHS_NOALLOC_SCRATCH_BYTES == int(
        re.search(r"PRHS_NOALLOC_SCRATCH_BYTES\s+\((\d+)u << 20\)", text).group(1)) << 20
    for const, value in re.findall(r"^\s*(PRHS_\w+)\s*=\s*(-?\d+)", text, re.M):
        assert getattr(P, const) == int(value), const


def _score(L, d, q=FAKE, k=FAKE, s=FAKE, lse=None, ws=None, wsb=0):
    return L.prhs_score(ctypes.byref(d) if d is not None else None, q, k, s, lse, ws, wsb, None)


def _select(L, d, scores=FAKE, lse=FAKE, mode=P.PRHS_TOPN, n=64, dt=0.05, idx=FAKE, cap=64, cnt=FAKE):
    return L.prhs_select_topk(ctypes.byref(d) if d is not None else None, scores, lse, mode, n, dt,
                              idx, cap, cnt, None, None, None)


def _cis(L, d, a=FAKE, acap=64, acnt=FAKE, r=2, qc=None, qa=None, tau=0.8, o=FAKE, ocap=320,
         ocnt=FAKE, ok=None):
    return L.prhs_cis_reuse(ctypes.byref(d) if d is not None else None, a, acap, acnt, r, qc, qa,
                            tau, o, ocap, ocnt, ok, None)


def _reuse(L, d, a=FAKE, acap=64, acnt=FAKE, r=2, q=FAKE, k=FAKE, v=FAKE, o=FAKE, ocap=320,
           ocnt=FAKE, out=FAKE, lsel=FAKE, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = 1 << 30
    return L.prhs_reuse_step(ctypes.byref(d) if d is not None else None, a, acap, acnt, r, q, k, v,
                             o, ocap, ocnt, out, lsel, ws, wsb, None)


def _decode(L, d, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cap=64, cnt=FAKE, s=FAKE, lse=FAKE, out=FAKE,
            lsel=FAKE, dl=FAKE, tau=FAKE, ws=FAKE, wsb=None, sel=None):
    if wsb is None:
        wsb = 1 << 30
    return L.prhs_sparse_decode(ctypes.byref(d) if d is not None else None, q, k, v, idx, cap, cnt,
                                sel, s, lse, out, lsel, dl, tau, ws, wsb, None)


def _dense(L, d, q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = 1 << 30
    return L.prhs_dense_decode(ctypes.byref(d) if d is not None else None, q, k, v, out, lse, ws,
                               wsb, None)


@pytest.mark.parametrize("field,value,code", [
    ("n_q_heads", 7, P.PRHS_E_DIMS),
    ("n_kv_heads", 0, P.PRHS_E_DIMS),
    ("batch", 0, P.PRHS_E_DIMS),
    ("batch", 10000, P.PRHS_E_DIMS),
    ("head_dim", 96, P.PRHS_E_DIMS),
    ("ctx_len", 0, P.PRHS_E_DIMS),
    ("dtype", 7, P.PRHS_E_DTYPE),
    ("kv_stride_t", 64, P.PRHS_E_DIMS),
    ("kv_stride_t", 132, P.PRHS_E_ALIGN),
    ("kv_stride_h", -128, P.PRHS_E_DIMS),
    ("kv_stride_b", 4, P.PRHS_E_ALIGN),
    ("scores_ld", 999, P.PRHS_E_DIMS),
    ("scores_ld", 1002, P.PRHS_E_ALIGN),
])
def test_bad_dims_rejected_by_every_call(L, field, value, code):
    d = _dims(**{field: value})
    assert _score(L, d) == code
    assert _select(L, d) == code
    assert _cis(L, d) == code
    assert _reuse(L, d) == code
    assert _decode(L, d) == code
    assert _dense(L, d) == code
    assert _adaptive(L, d) == code
    assert _expand(L, d) == code
    assert L.prhs_dropped_mass(ctypes.byref(d), FAKE, FAKE, FAKE, None, None) == code
    assert L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_SCORE, 0) == 0
    assert L.prhs_last_error()


def test_null_dims(L):
    assert _score(L, None) == P.PRHS_E_NULL
    assert _select(L, None) == P.PRHS_E_NULL
    assert _cis(L, None) == P.PRHS_E_NULL
    assert _reuse(L, None) == P.PRHS_E_NULL
    assert _decode(L, None) == P.PRHS_E_NULL
    assert L.prhs_dropped_mass(None, FAKE, FAKE, FAKE, None, None) == P.PRHS_E_NULL


def test_score_argument_checks(L):
    d = _dims()
    need = L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_SCORE, 0)
    assert need == 2 * 8 * 4 * 8          # B*H_q*chunks(256 keys)*(max, sum)
    assert _score(L, d, q=None) == P.PRHS_E_NULL
    assert _score(L, d, k=None) == P.PRHS_E_NULL
    assert _score(L, d, s=None) == P.PRHS_E_NULL
    assert _score(L, d, q=FAKE_MIS) == P.PRHS_E_ALIGN
    assert _score(L, d, s=FAKE_MIS) == P.PRHS_E_ALIGN
    assert _score(L, d, lse=FAKE, ws=None) == P.PRHS_E_WORKSPACE
    assert _score(L, d, lse=FAKE, ws=FAKE, wsb=need - 1) == P.PRHS_E_WORKSPACE
    assert _score(L, d, lse=FAKE, ws=FAKE_MIS, wsb=need) == P.PRHS_E_ALIGN


def test_select_argument_checks(L):
    d = _dims()
    assert _select(L, _dims(ctx_len=P.PRHS_MAX_SELECT_CTX + 1, scores_ld=P.PRHS_MAX_SELECT_CTX + 4)) == P.PRHS_E_DIMS
    assert _select(L, d, scores=None) == P.PRHS_E_NULL
    assert _select(L, d, idx=None) == P.PRHS_E_NULL
    assert _select(L, d, cnt=None) == P.PRHS_E_NULL
    assert _select(L, d, mode=5) == P.PRHS_E_BUDGET
    assert _select(L, d, mode=P.PRHS_DELTA, lse=None) == P.PRHS_E_NULL
    assert _select(L, d, n=0) == P.PRHS_E_BUDGET
    assert _select(L, d, n=1001, cap=2000) == P.PRHS_E_BUDGET
    assert _select(L, d, n=65, cap=64) == P.PRHS_E_CAPACITY
    for bad in (-0.1, 1.5, math.nan):
        assert _select(L, d, mode=P.PRHS_DELTA, dt=bad) == P.PRHS_E_BUDGET
    assert _select(L, d, scores=FAKE_MIS) == P.PRHS_E_ALIGN
    assert L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_SELECT, 0) == 0


def test_cis_argument_checks(L):
    d = _dims()
    assert _cis(L, d, a=None) == P.PRHS_E_NULL
    assert _cis(L, d, acnt=None) == P.PRHS_E_NULL
    assert _cis(L, d, o=None) == P.PRHS_E_NULL
    assert _cis(L, d, ocnt=None) == P.PRHS_E_NULL
    assert _cis(L, d, r=-1) == P.PRHS_E_BUDGET
    assert _cis(L, d, acap=0) == P.PRHS_E_CAPACITY
    assert _cis(L, d, ocap=319) == P.PRHS_E_CAPACITY          # (2r+1)*64 = 320 < t
    assert _cis(L, d, r=100, ocap=999) == P.PRHS_E_CAPACITY   # min(t, ...) = 1000
    assert _cis(L, d, ok=FAKE) == P.PRHS_E_NULL
    assert _cis(L, d, ok=FAKE, qc=FAKE, qa=FAKE, tau=math.nan) == P.PRHS_E_BUDGET


def test_reuse_step_argument_checks(L):
    d = _dims()
    need = L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_DECODE, 320)
    for name in ("a", "acnt", "o", "ocnt", "q", "k", "v", "out", "lsel"):
        assert _reuse(L, d, **{name: None}) == P.PRHS_E_NULL, name
    assert _reuse(L, d, r=-1) == P.PRHS_E_BUDGET
    assert _reuse(L, d, acap=0) == P.PRHS_E_CAPACITY
    assert _reuse(L, d, ocap=319) == P.PRHS_E_CAPACITY           # (2r+1)*64 = 320 < t
    assert _reuse(L, d, r=100, ocap=999) == P.PRHS_E_CAPACITY    # min(t, ...) = 1000
    for name in ("q", "k", "v"):
        assert _reuse(L, d, **{name: FAKE_MIS}) == P.PRHS_E_ALIGN, name
    assert _reuse(L, d, ws=None) == P.PRHS_E_WORKSPACE
    assert _reuse(L, d, wsb=need - 4) == P.PRHS_E_WORKSPACE
    assert _reuse(L, d, ws=FAKE_MIS, wsb=need) == P.PRHS_E_ALIGN


def test_decode_argument_checks(L):
    d = _dims()
    need = L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_DECODE, 600)
    assert need == 2 * 8 * 3 * (128 + 2) * 4     # B*H_q*ceil(600/256)*(d+2) floats
    assert _decode(L, d, v=None) == P.PRHS_E_NULL
    assert _decode(L, d, idx=None) == P.PRHS_E_NULL
    assert _decode(L, d, cnt=None) == P.PRHS_E_NULL
    assert _decode(L, d, out=None) == P.PRHS_E_NULL
    assert _decode(L, d, lsel=None) == P.PRHS_E_NULL
    assert _decode(L, d, s=None, k=None) == P.PRHS_E_NULL
    assert _decode(L, d, s=None, q=None) == P.PRHS_E_NULL
    assert _decode(L, d, s=None, q=None, k=None, cap=0, sel=FAKE) == P.PRHS_E_CAPACITY  # sel_scores suffice
    assert _decode(L, d, lse=None) == P.PRHS_E_NULL              # delta without lse_all
    assert _decode(L, d, dl=None) == P.PRHS_E_NULL               # tau without delta
    assert _decode(L, d, cap=0) == P.PRHS_E_CAPACITY
    assert _decode(L, d, ws=None) == P.PRHS_E_WORKSPACE
    assert _decode(L, d, cap=600, wsb=need - 4) == P.PRHS_E_WORKSPACE
    assert _decode(L, d, v=FAKE_MIS) == P.PRHS_E_ALIGN
    assert L.prhs_dropped_mass(ctypes.byref(d), FAKE, FAKE, None, None, None) == P.PRHS_E_NULL
    assert L.prhs_dropped_mass(ctypes.byref(d), None, FAKE, FAKE, None, None) == P.PRHS_E_NULL


def test_decode_noalloc_argument_checks(L):
    """The allocation-free decode validates like prhs_sparse_decode and
    refuses, before any HIP call, a decode whose split partials exceed its
    per-device scratch."""
    d = _dims()

    def call(dims, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cap=64, cnt=FAKE, s=FAKE, lse=FAKE, out=FAKE,
             lsel=FAKE, dl=FAKE, tau=FAKE, sel=None):
        return L.prhs_sparse_decode_noalloc(ctypes.byref(dims) if dims is not None else None, q, k,
                                            v, idx, cap, cnt, sel, s, lse, out, lsel, dl, tau, None)
    assert call(None) == P.PRHS_E_NULL
    assert call(_dims(head_dim=96)) == P.PRHS_E_DIMS
    for kw in ("v", "idx", "cnt", "out", "lsel"):
        assert call(d, **{kw: None}) == P.PRHS_E_NULL, kw
    assert call(d, s=None, k=None) == P.PRHS_E_NULL
    assert call(d, lse=None) == P.PRHS_E_NULL
    assert call(d, dl=None) == P.PRHS_E_NULL
    assert call(d, cap=0) == P.PRHS_E_CAPACITY
    assert call(d, v=FAKE_MIS) == P.PRHS_E_ALIGN
    # the largest idx_cap whose split partials fit, and one past it
    per_tile = L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_DECODE, 256)
    cap_fit = P.PRHS_NOALLOC_SCRATCH_BYTES // per_tile * 256
    assert L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_DECODE, cap_fit) <= P.PRHS_NOALLOC_SCRATCH_BYTES
    assert L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_DECODE, cap_fit + 1) > P.PRHS_NOALLOC_SCRATCH_BYTES
    assert call(d, cap=cap_fit + 1) == P.PRHS_E_WORKSPACE
    assert b"allocation-free" in L.prhs_last_error()
    big = _dims(batch=64, n_q_heads=64, n_kv_heads=8, kv_stride_b=8 * 1000 * 128)
    assert call(big, cap=8193) == P.PRHS_E_WORKSPACE    # past one workgroup per head: 64*64*33*130*4 bytes


def test_append_argument_checks(L):
    d = _dims()

    def app(dims, kn=FAKE, vn=FAKE, k=FAKE, v=FAKE, pos=5):
        return L.prhs_append_kv(ctypes.byref(dims) if dims is not None else None, kn, vn, k, v,
                                pos, None)
    assert app(None) == P.PRHS_E_NULL
    for kw in ("kn", "vn", "k", "v"):
        assert app(d, **{kw: None}) == P.PRHS_E_NULL, kw
        assert app(d, **{kw: FAKE_MIS}) == P.PRHS_E_ALIGN, kw
    assert app(d, pos=-1) == P.PRHS_E_DIMS
    assert app(d, pos=d.ctx_len) == P.PRHS_E_DIMS
    assert app(_dims(head_dim=96)) == P.PRHS_E_DIMS


def test_dense_argument_checks(L):
    d = _dims()
    need = L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_DENSE, 0)
    assert need == 2 * 8 * 4 * (128 + 2) * 4     # B*H_q*ceil(1000/256)*(d+2) floats
    assert _dense(L, None) == P.PRHS_E_NULL
    for kw in ("q", "k", "v", "out", "lse"):
        assert _dense(L, d, **{kw: None}) == P.PRHS_E_NULL, kw
    assert _dense(L, d, ws=None) == P.PRHS_E_WORKSPACE
    assert _dense(L, d, wsb=need - 1) == P.PRHS_E_WORKSPACE
    assert _dense(L, d, k=FAKE_MIS) == P.PRHS_E_ALIGN
    assert _dense(L, d, ws=FAKE_MIS) == P.PRHS_E_ALIGN


def _step(L, d, mode=P.PRHS_TOPN, n=64, dt=0.05, q=FAKE, k=FAKE, v=FAKE, s=FAKE, lse=FAKE,
          idx=FAKE, cap=64, cnt=FAKE, out=FAKE, lsel=FAKE, dl=FAKE, tau=FAKE, ws=FAKE, wsb=None,
          theta=None):
    if wsb is None:
        wsb = 1 << 30
    return L.prhs_anchor_step(ctypes.byref(d) if d is not None else None, mode, n, dt, q, k, v, s,
                              lse, idx, cap, cnt, None, out, lsel, dl, tau, theta, ws, wsb, None)


def test_anchor_step_argument_checks(L):
    d = _dims()
    need = L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_ANCHOR_STEP, 64)
    heads, nch = 2 * 8, (1000 + 255) // 256
    a256 = lambda x: (x + 255) // 256 * 256
    assert need == (a256(heads * nch * 8) + a256(heads * nch * 4) + a256(heads * nch * 256 * 8)
                    + a256(heads * 64 * 4) + heads * 1 * (128 + 2) * 4)
    assert _step(L, None) == P.PRHS_E_NULL
    assert _step(L, _dims(head_dim=96)) == P.PRHS_E_DIMS
    assert _step(L, _dims(ctx_len=P.PRHS_MAX_SELECT_CTX + 1, scores_ld=P.PRHS_MAX_SELECT_CTX + 4)) == P.PRHS_E_DIMS
    for kw in ("q", "k", "v", "s", "lse", "idx", "cnt", "out", "lsel"):
        assert _step(L, d, **{kw: None}) == P.PRHS_E_NULL, kw
    assert _step(L, d, dl=None) == P.PRHS_E_NULL            # tau without delta
    assert _step(L, d, v=FAKE_MIS) == P.PRHS_E_ALIGN
    assert _step(L, d, mode=9) == P.PRHS_E_BUDGET
    assert _step(L, d, n=0) == P.PRHS_E_BUDGET
    assert _step(L, d, mode=P.PRHS_DELTA, dt=2.0) == P.PRHS_E_BUDGET
    assert _step(L, d, n=65) == P.PRHS_E_CAPACITY
    assert _step(L, d, ws=None) == P.PRHS_E_WORKSPACE
    assert _step(L, d, wsb=need - 1) == P.PRHS_E_WORKSPACE
    assert _step(L, d, ws=FAKE_MIS) == P.PRHS_E_ALIGN


def _adaptive(L, d, n=64, r=2, force=0, tau=0.9, q=FAKE, k=FAKE, v=FAKE, s=FAKE, lse=FAKE,
              aidx=FAKE, acnt=FAKE, aq=FAKE, didx=FAKE, dcap=320, dcnt=FAKE, ref=FAKE, out=FAKE,
              lsel=FAKE, dl=FAKE, tau_out=FAKE, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = 1 << 30
    return L.prhs_adaptive_step(ctypes.byref(d) if d is not None else None, n, r, force, tau, q, k,
                                v, s, lse, aidx, acnt, aq, didx, dcap, dcnt, ref, None, out, lsel,
                                dl, tau_out, None, ws, wsb, None)


def test_adaptive_step_argument_checks(L):
    d = _dims()
    need = L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_ANCHOR_STEP, 320)
    assert _adaptive(L, None) == P.PRHS_E_NULL
    assert _adaptive(L, _dims(head_dim=96)) == P.PRHS_E_DIMS
    assert _adaptive(L, _dims(ctx_len=P.PRHS_MAX_SELECT_CTX + 1,
                              scores_ld=P.PRHS_MAX_SELECT_CTX + 4)) == P.PRHS_E_DIMS
    for kw in ("q", "k", "v", "s", "lse", "aidx", "acnt", "aq", "didx", "dcnt", "ref", "out", "lsel"):
        assert _adaptive(L, d, **{kw: None}) == P.PRHS_E_NULL, kw
    assert _adaptive(L, d, dl=None) == P.PRHS_E_NULL          # tau without delta
    assert _adaptive(L, d, s=FAKE_MIS) == P.PRHS_E_ALIGN
    assert _adaptive(L, d, n=0) == P.PRHS_E_BUDGET
    assert _adaptive(L, d, n=1001) == P.PRHS_E_BUDGET
    assert _adaptive(L, d, r=-1) == P.PRHS_E_BUDGET
    assert _adaptive(L, d, tau=math.nan) == P.PRHS_E_BUDGET
    assert _adaptive(L, d, dcap=319) == P.PRHS_E_CAPACITY      # (2r+1)*n = 320
    assert _adaptive(L, d, n=300, dcap=999) == P.PRHS_E_CAPACITY   # min(t, 1500) = 1000
    assert _adaptive(L, d, ws=None) == P.PRHS_E_WORKSPACE
    assert _adaptive(L, d, wsb=need - 1) == P.PRHS_E_WORKSPACE
    assert _adaptive(L, d, ws=FAKE_MIS) == P.PRHS_E_ALIGN


def _expand(L, d, aidx=FAKE, acap=64, acnt=FAKE, draws=FAKE, m=300, out=FAKE, ocap=300,
            ocnt=FAKE, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = 1 << 30
    return L.prhs_random_expand(ctypes.byref(d) if d is not None else None, aidx, acap, acnt,
                                draws, m, out, ocap, ocnt, ws, wsb, None)


def test_random_expand_argument_checks(L):
    d = _dims()
    need = L.prhs_workspace_bytes(ctypes.byref(d), P.PRHS_OP_EXPAND, 0)
    assert need == 2 * 8 * 1000 * 4               # B*H_q*scores_ld floats
    assert _expand(L, None) == P.PRHS_E_NULL
    for kw in ("aidx", "acnt", "draws", "out", "ocnt"):
        assert _expand(L, d, **{kw: None}) == P.PRHS_E_NULL, kw
    assert _expand(L, d, acap=0) == P.PRHS_E_CAPACITY
    assert _expand(L, d, m=63) == P.PRHS_E_BUDGET        # below anchor_cap
    assert _expand(L, d, m=1001, ocap=1001) == P.PRHS_E_BUDGET
    assert _expand(L, d, ocap=299) == P.PRHS_E_CAPACITY
    assert _expand(L, d, ws=None) == P.PRHS_E_WORKSPACE
    assert _expand(L, d, wsb=need - 4) == P.PRHS_E_WORKSPACE
    assert _expand(L, d, ws=FAKE_MIS) == P.PRHS_E_ALIGN


def test_status_strings(L):
    codes = [P.PRHS_OK, P.PRHS_E_NULL, P.PRHS_E_DIMS, P.PRHS_E_DTYPE, P.PRHS_E_BUDGET,
             P.PRHS_E_CAPACITY, P.PRHS_E_WORKSPACE, P.PRHS_E_HIP, P.PRHS_E_ALIGN]
    texts = [L.prhs_status_string(c) for c in codes]
    assert len(set(texts)) == len(codes)
    assert L.prhs_status_string(-99) == b"unknown status"


def test_python_binding_raises(L):
    d = _dims()
    with pytest.raises(P.PrhsError) as e:
        P.prhs_select_topk(d, FAKE, FAKE, P.PRHS_TOPN, 0, 0.0, FAKE, 64, FAKE, stream=0)
    assert e.value.code == P.PRHS_E_BUDGET
    assert "n_budget" in str(e.value)


def test_probe_argument_checks(L):
    sink = FAKE
    assert L.prhs_probe_stream_read(None, 64, sink, None) == P.PRHS_E_NULL
    assert L.prhs_probe_stream_read(FAKE, 64, None, None) == P.PRHS_E_NULL
    assert L.prhs_probe_stream_read(FAKE_MIS, 64, sink, None) == P.PRHS_E_ALIGN
    assert L.prhs_probe_stream_read(FAKE, 0, sink, None) == P.PRHS_E_DIMS
    assert L.prhs_probe_stream_read(FAKE, 40, sink, None) == P.PRHS_E_DIMS


def test_headers_compile_as_c(tmp_path):
    """The boundary is a plain C ABI: both headers compile as C99 (with the HIP
    runtime API header for hipStream_t) and the library links as C."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    rocm_inc = "/opt/rocm/include"
    if gcc is None or not os.path.isdir(rocm_inc):
        pytest.skip("gcc or the ROCm headers are not available")
    src = tmp_path / "use.c"
    src.write_text('#include "prhs.h"\n#include "prhs_probe.h"\n'
                   "int main(void) {\n"
                   "  prhs_dims d = {0};\n"
                   "  const char* s = prhs_status_string(prhs_score(&d, 0, 0, 0, 0, 0, 0, 0));\n"
                   "  return s == 0;\n}\n")
    inc = os.path.join(os.path.dirname(HEADER))
    libdir = os.path.dirname(P._LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{inc}",
                        f"-I{rocm_inc}", str(src), "-o", str(tmp_path / "use"), f"-L{libdir}",
                        "-lprhs", f"-Wl,-rpath,{libdir}", "-Wl,--allow-shlib-undefined"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
