"""ctypes binding of libprhs.so: the C ABI declared in include/prhs.h.

Argument marshalling only. Every computation runs in the library's HIP
kernels; torch tensors serve as device memory and torch's current stream as
the HIP stream. The functions carry the C names and signatures; tensors (or
None for NULL) stand in for pointers. A nonzero status raises PrhsError.

Loading fails loudly when the library has not been built: there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch

# PRHS_LIB names another build of the same library (the sanitizer build)
_LIB_PATH = os.environ.get("PRHS_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                       "libprhs.so")

PRHS_OK = 0
PRHS_E_NULL = -1
PRHS_E_DIMS = -2
PRHS_E_DTYPE = -3
PRHS_E_BUDGET = -4
PRHS_E_CAPACITY = -5
PRHS_E_WORKSPACE = -6
PRHS_E_HIP = -7
PRHS_E_ALIGN = -8

PRHS_F32 = 0
PRHS_F16 = 1
PRHS_TOPN = 0
PRHS_DELTA = 1
PRHS_OP_SCORE = 0
PRHS_OP_SELECT = 1
PRHS_OP_DECODE = 2
PRHS_OP_ANCHOR_STEP = 3
PRHS_OP_DENSE = 4
PRHS_OP_EXPAND = 5
PRHS_MAX_SELECT_CTX = 262144
PRHS_NOALLOC_SCRATCH_BYTES = 4 << 20

EXPORTED = (
    "prhs_score", "prhs_select_topk", "prhs_cis_reuse", "prhs_reuse_step", "prhs_sparse_decode",
    "prhs_sparse_decode_noalloc", "prhs_dropped_mass", "prhs_anchor_step", "prhs_adaptive_step",
    "prhs_dense_decode", "prhs_random_expand", "prhs_append_kv", "prhs_workspace_bytes",
    "prhs_status_string", "prhs_last_error",
)
# measurement aid (include/prhs_probe.h)
PROBE_EXPORTED = ("prhs_probe_stream_read",)


class PrhsDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("ctx_len", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("kv_stride_b", ctypes.c_int64),
        ("kv_stride_h", ctypes.c_int64),
        ("kv_stride_t", ctypes.c_int64),
        ("scores_ld", ctypes.c_int32),
    ]


class PrhsError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"PrHS error {code}: {message}")
        self.code = code


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m sparse_top_kv_head_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        dp = ctypes.POINTER(PrhsDims)
        L.prhs_score.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp]
        L.prhs_select_topk.argtypes = [dp, vp, vp, i32, i32, f32, vp, i32, vp, vp, vp, vp]
        L.prhs_cis_reuse.argtypes = [dp, vp, i32, vp, i32, vp, vp, f32, vp, i32, vp, vp, vp]
        L.prhs_reuse_step.argtypes = [dp, vp, i32, vp, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                      sz, vp]
        L.prhs_sparse_decode.argtypes = [dp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         sz, vp]
        L.prhs_sparse_decode_noalloc.argtypes = [dp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                                 vp, vp, vp]
        L.prhs_dropped_mass.argtypes = [dp, vp, vp, vp, vp, vp]
        L.prhs_anchor_step.argtypes = [dp, i32, i32, f32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                       vp, vp, vp, vp, vp, sz, vp]
        L.prhs_dense_decode.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.prhs_random_expand.argtypes = [dp, vp, i32, vp, vp, i32, vp, i32, vp, vp, sz, vp]
        L.prhs_append_kv.argtypes = [dp, vp, vp, vp, vp, i32, vp]
        L.prhs_adaptive_step.argtypes = [dp, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.prhs_probe_stream_read.argtypes = [vp, sz, vp, vp]
        L.prhs_probe_stream_read.restype = ctypes.c_int
        L.prhs_workspace_bytes.argtypes = [dp, i32, i32]
        L.prhs_workspace_bytes.restype = sz
        L.prhs_status_string.argtypes = [ctypes.c_int]
        L.prhs_status_string.restype = ctypes.c_char_p
        L.prhs_last_error.argtypes = []
        L.prhs_last_error.restype = ctypes.c_char_p
        for name in ("prhs_score", "prhs_select_topk", "prhs_cis_reuse", "prhs_reuse_step",
                     "prhs_sparse_decode", "prhs_sparse_decode_noalloc",
                     "prhs_dropped_mass", "prhs_anchor_step", "prhs_dense_decode",
                     "prhs_adaptive_step", "prhs_random_expand", "prhs_append_kv"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(x):
    """Tensor -> device address; int -> itself; None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != PRHS_OK:
        L = lib()
        detail = L.prhs_last_error().decode()
        raise PrhsError(status, f"{L.prhs_status_string(status).decode()}: {detail}")


def make_dims(K: torch.Tensor, n_q_heads: int, scores_ld: int | None = None) -> PrhsDims:
    """Dims for a KV tensor [B, H_kv, t, d] (any strides with a contiguous d axis)."""
    B, Hkv, t, d = K.shape
    if K.stride(3) != 1:
        raise ValueError("the head_dim axis of K must be contiguous")
    dtype = {torch.float32: PRHS_F32, torch.float16: PRHS_F16}.get(K.dtype)
    if dtype is None:
        raise ValueError(f"unsupported dtype {K.dtype}")
    if scores_ld is None:
        scores_ld = (t + 3) // 4 * 4
    return PrhsDims(B, n_q_heads, Hkv, d, t, dtype, K.stride(0), K.stride(1), K.stride(2), scores_ld)


def prhs_workspace_bytes(dims: PrhsDims, op: int, cap: int = 0) -> int:
    return int(lib().prhs_workspace_bytes(ctypes.byref(dims), op, cap))


def alloc_workspace(dims, op, cap=0, device="cuda"):
    """A workspace of the size `op` needs (16-byte aligned)."""
    n = prhs_workspace_bytes(dims, op, cap)
    return torch.empty(((n + 15) // 16 * 16,), dtype=torch.uint8, device=device)


def prhs_status_string(status: int) -> str:
    return lib().prhs_status_string(status).decode()


def prhs_score(dims, q, k, scores, lse_all=None, ws=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(lib().prhs_score(ctypes.byref(dims), _p(q), _p(k), _p(scores), _p(lse_all), _p(ws),
                            ws_bytes, _stream(stream)))


def prhs_select_topk(dims, scores, lse_all, mode, n_budget, delta_target, idx, idx_cap, count,
                     cap_hit=None, sel_scores=None, stream=None):
    _check(lib().prhs_select_topk(ctypes.byref(dims), _p(scores), _p(lse_all), mode, n_budget,
                                  delta_target, _p(idx), idx_cap, _p(count), _p(cap_hit),
                                  _p(sel_scores), _stream(stream)))


def prhs_cis_reuse(dims, anchor_idx, anchor_cap, anchor_count, radius, q_cur, q_anchor, sim_tau,
                   out_idx, out_cap, out_count, reuse_ok=None, stream=None):
    _check(lib().prhs_cis_reuse(ctypes.byref(dims), _p(anchor_idx), anchor_cap, _p(anchor_count),
                                radius, _p(q_cur), _p(q_anchor), sim_tau, _p(out_idx), out_cap,
                                _p(out_count), _p(reuse_ok), _stream(stream)))


def prhs_reuse_step(dims, anchor_idx, anchor_cap, anchor_count, radius, q, k, v, out_idx, out_cap,
                    out_count, out, lse_sel, ws=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(lib().prhs_reuse_step(ctypes.byref(dims), _p(anchor_idx), anchor_cap, _p(anchor_count),
                                 radius, _p(q), _p(k), _p(v), _p(out_idx), out_cap, _p(out_count),
                                 _p(out), _p(lse_sel), _p(ws), ws_bytes, _stream(stream)))


def prhs_sparse_decode(dims, q, k, v, idx, idx_cap, count, scores, lse_all, out, lse_sel,
                       delta=None, tau=None, ws=None, ws_bytes=None, sel_scores=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(lib().prhs_sparse_decode(ctypes.byref(dims), _p(q), _p(k), _p(v), _p(idx), idx_cap,
                                    _p(count), _p(sel_scores), _p(scores), _p(lse_all), _p(out),
                                    _p(lse_sel), _p(delta), _p(tau), _p(ws), ws_bytes,
                                    _stream(stream)))


def prhs_sparse_decode_noalloc(dims, q, k, v, idx, idx_cap, count, scores, lse_all, out, lse_sel,
                               delta=None, tau=None, sel_scores=None, stream=None):
    _check(lib().prhs_sparse_decode_noalloc(ctypes.byref(dims), _p(q), _p(k), _p(v), _p(idx),
                                            idx_cap, _p(count), _p(sel_scores), _p(scores),
                                            _p(lse_all), _p(out), _p(lse_sel), _p(delta), _p(tau),
                                            _stream(stream)))


def prhs_dropped_mass(dims, lse_sel, lse_all, delta, tau=None, stream=None):
    _check(lib().prhs_dropped_mass(ctypes.byref(dims), _p(lse_sel), _p(lse_all), _p(delta),
                                   _p(tau), _stream(stream)))


def prhs_adaptive_step(dims, n_budget, radius, force_refresh, sim_tau, q, k, v, scores, lse_all,
                       anchor_idx, anchor_count, anchor_q, dil_idx, dil_cap, dil_count, refresh,
                       sim, out, lse_sel, delta=None, tau=None, theta=None, ws=None, ws_bytes=None,
                       stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(lib().prhs_adaptive_step(ctypes.byref(dims), n_budget, radius, int(bool(force_refresh)),
                                    sim_tau, _p(q), _p(k), _p(v), _p(scores), _p(lse_all),
                                    _p(anchor_idx), _p(anchor_count), _p(anchor_q), _p(dil_idx),
                                    dil_cap, _p(dil_count), _p(refresh), _p(sim), _p(out),
                                    _p(lse_sel), _p(delta), _p(tau), _p(theta), _p(ws), ws_bytes,
                                    _stream(stream)))


def prhs_random_expand(dims, anchor_idx, anchor_cap, anchor_count, draws, m, out_idx, out_cap,
                       out_count, ws=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(lib().prhs_random_expand(ctypes.byref(dims), _p(anchor_idx), anchor_cap,
                                    _p(anchor_count), _p(draws), m, _p(out_idx), out_cap,
                                    _p(out_count), _p(ws), ws_bytes, _stream(stream)))


def prhs_dense_decode(dims, q, k, v, out, lse, ws=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(lib().prhs_dense_decode(ctypes.byref(dims), _p(q), _p(k), _p(v), _p(out), _p(lse),
                                   _p(ws), ws_bytes, _stream(stream)))


def prhs_append_kv(dims, k_new, v_new, k, v, pos, stream=None):
    _check(lib().prhs_append_kv(ctypes.byref(dims), _p(k_new), _p(v_new), _p(k), _p(v), pos,
                                _stream(stream)))


def prhs_anchor_step(dims, mode, n_budget, delta_target, q, k, v, scores, lse_all, idx, idx_cap,
                     count, cap_hit, out, lse_sel, delta=None, tau=None, theta=None, ws=None,
                     ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else 0
    _check(lib().prhs_anchor_step(ctypes.byref(dims), mode, n_budget, delta_target, _p(q), _p(k),
                                  _p(v), _p(scores), _p(lse_all), _p(idx), idx_cap, _p(count),
                                  _p(cap_hit), _p(out), _p(lse_sel), _p(delta), _p(tau),
                                  _p(theta), _p(ws), ws_bytes, _stream(stream)))


def prhs_probe_stream_read(buf, sink, nbytes=None, stream=None):
    """Read every byte of `buf` once (HBM read-ceiling probe)."""
    if nbytes is None:
        nbytes = buf.numel() * buf.element_size()
    _check(lib().prhs_probe_stream_read(_p(buf), nbytes, _p(sink), _stream(stream)))
