"""Decode-step driver over the C ABI: owns the per-step buffers and enqueues
score -> select -> sparse decode (anchor steps), dilate -> sparse decode (CIS
reuse steps) on one stream. Buffers are allocated once; a step allocates
nothing.
"""

from __future__ import annotations

import torch

from . import prhs as P


class DecodeEngine:
    """Buffers and calls for one layer shape.

    K, V layout [B, H_kv, t, d]; q [B, H_q, d]; index capacity ``cap`` per head
    (TOPN budget, DELTA cap, or the dilated size of a reused set). ``dense``
    sizes the workspace for dense_step as well.
    """

    def __init__(self, K: torch.Tensor, n_q_heads: int, cap: int, device=None, dense=False):
        self.dims = P.make_dims(K, n_q_heads)
        d = self.dims
        self._capacity = d.ctx_len
        dev = device or K.device
        self.nheads = d.batch * d.n_q_heads
        self.cap = cap
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.scores = torch.empty((d.batch, d.n_q_heads, d.scores_ld), **f32)
        self.lse_all = torch.empty((d.batch, d.n_q_heads), **f32)
        self.idx = torch.empty((d.batch, d.n_q_heads, cap), **i32)
        self.count = torch.empty((d.batch, d.n_q_heads), **i32)
        self.cap_hit = torch.empty((d.batch, d.n_q_heads), **i32)
        self.out = torch.empty((d.batch, d.n_q_heads, d.head_dim), **f32)
        self.lse_sel = torch.empty((d.batch, d.n_q_heads), **f32)
        self.delta = torch.empty((d.batch, d.n_q_heads), **f32)
        self.tau = torch.empty((d.batch, d.n_q_heads), **f32)
        self.reuse_ok = torch.empty((d.batch, d.n_q_heads), **i32)
        self.sel_scores = torch.empty((d.batch, d.n_q_heads, cap), **f32)
        # per-head score threshold hint carried from one anchor step to the next
        self.theta = torch.full((d.batch, d.n_q_heads), float("nan"), **f32)
        ws = max(P.prhs_workspace_bytes(d, P.PRHS_OP_SCORE),
                 P.prhs_workspace_bytes(d, P.PRHS_OP_DECODE, cap),
                 P.prhs_workspace_bytes(d, P.PRHS_OP_ANCHOR_STEP, cap),
                 P.prhs_workspace_bytes(d, P.PRHS_OP_DENSE) if dense else 0)
        self.ws = torch.empty(((ws + 15) // 16 * 16,), dtype=torch.uint8, device=dev)

    @property
    def capacity(self):
        """Largest context length the buffers hold (the K/V tensor the engine was built on)."""
        return self._capacity

    def set_ctx_len(self, t):
        """Attend over the first t keys of the cache from now on (a growing cache:
        t = t0 + step). Buffers and the workspace are sized for the capacity."""
        if not 1 <= t <= self._capacity:
            raise ValueError(f"ctx_len {t} outside [1, {self._capacity}]")
        self.dims.ctx_len = t

    def score(self, q, K, stream=None):
        P.prhs_score(self.dims, q, K, self.scores, self.lse_all, self.ws, stream=stream)

    def select(self, mode, n_budget, delta_target=0.0, stream=None):
        P.prhs_select_topk(self.dims, self.scores, self.lse_all, mode, n_budget, delta_target,
                           self.idx, self.cap, self.count, self.cap_hit, self.sel_scores,
                           stream=stream)

    def decode(self, q, K, V, use_scores=True, idx=None, count=None, cap=None, stream=None):
        idx = self.idx if idx is None else idx
        count = self.count if count is None else count
        cap = self.cap if cap is None else cap
        P.prhs_sparse_decode(self.dims, q, K, V, idx, cap, count,
                             self.scores if use_scores else None,
                             self.lse_all if use_scores else None, self.out, self.lse_sel,
                             self.delta if use_scores else None, self.tau if use_scores else None,
                             self.ws, stream=stream)

    def anchor_step(self, q, K, V, mode, n_budget, delta_target=0.0, stream=None, hint=True):
        """One fused call: score scan, selection, sparse attention with delta/tau.

        hint: carry the per-head threshold hint between anchor steps (TOPN).
        """
        P.prhs_anchor_step(self.dims, mode, n_budget, delta_target, q, K, V, self.scores,
                           self.lse_all, self.idx, self.cap, self.count, self.cap_hit, self.out,
                           self.lse_sel, self.delta, self.tau, self.theta if hint else None,
                           self.ws, stream=stream)

    def topn_step(self, q, K, V, N, stream=None):
        """Anchor step: exact top-N over fresh scores, then attention over it."""
        self.anchor_step(q, K, V, P.PRHS_TOPN, N, stream=stream)

    def delta_step(self, q, K, V, cap, delta_target, stream=None):
        """Smallest set with dropped mass <= delta_target (capped), then attention."""
        self.anchor_step(q, K, V, P.PRHS_DELTA, cap, delta_target, stream=stream)

    def reuse_step(self, q, K, V, anchor_idx, anchor_count, anchor_cap, radius,
                   q_anchor=None, sim_tau=0.0, stream=None):
        """CIS reuse step: dilate the anchor's set, then attend with gathered K and V rows
        (one call; with q_anchor, the dilation call also evaluates the similarity gate)."""
        if q_anchor is None:
            P.prhs_reuse_step(self.dims, anchor_idx, anchor_cap, anchor_count, radius, q, K, V,
                              self.idx, self.cap, self.count, self.out, self.lse_sel, self.ws,
                              stream=stream)
            return
        P.prhs_cis_reuse(self.dims, anchor_idx, anchor_cap, anchor_count, radius, q, q_anchor,
                         sim_tau, self.idx, self.cap, self.count, self.reuse_ok, stream=stream)
        self.decode(q, K, V, use_scores=False, stream=stream)

    def append_kv(self, k_new, v_new, K, V, pos, stream=None):
        """Growing cache: write one step's K and V rows (contiguous [B, H_kv, d])
        into row ``pos`` of the cache (pos < the current ctx_len)."""
        P.prhs_append_kv(self.dims, k_new, v_new, K, V, pos, stream=stream)

    def dense_step(self, q, K, V, stream=None):
        """Dense attention over every key (the baseline): out and lse_all."""
        P.prhs_dense_decode(self.dims, q, K, V, self.out, self.lse_all, self.ws, stream=stream)

    def dropped_mass(self, stream=None):
        P.prhs_dropped_mass(self.dims, self.lse_sel, self.lse_all, self.delta, self.tau, stream=stream)

    def capture(self, steps, mode, n_budget, delta_target=0.0):
        """Capture a sequence of anchor steps [(q, K, V), ...] into one HIP graph.

        The graph replays the same kernels on the same buffers; inputs must stay
        at the captured addresses. Returns the torch CUDAGraph (call .replay()).
        """
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for (q, K, V) in steps:
                self.anchor_step(q, K, V, mode, n_budget, delta_target)
        return g


class AdaptiveEngine:
    """Critical-index-set sharing with a per-head similarity gate, one call per step.

    Every ``period``-th step refreshes every head; in between, a head reuses its
    anchor set (dilated by ``radius``) while the cosine of its query with its
    anchor query stays at or above ``sim_tau``, and refreshes otherwise. The
    anchor sets and anchor queries live on the device across steps; the
    per-step decisions come back in ``refresh`` (1 = exact retrieval this step).
    """

    def __init__(self, K: torch.Tensor, n_q_heads: int, n_budget: int, radius: int, period: int,
                 sim_tau: float, hint=True):
        self.dims = P.make_dims(K, n_q_heads)
        d = self.dims
        dev = K.device
        self.n_budget, self.radius, self.period, self.sim_tau = n_budget, radius, period, sim_tau
        self.dil_cap = min(d.ctx_len, (2 * radius + 1) * n_budget)
        B, H = d.batch, d.n_q_heads
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.scores = torch.empty((B, H, d.scores_ld), **f32)
        self.lse_all = torch.empty((B, H), **f32)
        self.anchor_idx = torch.empty((B, H, n_budget), **i32)
        self.anchor_count = torch.zeros((B, H), **i32)
        self.anchor_q = torch.zeros((B, H, d.head_dim), dtype=K.dtype, device=dev)
        self.dil_idx = torch.empty((B, H, self.dil_cap), **i32)
        self.dil_count = torch.zeros((B, H), **i32)
        self.refresh = torch.zeros((B, H), **i32)
        self.sim = torch.empty((B, H), **f32)
        self.out = torch.empty((B, H, d.head_dim), **f32)
        self.lse_sel = torch.empty((B, H), **f32)
        self.delta = torch.empty((B, H), **f32)
        self.tau = torch.empty((B, H), **f32)
        self.theta = torch.full((B, H), float("nan"), **f32) if hint else None
        ws = P.prhs_workspace_bytes(d, P.PRHS_OP_ANCHOR_STEP, self.dil_cap)
        self.ws = torch.empty(((ws + 15) // 16 * 16,), dtype=torch.uint8, device=dev)
        self.step_no = 0

    def step(self, q, K, V, stream=None):
        force = self.step_no % self.period == 0
        P.prhs_adaptive_step(self.dims, self.n_budget, self.radius, force, self.sim_tau, q, K, V,
                             self.scores, self.lse_all, self.anchor_idx, self.anchor_count,
                             self.anchor_q, self.dil_idx, self.dil_cap, self.dil_count,
                             self.refresh, self.sim, self.out, self.lse_sel, self.delta, self.tau,
                             self.theta, self.ws, stream=stream)
        self.step_no += 1
