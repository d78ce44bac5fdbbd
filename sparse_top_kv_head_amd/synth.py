"""Seeded synthetic decode workloads (inputs only; none of the method's arithmetic).

The pages time and evaluate PrHS on real models (LLaMA2-7B, Mistral-7B,
Qwen) over datasets that are not available here. These generators stand in
for them with random KV caches of the same layer shapes and with the structure
the pages report in attention (page "Near-Oracle KV Selection via Pre-hoc
Sparsity for Long-Context Inference"):

* critical keys form contiguous clusters that persist over adjacent queries
  (Fig. 2, Fig. 11) -- planted here by adding a bias along a query direction
  to a run of keys;
* adjacent decode queries of a head are highly similar (Fig. 2 uses cosine
  above 0.8; Fig. 10 shows the similarity concentrated at high values) -- the
  query walk q_{s+1} = normalize(q_s + 0.2 eps) * |q_0| gives about 0.97;
* a few leading sink keys take large weight (StreamingLLM is in the pages'
  reference list) -- keys 0..3 get a larger bias.

Everything is deterministic in the seed. Host-side draws (queries, cluster
positions, biases) use numpy's PCG64; the K/V noise is drawn with a seeded
``torch.Generator`` on the device that will hold the tensors, so the same seed
gives the same structure but device-dependent noise. Consumers that need exact
values (the oracle) always read the stored tensors back.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int
    budget: int                 # TOPN budget N, or the cap in delta mode
    steps: int
    dtype: str                  # "f32" or "f16": storage type of q, K and V
    seed: int
    n_clusters: tuple           # (lo, hi) inclusive, per KV head
    cluster_len: tuple          # (lo, hi) inclusive
    bias: tuple                 # (lo, hi) uniform; lo == hi for a fixed bias
    bias_target: str            # "q0": toward the step-0 query; "step": toward a drawn step's query
    sink_bias: float            # 0 disables the 4 sink keys
    mode: str = "topn"          # "topn", "cis" or "delta"
    refresh_period: int = 1     # CIS: exact retrieval every this many steps
    radius: int = 0             # CIS: dilation radius
    delta_star: float = 0.05    # delta mode target
    n_layers: int = 1           # independent KV caches (delta config)
    q_scale: tuple = (1.0, 1.0)  # per-layer query scale range (the "sharp" variant)

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.float16

    @property
    def elem_bytes(self):
        return 4 if self.dtype == "f32" else 2

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


N_SINKS = 4

CONFIGS = {
    # Toy decode: one layer, 4 MHA heads, d=64, fp32, t=512, N=64, 8 steps.
    "toy": DecodeConfig("toy", 1, 4, 4, 64, 512, 64, 8, "f32", 1001,
                        (6, 6), (8, 8), (2.0, 2.0), "q0", 0.0),
    # LLaMA2-7B-shaped layer: 32 MHA heads, d=128, fp16, t=4096, N=256, 64 steps.
    "llama2_4k": DecodeConfig("llama2_4k", 1, 32, 32, 128, 4096, 256, 64, "f16", 1002,
                              (32, 32), (4, 32), (1.5, 1.5), "step", 3.0),
    # LLaMA2-7B-shaped CIS reuse: batch 8, t=8192, N=512, 128 steps,
    # exact retrieval every 4th step, +-2 dilation otherwise.
    "llama2_cis_8k": DecodeConfig("llama2_cis_8k", 8, 32, 32, 128, 8192, 512, 128, "f16", 1003,
                                  (32, 32), (4, 32), (1.5, 1.5), "step", 3.0,
                                  mode="cis", refresh_period=4, radius=2),
    # Mistral-7B-shaped GQA: batch 4, 32 query heads on 8 KV heads, t=32768, N=2048, 32 steps.
    "mistral_gqa_32k": DecodeConfig("mistral_gqa_32k", 4, 32, 8, 128, 32768, 2048, 32, "f16", 1004,
                                    (256, 256), (8, 64), (1.5, 1.5), "step", 3.0),
    # Delta-budgeted 32-layer decode: batch 16, 32 MHA heads, t=16384,
    # smallest N with delta <= 0.05, capped at 2048, 16 steps.
    "delta_16k": DecodeConfig("delta_16k", 16, 32, 32, 128, 16384, 2048, 16, "f16", 1005,
                              (64, 512), (4, 32), (0.5, 2.0), "step", 3.0,
                              mode="delta", delta_star=0.05, n_layers=32),
}


@dataclass
class Workload:
    cfg: DecodeConfig
    layer: int
    q: torch.Tensor            # [steps, B, H_q, d] storage dtype
    K: torch.Tensor            # [B, H_kv, t, d]
    V: torch.Tensor            # [B, H_kv, t, d]
    clusters: list = field(default_factory=list)  # (b, g, start, length, owner_h, target_step)


def _layer_rng(cfg: DecodeConfig, layer: int):
    ss = np.random.SeedSequence(cfg.seed)
    if cfg.n_layers > 1:
        ss = ss.spawn(cfg.n_layers)[layer]
    return np.random.default_rng(ss)


def query_walk(cfg: DecodeConfig, rng, q_scale=1.0):
    """[steps, B, H_q, d] float64 correlated query walk (host)."""
    B, H, d, S = cfg.batch, cfg.n_q_heads, cfg.head_dim, cfg.steps
    q = np.empty((S, B, H, d), dtype=np.float64)
    q[0] = rng.standard_normal((B, H, d)) * q_scale
    norm0 = np.linalg.norm(q[0], axis=-1, keepdims=True)
    for s in range(1, S):
        x = q[s - 1] + 0.2 * q_scale * rng.standard_normal((B, H, d))
        q[s] = x / np.linalg.norm(x, axis=-1, keepdims=True) * norm0
    return q


def _place_clusters(rng, t, count, len_lo, len_hi):
    """Non-overlapping runs with starts uniform in [N_SINKS, t - L]."""
    taken = np.zeros(t, dtype=bool)
    out = []
    attempts = 0
    while len(out) < count and attempts < 50 * count + 100:
        attempts += 1
        L = int(rng.integers(len_lo, len_hi + 1))
        if t - L < N_SINKS:
            continue
        start = int(rng.integers(N_SINKS, t - L + 1))
        if taken[start:start + L].any():
            continue
        taken[start:start + L] = True
        out.append((start, L))
    return out


def layer_q_scale(cfg: DecodeConfig, layer: int) -> float:
    """The query scale make_workload draws for ``layer`` (the first draw of its stream)."""
    if cfg.q_scale[0] == cfg.q_scale[1]:
        return cfg.q_scale[0]
    return float(_layer_rng(cfg, layer).uniform(*cfg.q_scale))


def make_workload(cfg: DecodeConfig, device="cpu", layer: int = 0) -> Workload:
    """Build one layer's q walk, K and V for ``cfg`` on ``device``."""
    rng = _layer_rng(cfg, layer)
    B, Hq, Hkv, d, t = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ctx_len
    G = cfg.group
    q_scale = float(rng.uniform(*cfg.q_scale)) if cfg.q_scale[0] != cfg.q_scale[1] else cfg.q_scale[0]
    qw = query_walk(cfg, rng, q_scale)
    if cfg.bias[0] == cfg.bias[1]:
        bias = cfg.bias[0]
    else:
        bias = float(rng.uniform(*cfg.bias))
    n_lo, n_hi = cfg.n_clusters
    n_cl = int(rng.integers(n_lo, n_hi + 1))

    # Per (b, g): cluster runs, owners and target steps; per-row bias vectors.
    plan = []
    for b in range(B):
        for g in range(Hkv):
            runs = _place_clusters(rng, t, n_cl, *cfg.cluster_len)
            for (start, L) in runs:
                owner = g * G + int(rng.integers(0, G))
                step = 0 if cfg.bias_target == "q0" else int(rng.integers(0, cfg.steps))
                plan.append((b, g, start, L, owner, step))
    seeds = rng.integers(0, 2**62, size=2 * B)

    dev = torch.device(device)
    K = torch.empty((B, Hkv, t, d), dtype=cfg.torch_dtype, device=dev)
    V = torch.empty((B, Hkv, t, d), dtype=cfg.torch_dtype, device=dev)
    unit = qw / np.linalg.norm(qw, axis=-1, keepdims=True)
    unit_dev = torch.as_tensor(unit, dtype=torch.float32, device=dev)
    plan_arr = np.asarray(plan, dtype=np.int64).reshape(-1, 6)
    for b in range(B):
        gk = torch.Generator(device=dev)
        gk.manual_seed(int(seeds[2 * b]))
        gv = torch.Generator(device=dev)
        gv.manual_seed(int(seeds[2 * b + 1]))
        kb = torch.randn((Hkv, t, d), generator=gk, device=dev, dtype=torch.float32)
        vb = torch.randn((Hkv, t, d), generator=gv, device=dev, dtype=torch.float32)
        if cfg.sink_bias != 0.0:
            for g in range(Hkv):
                mean_dir = unit[0, b, g * G:(g + 1) * G].mean(axis=0)
                mean_dir = mean_dir / np.linalg.norm(mean_dir)
                kb[g, :N_SINKS] += torch.as_tensor(cfg.sink_bias * mean_dir, dtype=torch.float32, device=dev)
        mine = plan_arr[plan_arr[:, 0] == b]
        if len(mine):
            lens = mine[:, 3]
            rep = np.repeat(np.arange(len(mine)), lens)
            within = np.arange(rep.size) - np.repeat(np.cumsum(lens) - lens, lens)
            rows = mine[rep, 1] * t + mine[rep, 2] + within
            owner = torch.as_tensor(mine[rep, 4], device=dev)
            step = torch.as_tensor(mine[rep, 5], device=dev)
            vecs = unit_dev[step, b, owner] * bias
            kb.view(-1, d).index_add_(0, torch.as_tensor(rows, device=dev), vecs)
        K[b] = kb.to(cfg.torch_dtype)
        V[b] = vb.to(cfg.torch_dtype)
        del kb, vb
    q = torch.as_tensor(qw, dtype=cfg.torch_dtype).to(dev)
    return Workload(cfg, layer, q.contiguous(), K, V, plan)


def expansion_draws(batch, n_heads, t, seed, device="cpu", bits=23):
    """Random integers [batch, n_heads, t] (int32, below 2**bits) for the
    RandomExpansion control: its random choice is an input, so that every
    implementation makes the same choice. Seeded torch.Generator on ``device``."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    return torch.randint(0, 1 << bits, (batch, n_heads, t), generator=g, device=dev,
                         dtype=torch.int32)

