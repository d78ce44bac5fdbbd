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
    q_norm_jitter: float = 0.0  # sigma of the per-step log-normal query-norm factor

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
    # Query norms vary by a log-normal factor (sigma 0.05) per step, for Fig. 8's
    # norm statistics of sharing pairs.
    "llama2_cis_8k": DecodeConfig("llama2_cis_8k", 8, 32, 32, 128, 8192, 512, 128, "f16", 1003,
                                  (32, 32), (4, 32), (1.5, 1.5), "step", 3.0,
                                  mode="cis", refresh_period=4, radius=2, q_norm_jitter=0.05),
    # The same with queries scaled by 3: attention concentrated enough that the
    # exact top-512 keeps about 97 % of the mass (the regime of Tables VI/VII).
    "llama2_cis_8k_sharp": DecodeConfig("llama2_cis_8k_sharp", 8, 32, 32, 128, 8192, 512, 128, "f16",
                                        1003, (32, 32), (4, 32), (1.5, 1.5), "step", 3.0,
                                        mode="cis", refresh_period=4, radius=2, q_norm_jitter=0.05,
                                        q_scale=(3.0, 3.0)),
    # Mistral-7B-shaped GQA: batch 4, 32 query heads on 8 KV heads, t=32768, N=2048, 32 steps.
    "mistral_gqa_32k": DecodeConfig("mistral_gqa_32k", 4, 32, 8, 128, 32768, 2048, 32, "f16", 1004,
                                    (256, 256), (8, 64), (1.5, 1.5), "step", 3.0),
    # Mistral-7B-shaped GQA at 128K context: batch 1, 32 query heads on 8 KV
    # heads, t=131072, N=2048, 16 steps (selection streams rows past 64K).
    "mistral_gqa_128k": DecodeConfig("mistral_gqa_128k", 1, 32, 8, 128, 131072, 2048, 16, "f16",
                                     1007, (1024, 1024), (8, 64), (1.5, 1.5), "step", 3.0),
    # GQA with 16 query heads per KV head: batch 2, 32 query heads on 2 KV
    # heads, t=32768, N=2048, 16 steps (the grouping one matrix-core scan
    # launch covers whole).
    "gqa16_32k": DecodeConfig("gqa16_32k", 2, 32, 2, 128, 32768, 2048, 16, "f16", 1006,
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
    q_scale: float = 1.0       # the drawn query scale of this layer
    bias: float = 0.0          # the drawn cluster bias of this layer
    n_clusters: int = 0        # the drawn cluster count per (b, h_kv)


def _layer_rng(cfg: DecodeConfig, layer: int):
    ss = np.random.SeedSequence(cfg.seed)
    if cfg.n_layers > 1:
        ss = ss.spawn(cfg.n_layers)[layer]
    return np.random.default_rng(ss)


def query_walk(cfg: DecodeConfig, rng, q_scale=1.0):
    """[steps, B, H_q, d] float64 correlated query walk (host). Each step keeps
    the direction of the last one plus noise; its norm is |q_0|, times
    exp(sigma * xi) with a fresh standard normal xi per step when
    cfg.q_norm_jitter = sigma > 0."""
    B, H, d, S = cfg.batch, cfg.n_q_heads, cfg.head_dim, cfg.steps
    q = np.empty((S, B, H, d), dtype=np.float64)
    q[0] = rng.standard_normal((B, H, d)) * q_scale
    norm0 = np.linalg.norm(q[0], axis=-1, keepdims=True)
    for s in range(1, S):
        x = q[s - 1] + 0.2 * q_scale * rng.standard_normal((B, H, d))
        norm = norm0
        if cfg.q_norm_jitter > 0.0:
            norm = norm0 * np.exp(cfg.q_norm_jitter * rng.standard_normal((B, H, 1)))
        q[s] = x / np.linalg.norm(x, axis=-1, keepdims=True) * norm
    return q


def _place_clusters(rng, t, rows, count, len_lo, len_hi):
    """For each of ``rows`` (b, g) pairs, ``count`` non-overlapping runs in
    [N_SINKS, t): lengths uniform in [len_lo, len_hi], then the free rows cut
    into count + 1 gaps at uniformly drawn points (every ordered arrangement of
    those lengths is equally likely; runs may touch). Runs that would not fit
    are dropped from the end. Returns (row, start, length) int64 arrays."""
    span = t - N_SINKS
    L = rng.integers(len_lo, len_hi + 1, size=(rows, count))
    keep = np.cumsum(L, axis=1) <= span
    L = np.where(keep, L, 0)
    free = span - L.sum(axis=1)
    cuts = np.sort(rng.integers(0, free[:, None] + 1, size=(rows, count)), axis=1)
    starts = N_SINKS + cuts + np.cumsum(L, axis=1) - L
    r, c = np.nonzero(keep)
    return r, starts[r, c], L[r, c]


def _layer_head(cfg: DecodeConfig, rng):
    """The first draws of a layer's stream: query scale, query walk, cluster
    bias and cluster count."""
    q_scale = float(rng.uniform(*cfg.q_scale)) if cfg.q_scale[0] != cfg.q_scale[1] else cfg.q_scale[0]
    qw = query_walk(cfg, rng, q_scale)
    bias = cfg.bias[0] if cfg.bias[0] == cfg.bias[1] else float(rng.uniform(*cfg.bias))
    n_cl = int(rng.integers(cfg.n_clusters[0], cfg.n_clusters[1] + 1))
    return q_scale, qw, bias, n_cl


def layer_draws(cfg: DecodeConfig, layer: int):
    """(query scale, cluster bias, cluster count) that make_workload draws for
    ``layer``, computed on the host without building the layer."""
    q_scale, _, bias, n_cl = _layer_head(cfg, _layer_rng(cfg, layer))
    return q_scale, bias, n_cl


def make_workload(cfg: DecodeConfig, device="cpu", layer: int = 0) -> Workload:
    """Build one layer's q walk, K and V for ``cfg`` on ``device``."""
    rng = _layer_rng(cfg, layer)
    B, Hq, Hkv, d, t = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ctx_len
    G = cfg.group
    q_scale, qw, bias, n_cl = _layer_head(cfg, rng)

    # Per (b, g): cluster runs, owners and target steps; per-row bias vectors.
    row, start, L = _place_clusters(rng, t, B * Hkv, n_cl, *cfg.cluster_len)
    b_of, g_of = row // Hkv, row % Hkv
    owner = g_of * G + rng.integers(0, G, size=row.size)
    step = (np.zeros(row.size, dtype=np.int64) if cfg.bias_target == "q0"
            else rng.integers(0, cfg.steps, size=row.size))
    plan_arr = np.stack([b_of, g_of, start, L, owner, step], axis=1).astype(np.int64)
    seeds = rng.integers(0, 2**62, size=2 * B)

    dev = torch.device(device)
    K = torch.empty((B, Hkv, t, d), dtype=cfg.torch_dtype, device=dev)
    V = torch.empty((B, Hkv, t, d), dtype=cfg.torch_dtype, device=dev)
    unit = qw / np.linalg.norm(qw, axis=-1, keepdims=True)
    unit_dev = torch.as_tensor(unit, dtype=torch.float32, device=dev)
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
    plan = [tuple(r) for r in plan_arr.tolist()]
    return Workload(cfg, layer, q.contiguous(), K, V, plan, q_scale, bias, n_cl)


def expansion_draws(batch, n_heads, t, seed, device="cpu", bits=23):
    """Random integers [batch, n_heads, t] (int32, below 2**bits) for the
    RandomExpansion control: its random choice is an input, so that every
    implementation makes the same choice. Seeded torch.Generator on ``device``."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    return torch.randint(0, 1 << bits, (batch, n_heads, t), generator=g, device=dev,
                         dtype=torch.int32)

