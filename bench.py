"""Sparse-decode benchmark of the PrHS hot path on one MI355X.

One step = one pass of the whole hot path over one decode query batch:
score (K scan) -> exact top-N select -> sparse attention over the selected
rows with the fused dropped mass, on the Mistral-7B-shaped GQA layer with a
32K context (batch 4, 32 query heads on 8 KV heads, d = 128, fp16, N = 2048).

Prints one JSON line. ``value`` is heads*steps/s over the timed steps with
inputs resident in HBM; the timed steps are captured once as a HIP graph and
replayed (the eager per-call rate is reported beside it). Independent copies of K and V are rotated so that no
step finds its KV cache in the 256 MB Infinity Cache left by the previous
one. ``roofline`` reports the scan kernel (the dominant kernel): algorithmic
bytes (the K cache it must read) over its mean duration from HIP events on
the launch stream. ``cpu_baseline`` times the fp64 numpy oracle on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "score_scan_mistral_gqa_32k_hbm_traffic.md")
SCAN_SOURCES = ["sparse_top_kv_head_amd/csrc/score.hip", "sparse_top_kv_head_amd/csrc/prhs_device.hpp",
                "sparse_top_kv_head_amd/csrc/prhs_launch.hpp"]


def scan_traffic_bytes():
    """HBM bytes per scan launch from the committed counter profile, or None when
    the scan kernel's sources changed since the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    rec = dict(line.split(": ", 1) for line in text.splitlines()
               if line.startswith(("scan_traffic_bytes_per_launch:", "scan_source_hash:")))
    h = hashlib.sha256()
    for f in SCAN_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if rec.get("scan_source_hash", "").strip() != h.hexdigest()[:16]:
        return None
    return float(rec["scan_traffic_bytes_per_launch"])


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="mistral_gqa_32k")
    ap.add_argument("--rotate", type=int, default=4, help="independent KV copies cycled over steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (for scaling HBM byte counters)")
    return ap.parse_args()


def cpu_baseline(w, n_steps, budget_s):
    """Time the fp64 oracle on a bounded sample of the workload (heads of the first steps)."""
    from oracle import prhs_oracle as O
    cfg = w.cfg
    K = w.K.double().cpu().numpy()
    V = w.V.double().cpu().numpy()
    q = w.q.double().cpu().numpy()
    heads = [(b, h) for b in range(cfg.batch) for h in range(cfg.n_q_heads)]
    done = 0
    t0 = time.perf_counter()
    s = 0
    while time.perf_counter() - t0 < budget_s:
        for (b, h) in heads:
            O.decode_step(q[s % n_steps], K, V, "topn", N=cfg.budget, heads=[(b, h)])
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        s += 1
    el = time.perf_counter() - t0
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        pass
    return {"value": done / el, "unit": "heads*steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} (head, step) oracle passes (score+top-{cfg.budget}+attention+delta, fp64) "
                      f"of the {cfg.name} workload in {el:.1f} s"}


def main():
    a = _parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the path shards by "
              f"(batch, KV head) with no communication, so N GPUs run N independent copies.",
              file=sys.stderr)
        sys.exit(2)
    from sparse_top_kv_head_amd import prhs as P
    from sparse_top_kv_head_amd.engine import DecodeEngine
    from sparse_top_kv_head_amd.synth import CONFIGS, make_workload

    P.lib()
    dev = torch.device("cuda:0")
    cfg = CONFIGS[a.config]
    w = make_workload(cfg, device=dev)
    Ks = [w.K] + [w.K.clone() for _ in range(a.rotate - 1)]
    Vs = [w.V] + [w.V.clone() for _ in range(a.rotate - 1)]
    eng = DecodeEngine(w.K, cfg.n_q_heads, cfg.budget)
    stream = torch.cuda.current_stream()
    N = cfg.budget

    def step(i):
        r = i % a.rotate
        eng.anchor_step(w.q[i % cfg.steps], Ks[r], Vs[r], P.PRHS_TOPN, N)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    # Eager: one library call per step (host launch overhead included).
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(a.steps):
        step(a.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    eager_ms = ev0.elapsed_time(ev1)

    # Timed: the same K steps captured once as a HIP graph and replayed, so the
    # kernels run back to back without host launch gaps.
    seq = [(w.q[(a.warmup + i) % cfg.steps], Ks[(a.warmup + i) % a.rotate], Vs[(a.warmup + i) % a.rotate])
           for i in range(a.steps)]
    graph = eng.capture(seq, P.PRHS_TOPN, N)
    graph.replay()  # one untimed replay
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev0.elapsed_time(ev1)

    # The scan kernel alone, same inputs and launch configuration as inside the
    # step (per-chunk partials on, no separate log-sum-exp merge): K launches
    # back to back between two events on the launch stream.
    part = P.alloc_workspace(eng.dims, P.PRHS_OP_SCORE, device=dev)
    ev0.record(stream)
    for i in range(a.steps):
        P.prhs_score(eng.dims, w.q[i % cfg.steps], Ks[i % a.rotate], eng.scores, None, part, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    scan_ms = np.array([ev0.elapsed_time(ev1) / a.steps])

    B, Hq, Hkv, d, t, eb = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ctx_len, cfg.elem_bytes
    heads = B * Hq
    value = heads * a.steps / (total_ms / 1e3)
    scan_bytes = B * Hkv * t * d * eb
    # distinct V rows per (b, kv head) selected at the last timed step (algorithmic gather bytes)
    idx = eng.idx.cpu().numpy()
    cnt = eng.count.cpu().numpy()
    G = Hq // Hkv
    rows = 0
    for b in range(B):
        for g in range(Hkv):
            rows += np.unique(np.concatenate([idx[b, h, :cnt[b, h]] for h in range(g * G, (g + 1) * G)])).size
    step_bytes = scan_bytes + rows * d * eb
    scan_gbs = scan_bytes / (scan_ms.mean() / 1e3) / 1e9
    traffic_bytes = scan_traffic_bytes()
    traffic = None if traffic_bytes is None else round(traffic_bytes / (scan_ms.mean() / 1e3) / 1e9, 1)
    res = {
        "metric": "sparse decode attn heads*steps/s at 32K ctx + achieved HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "heads*steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(total_ms / a.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: Mistral-7B-shaped GQA decode layer, B={B}, H_q={Hq}, "
                               f"H_kv={Hkv}, d={d}, t={t}, top-N={N}, fp16 K/V",
                   "batch": B, "ctx_len": t, "budget": N, "kv_copies_rotated": a.rotate},
        "roofline": {"bound": "hbm", "kernel": "score_scan_kernel<__half,128,4,256,16> (K scan GEMV, timed in its own loop)",
                     "achieved": round(scan_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(scan_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_bytes_per_launch": traffic_bytes,
                     "algorithmic_bytes_per_launch": scan_bytes,
                     "mean_launch_ms": round(float(scan_ms.mean()), 5)},
        "step": {"hbm_alg_bytes": int(step_bytes), "hbm_alg_gbs": round(step_bytes / (total_ms / a.steps / 1e3) / 1e9, 1),
                 "frac_of_peak": round(step_bytes / (total_ms / a.steps / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "eager_ms_per_step": round(eager_ms / a.steps, 5),
                 "scan_ms_p50": round(float(np.median(scan_ms)), 5),
                 "mean_selected_rows_per_head": float(cnt.mean()),
                 "wall_s": round(wall, 4)},
    }
    if a.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["calibration_copy_bytes"] = src.numel()
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, cfg.steps, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
