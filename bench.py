"""Benchmark of the multi-LoRA adapted linear layer on one MI355X.

One step = one mlora_linear call (base product, per-token LoRA shrink and expand, accumulate
and round) over the decode workload: T = 64 one-token requests through a 4096 -> 4096 bf16
layer with 100 resident rank-16 adapters (alpha 32), 6 tokens on the base model only.
Inputs are resident in HBM before the timed region; the step cycles through enough distinct
copies of {x, W, A, B, y} (over twice the 256 MB Infinity Cache) that every step's bytes come
from HBM.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
METRIC = "multi-LoRA layer tokens/s + % HBM GB/s (decode) / % MFMA peak (prefill)"


def algorithmic(L):
    """Bytes and flops the method itself must move / compute for one call: W, x, y once, each
    distinct used adapter's A and B rows once at its true rank, the index map and scales."""
    import numpy as np
    used = np.unique(L.idx[L.idx >= 0])
    adapter = sum(int(L.rank[a]) * (L.n_slices * L.n_in + L.n_out) * 2 for a in used)
    a_only = sum(int(L.rank[a]) * L.n_slices * L.n_in * 2 for a in used)
    base = L.n_out * L.n_in * 2 + L.T * L.n_in * 2 + L.T * L.n_out * 2
    meta = L.idx.size * 4 + L.scale.size * 4 + L.S * 4
    flops = 2.0 * L.T * L.n_in * L.n_out
    for t in range(L.T):
        for j in range(L.K):
            a = L.idx[t, j]
            if a >= 0:
                flops += 2.0 * int(L.rank[a]) * (L.n_slices * L.n_in + L.n_out)
    return {"bytes": base + adapter + meta, "adapter_bytes": adapter, "a_bytes": a_only,
            "W_bytes": L.n_out * L.n_in * 2, "x_bytes": L.T * L.n_in * 2,
            "distinct_adapters": int(len(used)), "flops": flops}


def cpu_baseline(L, budget_s: float):
    """The oracle, as it stands, on the host cores: whole batches until budget_s has passed."""
    import oracle
    oracle.build(force=False)
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.linear(L)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": n * L.T / el, "unit": "tokens/s", "cores": min(cores, threads),
            "kind": "oracle",
            "sample": f"{n} full batches of the same {L.T}-token workload ({n * L.T} tokens, "
                      f"{el:.1f} s, fp64 oracle, OpenMP over tokens)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--sets", type=int, default=0, help="rotating input copies (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the layer shards without communication; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    from lora_serving_amd import mlora, synth
    from tests.gpu_util import DevLayer

    L = synth.workload_decode()
    alg = algorithmic(L)
    D = DevLayer(L)
    per_set = (D.x.numel() + D.W.numel() + D.A.numel() + D.B.numel()) * 2 + L.T * L.n_out * 2
    nsets = args.sets or max(2, -(-600 * 2 ** 20 // per_set))
    sets = []
    for i in range(nsets):
        if i == 0:
            x, W, A, B = D.x, D.W, D.A, D.B
        else:
            x, W, A, B = D.x.clone(), D.W.clone(), D.A.clone(), D.B.clone()
        slots = mlora.Slots(A, B, D.factor, slice_start=[int(v) for v in L.slice_start])
        y = torch.empty((L.T, L.n_out), dtype=torch.bfloat16, device="cuda")
        sets.append((x, W, slots, y))
    idx, scale, ws = D.idx, D.scale, D.ws

    def step(i):
        x, W, slots, y = sets[i % nsets]
        mlora.mlora_linear(x, W, slots, idx, scale, y, ws=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()     # the stream the library launches on

    # timed region: K steps back to back, one event pair around all of them
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    tokens_per_s = L.T / (ms * 1e-3)
    achieved = alg["bytes"] / (ms * 1e-3) / 1e9

    out = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random bf16 weights and adapters)",
        "config": {"workload": "bgmv_decode: T=64 one-token requests, 4096->4096 bf16, "
                               "100 adapters rank 16 alpha 32, 6 tokens base-only, K=1",
                   "T": L.T, "n_in": L.n_in, "n_out": L.n_out, "S": L.S, "R": L.R, "K": L.K,
                   "distinct_adapters": alg["distinct_adapters"], "rotating_sets": nsets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "scope": "whole step (all kernels of the layer)",
                     "algorithmic_bytes": alg["bytes"]},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(L, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
