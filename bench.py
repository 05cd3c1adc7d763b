"""Benchmark of the multi-LoRA adapted linear layer on one MI355X.

One step = one mlora_linear call per layer of the workload (base product, LoRA shrink and
expand, accumulate and round y once).  The headline workload is the decode batch: T = 64
one-token requests through a 4096 -> 4096 bf16 layer with 100 resident rank-16 adapters
(alpha 32), 6 tokens on the base model only.  Inputs are resident in HBM before the timed
region; when one copy of the inputs fits the 256 MB Infinity Cache, the step cycles through
enough distinct copies of {x, W, A, B, y} (over 600 MB) that every step's bytes come from HBM.

Prints one JSON line.  Besides the headline workload it carries a `configs` list with one
entry per other workload (tiny, prefill, mixed_qkv, compose), each timed the same way in the
same process: ms per step, tokens/s, the main product kernel's event-timed duration and its
fraction of the HBM or MFMA roofline, and the CPU oracle's rate on a bounded sample.

Workloads (--workload): tiny, decode, prefill (16384 tokens, 4096 -> 11008, 100 x rank 64),
mixed_qkv (256 decode + 2048 prefill tokens, merged QKV 4096 -> 6144, ranks 8/16/64 padded to
64), compose (8192 tokens, K = 3 slots, 4096 -> 4096 and 11008 -> 4096 layers), decode256,
lm_head (the decode batch on a 4096 -> 100,000 vocabulary projection).
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
METRIC_BGMV = "BGMV shrink + expand tokens/s + % HBM GB/s (the standalone mlora_shrink / mlora_expand pair)"
METRIC_PLAN = "mapping plan tokens/s + % HBM GB/s (mlora_plan: stable sort of the (token, slot) pairs by slot)"

DESCRIPTIONS = {
    "tiny": "tiny: T=16, 256->256, 4 adapters rank 8 alpha 16, P(-1)=0.25, K=1",
    "decode": "bgmv_decode: T=64 one-token requests, 4096->4096 bf16, 100 adapters rank 16 "
              "alpha 32, 6 tokens base-only, K=1",
    "prefill": "sgmv_prefill: T=16384 = 32 requests x 512 contiguous tokens, 4096->11008 bf16, "
               "100 adapters rank 64 alpha 128, request adapter ~ Zipf(1.1), K=1",
    "mixed_qkv": "mixed_qkv: T=2304 = 256 decode + 2048 prefill tokens, merged QKV "
                 "4096->(4096,1024,1024), 64 adapters ranks {8,16,64} padded to 64, alpha 2r",
    "compose": "k3_compose: T=8192 = 64 requests x 128 tokens, K=3 slots, 32 adapters rank 16 "
               "alpha 32 (half rsLoRA), s~U(0.2,1); layers 4096->4096 and 11008->4096",
    "decode256": "decode256: T=256 one-token requests, 4096->4096 bf16, 100 adapters rank 16 "
                 "alpha 32, 26 tokens base-only, K=1",
    "lm_head": "lm_head: T=64 one-token requests, 4096->100000 (vocabulary) bf16, 100 adapters "
               "rank 16 alpha 32, 6 tokens base-only, K=1",
    "mixed_qkv_decode": "mixed_qkv_decode: the mixed batch's 256 one-token requests alone, merged "
                        "QKV 4096->(4096,1024,1024), 64 adapters ranks {8,16,64} padded to 64",
    "decode_tp8_col": "decode_tp8_col: one GPU's share of the decode layer under 8-way column "
                      "parallelism, 4096->512 (its rows of W and B), T=64, 100 adapters rank 16",
    "decode_tp8_row": "decode_tp8_row: one GPU's share of the decode layer under 8-way row "
                      "parallelism, 512->4096 (its columns of W, A, x), T=64, 100 adapters rank 16",
}
# the workloads of the `configs` list, in this order, when the headline is the decode batch
CONFIG_ORDER = ["tiny", "prefill", "mixed_qkv", "compose"]


def algorithmic(L):
    """Bytes and flops the method itself must move / compute for one call of the layer: W, x, y
    once, each distinct used adapter's A and B rows once at its true rank, the index map and
    scales; flops 2 T n_in n_out plus 2 r (n_slices n_in + n_out) per used (token, slot)."""
    import numpy as np
    used = np.unique(L.idx[L.idx >= 0])
    a_bytes = sum(int(L.rank[a]) * L.n_slices * L.n_in * 2 for a in used)
    b_bytes = sum(int(L.rank[a]) * L.n_out * 2 for a in used)
    w_bytes = L.n_out * L.n_in * 2
    x_bytes = L.T * L.n_in * 2
    y_bytes = L.T * L.n_out * 2
    meta = L.idx.size * 4 + L.scale.size * 4 + L.S * 4
    ranks = np.where(L.idx >= 0, L.rank[np.maximum(L.idx, 0)], 0).astype(np.float64)
    base_flops = 2.0 * L.T * L.n_in * L.n_out
    shrink_flops = float(np.sum(2.0 * ranks * L.n_slices * L.n_in))
    expand_flops = float(np.sum(2.0 * ranks * L.n_out))
    return {"bytes": w_bytes + x_bytes + y_bytes + a_bytes + b_bytes + meta,
            "flops": base_flops + shrink_flops + expand_flops,
            "distinct_adapters": int(len(used)),
            # the part of the call done by the main product kernel, per path
            "decode_kernel_bytes": w_bytes + x_bytes + a_bytes + meta,
            "grouped_kernel_bytes": w_bytes + x_bytes,         # the decode GEMM on the base alone
            "decode_kernel_flops": base_flops + shrink_flops,
            "tiled_kernel_bytes": w_bytes + x_bytes + y_bytes + b_bytes + meta,
            "tiled_kernel_flops": base_flops + expand_flops,
            # the standalone pair: shrink reads x and A, writes v; expand reads v, B and y and
            # writes y (v is fp32 [K][T][n_slices R])
            "shrink_bytes": x_bytes + a_bytes + L.K * L.T * L.n_slices * L.R * 4 + meta,
            "expand_bytes": 2 * y_bytes + b_bytes + L.K * L.T * L.n_slices * L.R * 4 + meta,
            "bgmv_flops": shrink_flops + expand_flops}


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the counter summary committed under
    profiles/ (FETCH_SIZE and WRITE_SIZE runs, calibrated with a plain copy kernel), or None when
    there is none or the kernel's sources changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md"))):
        fields = {}
        for line in open(path):
            line = line.strip()
            if line.startswith("traffic_") and ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        if fields.get("traffic_kernel") != kernel:
            continue
        if fields.get("traffic_workload", "decode") != workload:
            continue
        h = hashlib.sha256()
        for f in fields.get("traffic_sources", "").split():
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != fields.get("traffic_sources_sha256"):
            return None
        return float(fields["traffic_bytes_per_launch"])
    return None


def measured_ceilings(roof):
    """Ceilings measured in the same process, next to the datasheet peaks: a plain device copy
    (bytes read + written per second) and a large bf16 GEMM through torch.matmul (hipBLASLt);
    plus the main kernel's achieved figure as a fraction of the matching one."""
    import torch
    n = 2 ** 28                                  # 1 GiB of fp32, 4x the Infinity Cache
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * n * 4 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(m, m, dtype=torch.bfloat16, device="cuda").t().contiguous()
    for _ in range(2):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2.0 * m ** 3 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    probe = copy_gbps if roof["unit"] == "GB/s" else gemm_tf
    return {"copy_GBps": copy_gbps, "gemm_bf16_TFLOPs": gemm_tf,
            "gemm_shape": [m, m, m], "achieved_over_probe": roof["achieved"] / probe}


def host_info():
    """Core counts and CPU model of the host the CPU baseline runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "cpu_model": model}


def cpu_baseline(layers, budget_s: float, with_base: bool = True):
    """The oracle's plain fp32 loop (the same C source built with fp32 sums), as it stands, on
    the host cores, on a bounded sample of the workload's tokens (whole batches while they
    take under the budget, else random 32-token samples per layer), scaled to tokens/s; without
    the base product for the shrink/expand pair."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    total_tokens = sum(L.T for L in layers) / len(layers)
    t0 = time.perf_counter()
    n_tok = 0
    rounds = 0
    rng = np.random.default_rng(0)
    while True:
        for L in layers:
            if L.T <= 128:
                oracle.linear(L, with_base=with_base, acc="f32")
                n_tok += L.T / len(layers)
            else:
                toks = np.sort(rng.choice(L.T, size=32, replace=False))
                oracle.linear(L, tokens=toks, with_base=with_base, acc="f32")
                n_tok += 32 / len(layers)
        rounds += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    hi = host_info()
    threads = int(hi["omp_num_threads"] or hi["affinity_cores"])
    what = ("full batches" if all(L.T <= 128 for L in layers)
            else "random 32-token samples per layer")
    out = {"value": n_tok / el, "unit": "tokens/s", "cores": min(hi["affinity_cores"], threads),
           "kind": "oracle",
           "sample": f"{rounds} rounds of {what} of the same workload ({n_tok:.0f} tokens of "
                     f"{total_tokens:.0f} per step, {el:.1f} s, fp32-accumulate build of the "
                     f"oracle, OpenMP over tokens)",
           "precision": "fp32 sums (oracle.c built with -DORACLE_ACC=float); parity uses the "
                        "fp64 build"}
    out.update(hi)
    return out


def cpu_baseline_plan(L, budget_s: float):
    """The oracle's plan (a plain stable counting sort in C, one thread) on the host, repeated
    on the batch's whole index map until the budget is spent, scaled to tokens/s."""
    import oracle
    oracle.build(force=False)
    t0 = time.perf_counter()
    rounds = 0
    while True:
        oracle.plan(L.idx, L.S)
        rounds += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    out = {"value": rounds * L.T / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": f"{rounds} plans of the whole index map ({L.T} tokens x {L.K} slots, "
                     f"{el:.1f} s, one thread)"}
    out.update(host_info())
    return out


class Prepared:
    """Device inputs of one workload (rotating copies for decode-sized steps) and one step of
    the chosen operation over them."""

    def __init__(self, name, op="linear", w_layout="auto", sets=0, flags=0):
        import torch
        from lora_serving_amd import mlora, synth
        from lora_serving_amd.device import DevLayer
        self.name, self.op = name, op
        layers = synth.WORKLOADS[name]()
        self.layers = layers if isinstance(layers, list) else [layers]
        self.decode_like = all(L.T <= 512 for L in self.layers)
        if op in ("bgmv", "plan"):
            w_layout = "unused"                      # neither reads the base weight
        elif w_layout == "auto":
            w_layout = "packed" if self.decode_like else "rowmajor"
        self.w_layout = w_layout
        self.algs = [algorithmic(L) for L in self.layers]
        self.devs = [DevLayer(L) for L in self.layers]
        # the kernels mlora_linear runs for each layer (the library's own host-side choice)
        names = {mlora.MLORA_PATH_DECODE: "decode", mlora.MLORA_PATH_TILED: "tiled",
                 mlora.MLORA_PATH_GROUPED: "grouped"}
        self.paths = [names.get(mlora.mlora_linear_path(D.L.T, D.L.n_in, D.L.n_out, D.slots,
                                                        D.L.K, flags), "?")
                      for D in self.devs]
        # rotating copies so that decode-sized steps read HBM, not the Infinity Cache (a
        # workload under 1 MB is latency-bound and keeps one copy)
        per_set = sum((D.x.numel() + D.W.numel() + D.A.numel() + D.B.numel()) * 2 +
                      D.L.T * D.L.n_out * 2 for D in self.devs)
        if sets:
            nsets = sets
        elif per_set < 2 ** 20 or per_set >= 256 * 2 ** 20:
            nsets = 1
        else:
            nsets = max(2, -(-600 * 2 ** 20 // per_set))
        if op == "plan":
            nsets = 1                                # reads only the index map
            L0 = self.layers[0]
            i32 = lambda n: torch.empty((max(n, 1),), dtype=torch.int32, device="cuda")
            self.plan_out = (i32(L0.T * L0.K), i32(L0.S), i32(L0.S), i32(L0.S), i32(2))
        self.nsets = nsets
        self.sets = []
        for i in range(nsets):
            one = []
            for D in self.devs:
                if i == 0:
                    x, W, A, B = D.x, D.W, D.A, D.B
                else:
                    x, W, A, B = D.x.clone(), D.W.clone(), D.A.clone(), D.B.clone()
                slots = mlora.Slots(A, B, D.factor,
                                    slice_start=[int(v) for v in D.L.slice_start], rank=D.rank)
                y = torch.zeros((D.L.T, D.L.n_out), dtype=torch.bfloat16, device="cuda")
                if w_layout == "packed" and op == "linear":
                    W = mlora.mlora_pack_weight(W)
                v = (torch.empty((D.L.K, D.L.T, D.L.n_slices * D.L.R), dtype=torch.float32,
                                 device="cuda") if op == "bgmv" else None)
                one.append((x, W, slots, y, D, v))
            self.sets.append(one)
        self.flags = flags | (mlora.MLORA_W_PACKED if w_layout == "packed" else 0)
        self.mlora = mlora

    def step(self, i, only_layer=None):
        m = self.mlora
        for li, (x, W, slots, y, D, v) in enumerate(self.sets[i % self.nsets]):
            if only_layer is not None and li != only_layer:
                continue
            if self.op == "plan":
                m.mlora_plan(D.idx, D.L.S, *self.plan_out, D.ws)
                break                                # one plan per batch
            elif self.op == "bgmv":
                m.mlora_shrink(x, slots, D.idx, D.scale, v, ws=D.ws)
                m.mlora_expand(v, slots, D.idx, y)
            else:
                m.mlora_linear(x, W, slots, D.idx, D.scale, y, flags=self.flags, ws=D.ws)

    def launches_per_step(self, only_layer=None):
        """Launches of the traced kernel(s) per step."""
        if self.op == "plan":
            return 1                                 # the sort kernels, traced as one region
        layers = self.layers if only_layer is None else [self.layers[only_layer]]
        if self.op == "bgmv":
            return 2 * len(layers)                   # shrink, expand
        return sum((L.T + 511) // 512 if self.decode_like else 1 for L in layers)


def plan_form(pairs, slots):
    """The sort the library runs for a map of this size (one wave, one workgroup, or three
    kernels), by the same limits as its launcher."""
    if pairs <= 512 and slots <= 1000:
        return "sort_wave, one launch"
    if pairs <= 8192 and slots <= 1000:
        return "sort_small, one launch"
    return "sort_count + sort_scan + sort_scatter, one region"


_SLEEP_CYCLES_PER_US = None


def gpu_busy(us: float):
    """Keeps the GPU busy for about `us` microseconds (torch's spin kernel), so that the host can
    enqueue the timed steps before the first of them starts."""
    global _SLEEP_CYCLES_PER_US
    import torch
    if _SLEEP_CYCLES_PER_US is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)                      # load the kernel before timing it
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_US = 1_000_000 / max(e0.elapsed_time(e1) * 1e3, 1.0)
    torch.cuda._sleep(int(us * _SLEEP_CYCLES_PER_US))


def time_steps(P: Prepared, steps: int, warmup: int, graph: bool = False, only_layer=None):
    """ms per step over exactly `steps` timed steps (HIP events on the launch stream), after
    `warmup` untimed steps and one untimed pass over every rotating input set, bracketed by
    torch.cuda.synchronize() on both sides.  Between the first synchronize and the opening
    event a spin kernel keeps the GPU busy while the host enqueues the steps, so the region
    holds the steps' device time and not the host's launch latency."""
    import torch
    for i in range(warmup):
        P.step(i, only_layer)
    for i in range(P.nsets):                         # every input set touched once
        P.step(i, only_layer)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()             # the stream the library launches on
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        # whole passes over the input sets, at least 16 steps (a replay costs several
        # microseconds of its own), captured once after a warm-up pass on a side stream, as
        # capture asks; the timed region replays it, so steps round up to whole replays
        per_graph = P.nsets * -(-16 // P.nsets)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(per_graph):
                P.step(i, only_layer)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per_graph):
                P.step(i, only_layer)
        torch.cuda.synchronize()
        reps = -(-steps // per_graph)
        steps = reps * per_graph
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        gpu_busy(2000)
        ev0.record(stream)
        for _ in range(reps):
            g.replay()
        ev1.record(stream)
    else:
        gpu_busy(min(20000.0, 500.0 + 30.0 * steps))
        ev0.record(stream)
        for i in range(steps):
            P.step(i, only_layer)
        ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, steps


def trace_kernel(P: Prepared, steps: int, only_layer=None):
    """Durations (ms) of the main product kernel's launches over `steps` more steps, from the
    HIP event pairs the library records on its launch stream around each launch (the pairs add
    a little time per launch, so the step time is taken without them)."""
    import torch
    m = P.mlora
    cap = steps * P.launches_per_step(only_layer)
    torch.cuda.synchronize()
    m.mlora_trace_start(cap)
    gpu_busy(min(20000.0, 500.0 + 40.0 * steps))     # no host gap inside the first pairs
    for i in range(steps):
        P.step(i, only_layer)
    torch.cuda.synchronize()
    ks = m.mlora_trace_stop(cap)
    if len(ks) != cap:
        raise RuntimeError(f"expected {cap} traced launches, got {len(ks)}")
    return ks


def decode_gemm_name(T, n_in, n_out, n_cus=256):
    """Name of the decode GEMM kernel the library launches for one launch of up to 512 tokens:
    the persistent grid (decode_gemm_ps_kernel) when there are many more (chunk, tile, split)
    items than CUs, by the same conditions as the library's launcher (label only)."""
    Tc = min(T, 512)
    n_tiles = -(-n_out // 64)
    wblocks = -(-n_in // 128)
    n_chunks = -(-Tc // 64)
    per = 8
    while per > 4 and n_chunks * n_tiles * (-(-wblocks // per)) < n_cus:
        per //= 2
    sk = -(-n_in // (per * 128))
    if n_chunks > 1:
        n_lanes = 8 * ((n_cus // 8) // n_chunks) // sk
        ps = n_lanes >= 1 and n_tiles >= 2 * n_lanes
    else:
        ps = n_tiles * sk > n_cus and sk <= n_cus
    return "mlora::decode_gemm_ps_kernel" if ps else "mlora::decode_gemm_kernel"


def decode_shrink_apart(T, K, n_out, wd):
    """Whether the decode path runs the shrink apart from its GEMM (the per-pair kernel ahead of
    a GEMM of the base alone), by the same condition as the library's decode_shrink_apart: a
    64-row tile gets 2 or more (token, slot) pairs of a 64-token chunk and 4 or more 16-row
    pieces of them (8 with several chunks) (label and byte count only)."""
    n_tiles = -(-n_out // 64)
    pairs = -(-(min(T, 64) * K) // n_tiles)
    pieces = pairs * -(-wd // 16)
    return pairs >= 2 and pieces >= (8 if T > 64 else 4)


def linear_roofline(P: Prepared, kernel_ms, only_layer=None):
    """Roofline object of the main product kernel of mlora_linear: the decode GEMM against HBM
    (algorithmic bytes per launch) or the tiled GEMM against the bf16 MFMA peak (algorithmic
    flops per launch)."""
    idxs = range(len(P.layers)) if only_layer is None else [only_layer]
    algs = [P.algs[i] for i in idxs]
    k_avg_ms = sum(kernel_ms) / len(kernel_ms)
    per_step = P.launches_per_step(only_layer)
    if P.decode_like:
        paths = [P.paths[i] for i in idxs]
        # the GEMM reads the adapters' A rows only where the shrink rides in its pass
        lora = not (P.flags & P.mlora.MLORA_NO_ADAPTERS)
        base_only = [p == "grouped" or (p == "decode" and lora and
                                        decode_shrink_apart(P.layers[i].T, P.layers[i].K,
                                                            P.layers[i].n_out,
                                                            P.layers[i].n_slices * P.layers[i].R))
                     for i, p in zip(idxs, paths)]
        k_bytes = sum(a["grouped_kernel_bytes" if b else "decode_kernel_bytes"]
                      for a, b in zip(algs, base_only)) / per_step
        achieved = k_bytes / (k_avg_ms * 1e-3) / 1e9
        if all(p == "grouped" for p in paths):
            what = "base product (grouped decode: the LoRA terms in the group kernels)"
        elif all(base_only):
            what = "base product (the shrink apart, in shrink_rows_kernel)"
        else:
            what = "base product + LoRA shrink"
        import torch
        L0 = P.layers[idxs[0]]
        n_cus = torch.cuda.get_device_properties(0).multi_processor_count
        return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                "kernel": f"{decode_gemm_name(L0.T, L0.n_in, L0.n_out, n_cus)} ({what})",
                "kernel_avg_us": k_avg_ms * 1e3, "algorithmic_bytes_per_launch": k_bytes}
    k_flops = sum(a["tiled_kernel_flops"] for a in algs) / per_step
    achieved = k_flops / (k_avg_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
            "kernel": "mlora::prefill_gemm_kernel (base product + LoRA expand as extra K-steps)",
            "kernel_avg_us": k_avg_ms * 1e3, "algorithmic_flops_per_launch": k_flops}


def binding(nbytes, nflops, ms):
    """A call against both roofs: its algorithmic bytes at the HBM peak and flops at the bf16
    MFMA peak, as times, and the longer of the two over the measured time."""
    t_b = nbytes / (HBM_PEAK_GBPS * 1e9)
    t_f = nflops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return {"t_bytes_us": t_b * 1e6, "t_flops_us": t_f * 1e6,
            "bound": "hbm" if t_b >= t_f else "mfma", "frac": max(t_b, t_f) / (ms * 1e-3)}


def part_layer(L, sl):
    """The tokens sl of layer L as a layer of their own (for the algorithmic work of a part)."""
    import dataclasses
    return dataclasses.replace(L, T=sl.stop - sl.start, x=L.x[sl], idx=L.idx[sl],
                               scale=L.scale[sl], segments=[])


def config_entry(name, steps, warmup, cpu_s, with_cpu, graph=False):
    """One entry of the `configs` list: the workload's mlora_linear step timed like the
    headline, its main kernel's roofline, per-layer or per-part times where the workload has
    them, and the CPU oracle's rate."""
    import torch
    P = Prepared(name)
    ms, steps_done = time_steps(P, steps, warmup, graph=graph)
    ks = trace_kernel(P, steps_done)
    roof = linear_roofline(P, ks)
    # HBM bytes per launch from a committed counter summary of this kernel on this workload,
    # while its sources are unchanged (else null)
    roof["traffic"] = committed_traffic(roof["kernel"].split()[0].split("::")[-1], name)
    T = P.layers[0].T
    tot_bytes = sum(a["bytes"] for a in P.algs)
    tot_flops = sum(a["flops"] for a in P.algs)
    e = {"workload": DESCRIPTIONS[name], "name": name, "T": T,
         "layers": [[L.n_in, L.n_out] for L in P.layers],
         "distinct_adapters": [a["distinct_adapters"] for a in P.algs],
         "steps": steps_done, "warmup": warmup, "rotating_sets": P.nsets,
         "w_layout": P.w_layout, "path": P.paths, "ms_per_step": ms,
         "tokens_per_s": T / (ms * 1e-3),
         "roofline": roof,
         "step_algorithmic": {"bytes": tot_bytes, "flops": tot_flops},
         "step_achieved": {"GBps": tot_bytes / (ms * 1e-3) / 1e9,
                           "TFLOPs": tot_flops / (ms * 1e-3) / 1e12},
         # the step against both roofs: the longer of its bytes at 8 TB/s and its flops at the
         # bf16 MFMA peak, over the measured step time
         "step_binding": binding(tot_bytes, tot_flops, ms)}
    if name == "tiny":
        e["roofline"]["note"] = ("latency-bound (about 0.2 MB and 2 MFLOP per call, far below "
                                 "both roofs): reported, no roofline claim")
    if len(P.layers) > 1:
        # each layer timed alone, the same way
        per = []
        for li, L in enumerate(P.layers):
            lms, _ = time_steps(P, steps, 1, only_layer=li)
            lks = trace_kernel(P, steps, only_layer=li)
            lr = linear_roofline(P, lks, only_layer=li)
            per.append({"n_in": L.n_in, "n_out": L.n_out, "ms_per_call": lms,
                        "tokens_per_s": L.T / (lms * 1e-3), "kernel_avg_us": lr["kernel_avg_us"],
                        "kernel_frac": lr["frac"], "kernel_bound": lr["bound"]})
        e["per_layer"] = per
    if name == "mixed_qkv":
        # the batch's two parts run alone through mlora_linear (each takes the path the
        # library picks for it): the 256 one-token requests and the 2048-token segment
        m = P.mlora
        (x, W, slots, y, D, _v) = P.sets[0][0]
        L = D.L
        nd = sum(1 for (_s, n) in L.segments if n == 1)
        parts = {}
        for pname, sl in (("decode_part", slice(0, nd)), ("prefill_part", slice(nd, L.T))):
            xs, ids, scs, ys = x[sl], D.idx[sl], D.scale[sl], y[sl]

            def run():
                m.mlora_linear(xs, W, slots, ids, scs, ys, flags=P.flags, ws=D.ws)
            for _ in range(max(warmup, 2)):
                run()
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gpu_busy(500.0 + 30.0 * steps)
            ev0.record()
            for _ in range(steps):
                run()
            ev1.record()
            torch.cuda.synchronize()
            pms = ev0.elapsed_time(ev1) / steps
            Lp = part_layer(L, sl)
            ap = algorithmic(Lp)
            parts[pname] = {"T": sl.stop - sl.start, "ms_per_call": pms,
                            "tokens_per_s": (sl.stop - sl.start) / (pms * 1e-3),
                            "path": {m.MLORA_PATH_DECODE: "decode", m.MLORA_PATH_TILED: "tiled",
                                     m.MLORA_PATH_GROUPED: "grouped"}.get(
                                m.mlora_linear_path(Lp.T, Lp.n_in, Lp.n_out, slots, Lp.K,
                                                    P.flags & ~m.MLORA_W_PACKED), "?"),
                            "binding": binding(ap["bytes"], ap["flops"], pms)}
        e["split"] = parts
    if with_cpu:
        e["cpu_baseline"] = cpu_baseline(P.layers, cpu_s)
    del P
    torch.cuda.empty_cache()
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (0 = per workload)")
    ap.add_argument("--warmup", type=int, default=-1)
    ap.add_argument("--workload", default="decode", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--configs", default="auto", choices=["auto", "none"],
                    help="auto: with the default decode headline (op linear) also time tiny, "
                         "prefill, mixed_qkv and compose into the `configs` list; none: only "
                         "the headline workload")
    ap.add_argument("--sets", type=int, default=0, help="rotating input copies (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle budget of the headline (each config entry gets half)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--flags", type=int, default=0, help="extra mlora_linear flags")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain copy kernel over MIB MiB (counter calibration)")
    ap.add_argument("--w-layout", default="auto", choices=["auto", "packed", "rowmajor"],
                    help="base weight as given (row-major) or packed once before timing "
                         "(mlora_pack_weight; same output bits); auto = packed for decode-sized "
                         "batches, where it is faster, row-major for the tiled path")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured copy-bandwidth and bf16 GEMM ceilings")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of a HIP graph holding whole passes over "
                         "the rotating input sets, at least 16 steps (the host's cost per call "
                         "paid once per replay)")
    ap.add_argument("--op", default="linear", choices=["linear", "bgmv", "plan"],
                    help="linear: mlora_linear (the whole layer); bgmv: the standalone pair "
                         "mlora_shrink + mlora_expand (y += LoRA delta), per layer; plan: "
                         "mlora_plan on the batch's index map (shared by its layers)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the layer shards without communication; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    P = Prepared(args.workload, op=args.op, w_layout=args.w_layout, sets=args.sets,
                 flags=args.flags)
    layers, algs = P.layers, P.algs
    steps = args.steps or (2000 if P.decode_like else 20)
    warmup = args.warmup if args.warmup >= 0 else (100 if P.decode_like else 3)

    if args.calibrate_copy:
        # a plain elementwise copy of known size, for scaling the HBM byte counters
        src = torch.ones(args.calibrate_copy * 2 ** 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ms, steps = time_steps(P, steps, warmup, graph=args.graph)
    kernel_ms = trace_kernel(P, steps)
    # single-call latency: one input set, each call waited for (no rotation, launch included)
    lat = []
    for i in range(50 if P.decode_like else 5):
        t0 = time.perf_counter()
        P.step(0)
        torch.cuda.synchronize()
        lat.append(time.perf_counter() - t0)
    single_call_us = sorted(lat)[len(lat) // 2] * 1e6
    T = layers[0].T
    tokens_per_s = T / (ms * 1e-3)
    tot_bytes = sum(a["bytes"] for a in algs)
    tot_flops = sum(a["flops"] for a in algs)
    k_avg_ms = sum(kernel_ms) / len(kernel_ms)
    if args.op == "plan":
        # bytes the sort must move: idx read, perm written, segment table and counts written
        import numpy as np
        L0 = layers[0]
        n_used = int(np.count_nonzero(L0.idx >= 0))
        n_seg = int(len(np.unique(L0.idx[L0.idx >= 0])))
        k_bytes = 4.0 * L0.T * L0.K + 4.0 * n_used + 12.0 * n_seg + 8.0
        achieved = k_bytes / (k_avg_ms * 1e-3) / 1e9
        tot_bytes, tot_flops = k_bytes, 0.0
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                "kernel": "mlora_plan (" + plan_form(L0.T * L0.K, L0.S) + ")",
                "kernel_avg_us": k_avg_ms * 1e3, "algorithmic_bytes_per_launch": k_bytes,
                "pairs": L0.T * L0.K, "used_pairs": n_used, "segments": n_seg}
    elif args.op == "bgmv":
        # the pair's two kernels; the roofline object describes the longer one
        sh_ms = sum(kernel_ms[0::2]) / len(kernel_ms[0::2])
        ex_ms = sum(kernel_ms[1::2]) / len(kernel_ms[1::2])
        sh_b = sum(a["shrink_bytes"] for a in algs) / len(layers)
        ex_b = sum(a["expand_bytes"] for a in algs) / len(layers)
        # the expand kernel the library picks: slot widths up to 32 have their own
        ex_name = ("mlora::expand_narrow_kernel" if layers[0].R <= 32 else
                   "mlora::expand_tokens_kernel")
        kern = [("mlora::shrink_rows_kernel (mlora_shrink)", sh_ms, sh_b),
                (ex_name + " (mlora_expand)", ex_ms, ex_b)]
        kern.sort(key=lambda k: -k[1])
        kname, k_avg_ms, k_bytes = kern[0]
        achieved = k_bytes / (k_avg_ms * 1e-3) / 1e9
        tot_bytes = sh_b * len(layers) + ex_b * len(layers)
        tot_flops = sum(a["bgmv_flops"] for a in algs)
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                "kernel": kname, "kernel_avg_us": k_avg_ms * 1e3,
                "algorithmic_bytes_per_launch": k_bytes,
                "other_kernel": {"kernel": kern[1][0], "kernel_avg_us": kern[1][1] * 1e3,
                                 "algorithmic_bytes_per_launch": kern[1][2],
                                 "achieved_GBps": kern[1][2] / (kern[1][1] * 1e-3) / 1e9}}
    else:
        roof = linear_roofline(P, kernel_ms)
        if P.decode_like:
            roof["traffic"] = committed_traffic("decode_gemm_kernel", args.workload)
        else:
            roof["traffic"] = committed_traffic("prefill_gemm_kernel", args.workload)
    roof["step_achieved_GBps"] = tot_bytes / (ms * 1e-3) / 1e9
    if not P.decode_like and args.op == "linear":
        roof["step_achieved_TFLOPs"] = tot_flops / (ms * 1e-3) / 1e12
    out = {
        "metric": {"bgmv": METRIC_BGMV, "plan": METRIC_PLAN}.get(args.op, METRIC),
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random bf16 weights and adapters)",
        "config": {"workload": DESCRIPTIONS[args.workload], "T": T,
                   "layers": [[L.n_in, L.n_out] for L in layers], "S": layers[0].S,
                   "R": layers[0].R, "K": layers[0].K,
                   "distinct_adapters": [a["distinct_adapters"] for a in algs],
                   "rotating_sets": P.nsets, "w_layout": P.w_layout, "path": P.paths,
                   "op": args.op,
                   "graph": args.graph},
        "roofline": roof,
        "step_algorithmic": {"bytes": tot_bytes, "flops": tot_flops},
    }
    out["single_call_us"] = single_call_us
    if not args.no_probes:
        out["probes"] = measured_ceilings(roof)
    if not args.no_cpu:
        if args.op == "plan":
            out["cpu_baseline"] = cpu_baseline_plan(layers[0], args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(layers, args.cpu_seconds,
                                               with_base=args.op == "linear")
    del P
    torch.cuda.empty_cache()
    if (args.configs == "auto" and args.workload == "decode" and args.op == "linear"
            and not args.graph):
        csteps = args.steps or 20
        cwarm = args.warmup if args.warmup >= 0 else 3
        out["configs"] = []
        for name in CONFIG_ORDER:
            print(f"bench: config {name}", file=sys.stderr, flush=True)
            out["configs"].append(config_entry(name, csteps, cwarm, args.cpu_seconds / 2,
                                               not args.no_cpu))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
