"""Benchmark of the per-token adapter-routing hot path on one MI355X.

Workload (default): the 4-modality kernel benchmark shape -- N=2048 tokens, d=4096, K=4
adapters (text/image/audio/video) of rank 16, vocabulary routing, k=1, bf16 data with fp32
accumulation; modality runs with geometric lengths (mean 64) and mix 0.4/0.3/0.15/0.15.

One step = one pass of the whole hot path over one batch: vocabulary routing, dispatch
(histogram, offsets, stable permutation) and the LoRA apply (shrink, expand, gate-weighted
alpha/r add into y) on adapters held in a hot-set slab.  The headline step is the one-launch
form (`molora_step_vocab`); the three-launch form (route, dispatch, apply) and the
per-sequence comparator (K masked dense passes) are timed beside it.  Inputs are resident in
HBM; S buffer sets (about 410 MB in all, above the 256 MB Infinity Cache) rotate so that
every step streams x / y0 / y from HBM.  Timed steps are replayed from one HIP graph that
holds one step per buffer set.

Prints one JSON line.  `--gpus N` with N > 1 is refused: this build measures one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ("token_adapter_routing_amd/csrc/apply.hip", "token_adapter_routing_amd/csrc/molora_mfma.h",
                  "token_adapter_routing_amd/csrc/molora_dev.h", "token_adapter_routing_amd/csrc/dispatch_dev.h",
                  "token_adapter_routing_amd/csrc/tile8_dev.h")
COUNTER_SUMMARY = "step_vocab_modality4.md"


def kernel_source_hash() -> str:
    src = "".join(open(os.path.join(ROOT, f)).read() for f in KERNEL_SOURCES)
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def counter_traffic(summary: str):
    """HBM bytes per launch of the dominant kernel from a committed rocprofv3 counter summary
    (FETCH_SIZE / WRITE_SIZE scaled by a copy calibration), or None when the kernel sources
    changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if kernel_source_hash() != fields.get("kernel_source_sha256_16"):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--sets", type=int, default=8, help="rotating input/output buffer sets")
    p.add_argument("--latency-reps", type=int, default=1000)
    p.add_argument("--kernel-reps", type=int, default=200)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip the three-launch and per-sequence lines")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run plain device copies of known size (for HBM counter scaling)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported in this build "
              f"(token data parallelism would replicate the hot set and split tokens, with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import token_adapter_routing_amd as m

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    m.load_library()

    if args.copy_calibration:
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 5}))
        return

    case = synth.modality4()
    t = case.targets[0]
    N, d_in, d_out, K, r, k = case.N, t.d_in, t.d_out, case.K, case.r, case.k

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    hs = m.molora_hotset_init([(bf(t.A), bf(t.B))], case.scale)
    bounds = case.bounds.tolist()
    S = args.sets
    sets = []
    ids_h = torch.from_numpy(case.ids)
    x_h = bf(t.x)
    y0_h = bf(t.y0)
    for s in range(S):
        sets.append(dict(
            ids=ids_h.to(dev), x=x_h.clone(), y0=y0_h.clone(),
            y=torch.empty(N, d_out, dtype=torch.bfloat16, device=dev),
            route=(torch.empty(N, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.float32, device=dev)),
            meta=(torch.empty(K, dtype=torch.int32, device=dev), torch.empty(K + 1, dtype=torch.int32, device=dev),
                  torch.empty(N, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.float32, device=dev),
                  torch.empty(N, dtype=torch.int32, device=dev))))
    del x_h, y0_h

    def step(s):  # one launch: route + dispatch + apply
        b = sets[s]
        m.molora_step_vocab(hs, b["ids"], bounds, b["x"], b["y0"], y=b["y"], route=b["route"], meta=b["meta"])

    def step3(s):  # three launches
        b = sets[s]
        idx, w = b["route"]
        mt = b["meta"]
        m.molora_route_vocab(b["ids"], bounds, idx=idx, w=w)
        m.molora_dispatch(idx, w, K, 1, out=mt)
        m.molora_apply(hs, b["x"], b["y0"], mt[1], mt[2], mt[3], mt[4], k=1, y=b["y"], path=m.PATH_AUTO)

    for s in range(S):
        step(s)
        step3(s)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    torch.cuda.current_stream().wait_stream(stream)

    def graph_of(fn, sets_range):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for s in sets_range:
                fn(s)
        return g

    reps = max(1, args.steps // S)
    steps = reps * S
    wreps = max(1, args.warmup // S)

    def time_graph(g):
        with torch.cuda.stream(stream):
            for _ in range(wreps):
                g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, time.perf_counter() - t0

    # ---------------- timed region (headline): `steps` one-launch steps
    g_all = graph_of(step, range(S))
    ms_per_step, wall = time_graph(g_all)
    value = N / (ms_per_step * 1e-3)

    # ---------------- dominant kernel: the one-launch step, back to back on `stream`
    kreps = max(S, args.kernel_reps // S * S)
    ka = torch.cuda.Event(enable_timing=True)
    kb = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for s in range(S):
            step(s)
        ka.record(stream)
        for i in range(kreps):
            step(i % S)
        kb.record(stream)
    torch.cuda.synchronize()
    kernel_us = ka.elapsed_time(kb) * 1e3 / kreps
    adapters = K * (d_in * r + r * d_out) * 2
    step_bytes = (N * d_in * 2 + 2 * N * d_out * 2  # x read, y0 read, y written (bf16)
                  + adapters                         # hot-set adapters used (all K)
                  + N * 4                            # token ids
                  + N * (4 + 4 + 4 + 4 + 4) + (2 * K + 1) * 4)  # idx, w, perm, perm_w, inv, counts, offsets
    kernel_gbs = step_bytes / (kernel_us * 1e-6) / 1e9

    # ---------------- step latency percentiles over single-step graph replays
    g_one = [graph_of(step, [s]) for s in range(S)]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.latency_reps)]
    with torch.cuda.stream(stream):
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            g_one[i % S].replay()
            b.record(stream)
    torch.cuda.synchronize()
    lat = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    p50 = lat[len(lat) // 2]
    p99 = lat[min(len(lat) - 1, int(0.99 * len(lat)))]
    cv = statistics.pstdev(lat) / statistics.mean(lat)

    out = {
        "metric": "routed tokens/s at N=2048 d=4096 K=4; % of HBM roofline; P99 step latency",
        "value": value,
        "unit": "routed tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": wreps * S,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; modality runs, bf16 N(0,1) activations, LoRA A~N(0,1/d), B~N(0,1/r))",
        "config": {"workload": "4-modality vocab routing N=2048 d=4096 K=4 r=16 k=1", "N": N, "d": d_in, "K": K,
                   "r": r, "k": k, "alpha_over_r": case.scale, "buffer_sets": S,
                   "launch": "hipGraph, one step per buffer set",
                   "step": "molora_step_vocab (route + dispatch + tile-local apply in one launch)"},
        "step_roofline_frac": step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "step_latency_us": {"p50": p50, "p99": p99, "cv": cv, "replays": len(lat), "graph": "single step"},
        "wall_s_timed_region": wall,
        "roofline": {"bound": "hbm", "achieved": kernel_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kernel_gbs / HBM_PEAK_GBS, "traffic": counter_traffic(COUNTER_SUMMARY),
                     "kernel": "step_vocab", "kernel_us": kernel_us, "algorithmic_bytes": step_bytes},
    }

    if not args.no_extras:
        # three launches per step (route_vocab, dispatch, apply)
        ms3, _ = time_graph(graph_of(step3, range(S)))
        # per-sequence comparator: K masked dense passes over all N tokens (metadata from the routing)
        seq = []
        for s in range(S):
            b = sets[s]
            offs, perm, pw = m.molora_seqpass_meta(b["route"][0], K)
            seq.append((offs, perm, pw))
        torch.cuda.synchronize()

        def seq_step(s):
            b = sets[s]
            offs, perm, pw = seq[s]
            m.molora_apply(hs, b["x"], b["y0"], offs[0], perm, pw[0], perm, k=1, y=b["y"], path=m.PATH_GROUPED)
            for e in range(1, K):
                m.molora_apply(hs, b["x"], b["y"], offs[e], perm, pw[e], perm, k=1, y=b["y"], path=m.PATH_GROUPED)

        seq_ms, _ = time_graph(graph_of(seq_step, range(S)))
        out["three_launch_step"] = {"ms_per_step": ms3, "routed_tokens_per_s": N / (ms3 * 1e-3)}
        out["per_sequence_comparator"] = {"ms_per_step": seq_ms, "passes": K,
                                          "speedup_per_token": seq_ms / ms_per_step}

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(out))


def cpu_baseline(case, seconds):
    """The CPU oracle as it stands (fp64 numpy), timed on this host on the same workload:
    route_vocab -> dispatch -> apply for the full batch, repeated for about `seconds`."""
    from oracle import apply, bf16_to_f64, dispatch, route_vocab
    t = case.targets[0]
    x, A, B, y0 = (bf16_to_f64(v) for v in (t.x, t.A, t.B, t.y0))  # conversion excluded
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()

    def one():
        idx, w = route_vocab(case.ids, case.bounds)
        counts, offsets, perm, perm_w, inv = dispatch(idx, w, case.K)
        return apply(y0, x, A, B, case.scale, perm, perm_w, offsets, 1)

    one()  # warm-up
    times = []
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or len(times) < 3:
        a = time.perf_counter()
        one()
        times.append(time.perf_counter() - a)
    med = statistics.median(times)
    return {"value": case.N / med, "unit": "routed tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"full batch (N={case.N}) route+dispatch+apply, {len(times)} runs, median {med * 1e3:.1f} ms",
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
