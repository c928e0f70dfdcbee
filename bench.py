"""Benchmark of the per-token adapter-routing hot path on one MI355X.

Workload (default): the 4-modality kernel benchmark shape -- N=2048 tokens, d=4096, K=4
adapters (text/image/audio/video) of rank 16, vocabulary routing, k=1, bf16 data with fp32
accumulation; modality runs with geometric lengths (mean 64) and mix 0.4/0.3/0.15/0.15.

One step = one pass of the whole hot path over one batch: vocabulary routing, dispatch
(histogram, offsets, stable permutation) and the LoRA apply (shrink, expand, gate-weighted
alpha/r add into y) on adapters held in a hot-set slab.  The headline step is
`molora_step_vocab` with a workspace: two launches that split the reduction and the output
columns into 512-wide slices (routing and the dispatch outputs happen inside them).  The
one-launch tile form, the three-launch form (route, dispatch, apply) and the per-sequence
comparator (K masked dense passes) are timed beside it.  Inputs are resident in
HBM; S buffer sets (about 410 MB in all, above the 256 MB Infinity Cache) rotate so that
every step streams x / y0 / y from HBM.  Timed steps are replayed from one HIP graph that
holds one step per buffer set.

Prints one JSON line.  `--gpus N` with N > 1 is refused: this build measures one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import re
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
                  "token_adapter_routing_amd/csrc/tile8_dev.h", "token_adapter_routing_amd/csrc/block_dev.h",
                  "token_adapter_routing_amd/csrc/gm_dev.h")
COUNTER_SUMMARY = "step_split_modality4.md"


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and whitespace removed, so that editing a
    comment does not mark the recorded counters stale)."""
    src = "".join(open(os.path.join(ROOT, f)).read() for f in KERNEL_SOURCES)
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
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
    p.add_argument("--kernel-reps", type=int, default=200,
                   help="unused: the step's kernels are timed by the graph replay (kept for older command lines)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip the three-launch and per-sequence lines")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run plain device copies of known size (for HBM counter scaling)")
    p.add_argument("--rows", default="C0,C2,C3,C4,C4stack,paging,tiling,backward,xf",
                   help="other configurations to measure beside the headline (comma list, or 'none')")
    p.add_argument("--row-reps", type=int, default=100, help="graph replays per timed row entry")
    p.add_argument("--stack-replays", type=int, default=1000, help="single-graph replays of the 28-layer stack row")
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
    # partial-sum workspace of the split step (written by its first launch, read by its second)
    ws = torch.zeros(m.molora_step_workspace(hs, 0, N), dtype=torch.uint8, device=dev)
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

    def step(s):  # two launches: route + shrink slices + dispatch, then expand slices
        b = sets[s]
        m.molora_step_vocab(hs, b["ids"], bounds, b["x"], b["y0"], y=b["y"], route=b["route"], meta=b["meta"], ws=ws)

    def step1(s):  # one launch: route + dispatch + 8-token tile apply
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
        step1(s)
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

    K_steps, W_steps = max(1, args.steps), max(0, args.warmup)

    def spin(stream_):
        with torch.cuda.stream(stream_):
            torch.cuda._sleep(200000)

    def time_steps(fn):
        """Exactly W_steps untimed steps, then exactly K_steps timed steps, each run as one HIP
        graph that cycles through the S buffer sets (step i uses set i mod S); HIP events on the
        launch stream bracket the timed graph.  Returns (ms per step, wall seconds)."""
        if W_steps:
            gw = graph_of(fn, [i % S for i in range(W_steps)])
            with torch.cuda.stream(stream):
                gw.replay()
            torch.cuda.synchronize()
            del gw
        g = graph_of(fn, [i % S for i in range(K_steps)])
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            # a short spin kernel ahead of the start event keeps the GPU busy while the host submits
            # the graph, so the events time the steps, not the submission (as in a serving loop
            # whose next graph is queued while the previous one runs)
            spin(stream)
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K_steps, time.perf_counter() - t0

    # ---------------- timed region (headline): exactly `steps` split steps
    ms_per_step, wall = time_steps(step)
    consistency = {"steps_requested": args.steps, "steps_timed": K_steps, "steps_match": K_steps == args.steps,
                   "warmup_requested": args.warmup, "warmup_run": W_steps, "warmup_match": W_steps == args.warmup,
                   "buffer_sets": S}
    value = N / (ms_per_step * 1e-3)

    # ---------------- the step's kernels (split_shrink + split_expand): their time per step is the
    # graph-replayed step above (HIP events on `stream`, no host launch in between); rocprofv3's
    # average durations of the two kernels in the same command add up to it
    kernel_us = ms_per_step * 1e3
    adapters = K * (d_in * r + r * d_out) * 2
    step_bytes = (N * d_in * 2 + 2 * N * d_out * 2  # x read, y0 read, y written (bf16)
                  + adapters                         # hot-set adapters used (all K)
                  + N * 4                            # token ids
                  + N * (4 + 4 + 4 + 4 + 4) + (2 * K + 1) * 4)  # idx, w, perm, perm_w, inv, counts, offsets
    kernel_gbs = step_bytes / (kernel_us * 1e-6) / 1e9

    # ---------------- a reference for the step's bytes: one torch elementwise kernel that reads two
    # [N][d] bf16 tensors and writes one (the x, y0 and y streams of a step, without the adapters)
    def stream_ref(s_):
        b = sets[s_]
        torch.add(b["x"], b["y0"], out=b["y"])
    ref_ms, _ = time_steps(stream_ref)

    # ---------------- step latency percentiles over single-step graph replays
    g_one = [graph_of(step, [s_]) for s_ in range(S)]
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
        "steps": K_steps,
        "warmup": W_steps,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; modality runs, bf16 N(0,1) activations, LoRA A~N(0,1/d), B~N(0,1/r))",
        "config": {"workload": "4-modality vocab routing N=2048 d=4096 K=4 r=16 k=1", "N": N, "d": d_in, "K": K,
                   "r": r, "k": k, "alpha_over_r": case.scale, "buffer_sets": S,
                   "launch": "one hipGraph of `steps` steps cycling through the buffer sets",
                   "step": "molora_step_vocab with a workspace (split_shrink: routing, 512-wide d_in slices, "
                           "dispatch outputs; split_expand: 512-wide output slices)"},
        "step_roofline_frac": step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "step_latency_us": {"p50": p50, "p99": p99, "cv": cv, "replays": len(lat), "graph": "single step"},
        "wall_s_timed_region": wall,
        "consistency": consistency,
        "streaming_reference": {"what": "torch.add(x, y0, out=y) on the same buffer sets: 2 reads + 1 write of "
                                        "[2048][4096] bf16 per step, one kernel, same graph timing",
                                "us_per_step": ref_ms * 1e3,
                                "GBps": 3 * N * d_in * 2 / (ref_ms * 1e-3) / 1e9},
        "roofline": {"bound": "hbm", "achieved": kernel_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kernel_gbs / HBM_PEAK_GBS, "traffic": counter_traffic(COUNTER_SUMMARY),
                     "kernel": "split_shrink + split_expand (the two launches of one step)",
                     "kernel_us": kernel_us, "algorithmic_bytes": step_bytes},
    }

    if not args.no_extras:
        # the one-launch step (tile apply) and three launches per step (route_vocab, dispatch, apply)
        ms1, _ = time_steps(step1)
        ms3, _ = time_steps(step3)
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

        seq_ms, _ = time_steps(seq_step)
        out["one_launch_tile_step"] = {"ms_per_step": ms1, "routed_tokens_per_s": N / (ms1 * 1e-3)}
        out["three_launch_step"] = {"ms_per_step": ms3, "routed_tokens_per_s": N / (ms3 * 1e-3)}
        out["per_sequence_comparator"] = {"ms_per_step": seq_ms, "passes": K,
                                          "speedup_per_token": seq_ms / ms_per_step}

    rows = [r for r in args.rows.split(",") if r and r != "none"]
    if rows:
        del sets, g_one
        torch.cuda.synchronize()
        out["rows"] = measure_rows(m, torch, dev, rows, args.row_reps, args.stack_replays)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
        out["cpu_baseline_1core"] = cpu_baseline(case, args.cpu_seconds, threads=1)
    print(json.dumps(out))


# ----------------------------------------------------------------------------------------------
# the other configurations: each step replayed from a HIP graph with inputs resident in HBM


def graph_ms(torch, fn, reps, warm=5, inner=1):
    """Average ms of fn() replayed from one captured graph holding `inner` consecutive calls
    (fn must only enqueue work); inner > 1 amortises the host cost of a graph launch, which
    otherwise bounds workloads of a few microseconds."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(inner):
            fn()
    with torch.cuda.stream(stream):
        for _ in range(warm):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * inner), g, stream


def measure_rows(m, torch, dev, rows, reps, stack_replays=1000):
    import synth

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    res = {}
    if "C0" in rows:
        # tiny vocab case: launch-bound, no roofline claim
        c = synth.tiny_vocab()
        t = c.targets[0]
        hs = m.molora_hotset_init([(bf(t.A), bf(t.B))], c.scale)
        ids, x, y0 = i32(c.ids), bf(t.x), bf(t.y0)
        y = torch.empty(c.N, t.d_out, dtype=torch.bfloat16, device=dev)
        route = (torch.empty(c.N, dtype=torch.int32, device=dev), torch.empty(c.N, dtype=torch.float32, device=dev))
        meta = (torch.empty(c.K, dtype=torch.int32, device=dev), torch.empty(c.K + 1, dtype=torch.int32, device=dev),
                torch.empty(c.N, dtype=torch.int32, device=dev), torch.empty(c.N, dtype=torch.float32, device=dev),
                torch.empty(c.N, dtype=torch.int32, device=dev))
        ms, _, _ = graph_ms(torch, lambda: m.molora_step_vocab(hs, ids, c.bounds.tolist(), x, y0, y=y, route=route,
                                                               meta=meta), reps, inner=20)
        res["C0_tiny_vocab"] = {"workload": "vocab routing N=256 d=512 K=4 r=8 k=1", "us_per_step": ms * 1e3,
                                "routed_tokens_per_s": c.N / (ms * 1e-3),
                                "launch": "molora_step_vocab, one launch; 20 steps per graph"}
        del hs, ids, x, y0, y
    if "C2" in rows:
        res["C2_qwen_layer"] = row_qwen_layer(m, torch, dev, bf, f32, reps)
    if "C3" in rows:
        res["C3_decode_sweep"] = row_decode(m, torch, dev, bf, i32, reps)
    if "C4" in rows:
        res["C4_stress"] = row_stress(m, torch, dev, bf, f32, max(20, reps // 4))
    if "C4stack" in rows:
        res["C4_stack"] = row_stack(m, torch, dev, replays=stack_replays)
    if "tiling" in rows:
        res["tiling"] = row_tiling(m, torch, dev, bf, f32, i32, max(20, reps // 4))
    if "backward" in rows:
        res["backward"] = row_backward(m, torch, dev, bf, f32, max(20, reps // 4))
    if "xf" in rows:
        res["xf_end_to_end"] = row_xf(m, torch, dev, max(5, reps // 20))
    if "paging" in rows:
        res["C1_paging"] = row_paging(m, torch, dev, bf, i32, max(200, reps * 2))
    torch.cuda.synchronize()
    return res


def row_paging(m, torch, dev, bf, i32, steps):
    """Hot set against on-demand paging on the 4-modality workload (the pages' Table 4 runs the
    Table 3 configuration; Figures 7 and 8 compare latencies).  Paging step: every adapter the
    batch uses is copied from pinned host memory into a device staging buffer, written into its
    slot with molora_hotset_load, then the split step runs; launched eagerly, as paging rules out
    a captured graph.  Hot-set steps: the split step alone, eager and as a single-step graph.
    Each step is timed on its own with HIP events on the launch stream."""
    import statistics
    import synth
    c = synth.modality4()
    t = c.targets[0]
    N, K, r = c.N, c.K, c.r
    hs = m.molora_hotset_init([(bf(t.A), bf(t.B))], c.scale)
    ids, x, y0 = i32(c.ids), bf(t.x), bf(t.y0)
    y = torch.empty(N, t.d_out, dtype=torch.bfloat16, device=dev)
    route = (torch.empty(N, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.float32, device=dev))
    meta = (torch.empty(K, dtype=torch.int32, device=dev), torch.empty(K + 1, dtype=torch.int32, device=dev),
            torch.empty(N, dtype=torch.int32, device=dev), torch.empty(N, dtype=torch.float32, device=dev),
            torch.empty(N, dtype=torch.int32, device=dev))
    ws = torch.zeros(m.molora_step_workspace(hs, 0, N), dtype=torch.uint8, device=dev)
    hostA = torch.from_numpy(t.A.view(np.int16)).view(torch.bfloat16).pin_memory()
    hostB = torch.from_numpy(t.B.view(np.int16)).view(torch.bfloat16).pin_memory()
    stA, stB = torch.empty_like(hostA, device=dev), torch.empty_like(hostB, device=dev)
    # adapters the batch uses, decided on the host from its token ids before the timed steps
    used = sorted(set(int(e) for e in np.searchsorted(c.bounds, c.ids, side="right") - 1 if 0 <= e < K))
    bounds = c.bounds.tolist()
    stream = torch.cuda.Stream()

    def step():
        m.molora_step_vocab(hs, ids, bounds, x, y0, y=y, route=route, meta=meta, ws=ws, stream=stream)

    def paged():
        for e in used:
            stA[e].copy_(hostA[e], non_blocking=True)
            stB[e].copy_(hostB[e], non_blocking=True)
        for e in used:
            m.molora_hotset_load(hs, 0, e, stA[e], stB[e], stream=stream)
        step()

    def timed(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        with torch.cuda.stream(stream):
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            for a, b in evs:
                a.record(stream)
                fn()
                b.record(stream)
        torch.cuda.synchronize()
        lat = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        return {"p50_us": lat[len(lat) // 2], "p99_us": lat[min(len(lat) - 1, int(0.99 * len(lat)))],
                "mean_us": statistics.mean(lat), "cv": statistics.pstdev(lat) / statistics.mean(lat), "steps": n}

    res = {"workload": "4-modality vocab routing N=2048 d=4096 K=4 r=16 k=1",
           "adapters_paged_per_step": len(used), "host_to_device_bytes_per_step": len(used) * (hostA[0].numel() +
                                                                                               hostB[0].numel()) * 2,
           "paging_eager": timed(paged, steps), "hot_set_eager": timed(step, steps)}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    res["hot_set_graph"] = timed(g.replay, steps)
    res["paging_over_hot_set_eager_p50"] = res["paging_eager"]["p50_us"] / res["hot_set_eager"]["p50_us"]
    res["paging_over_hot_set_graph_p50"] = res["paging_eager"]["p50_us"] / res["hot_set_graph"]["p50_us"]
    res["paging_over_hot_set_graph_p99"] = res["paging_eager"]["p99_us"] / res["hot_set_graph"]["p99_us"]
    del g
    res["access_patterns"] = paging_patterns(m, torch, dev, hs, c, step, timed, stream, steps)
    del hs
    return res


def paging_patterns(m, torch, dev, hs, c, step, timed, stream, steps, L=16, burst=8):
    """Paging under access patterns (the pages' Figure 8): L logical adapters live in pinned host
    memory behind the hot set's K slots, one slot per modality of the batch (a direct-mapped cache:
    slot s keeps the adapter modality s used last); each step's batch (the 4-modality ids) needs
    K of them.  bursty: the same K for `burst` steps, then K others; uniform: K distinct adapters
    drawn at random each step; adversarial: the K slots cycle through all L adapters, so every
    access misses.  A miss pages the adapter into its slot (2 copies + molora_hotset_load)."""
    import synth
    t = c.targets[0]
    K = c.K
    A, B = synth._lora_weights(16, 0, L, t.d_in, t.d_out, c.r)
    hostA = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).pin_memory()
    hostB = torch.from_numpy(B.view(np.int16)).view(torch.bfloat16).pin_memory()
    stA = torch.empty(K, t.d_in, c.r, dtype=torch.bfloat16, device=dev)
    stB = torch.empty(K, c.r, t.d_out, dtype=torch.bfloat16, device=dev)
    g = np.random.default_rng(np.random.SeedSequence([20260316, 1, 99]))
    n = steps + 10

    def sets(kind):
        if kind == "bursty":
            out = []
            for i in range(n):
                if i % burst == 0:
                    cur = [int(v) for v in g.choice(L, K, replace=False)]
                out.append(cur)
            return out
        if kind == "uniform":
            return [[int(v) for v in g.choice(L, K, replace=False)] for _ in range(n)]
        return [[(K * i + j) % L for j in range(K)] for i in range(n)]  # adversarial: cycles all L

    res = {"logical_adapters": L, "slots": K}
    for kind in ("bursty", "uniform", "adversarial"):
        seq = sets(kind)
        resident = [-1] * K  # logical adapter held by each slot (slot = modality of the batch)
        misses = [0]
        it = iter(seq)

        def paged():
            need = next(it)
            for s_, a in enumerate(need):
                if resident[s_] != a:
                    stA[s_].copy_(hostA[a], non_blocking=True)
                    stB[s_].copy_(hostB[a], non_blocking=True)
                    m.molora_hotset_load(hs, 0, s_, stA[s_], stB[s_], stream=stream)
                    resident[s_] = a
                    misses[0] += 1
            step()

        r_ = timed(paged, steps)
        r_["page_ins_per_step"] = misses[0] / len(seq)
        res[kind] = r_
    return res


def row_qwen_layer(m, torch, dev, bf, f32, reps):
    """Learned top-k MoLoRA on one Qwen3-1.7B-shaped layer: router MLP (d->64->K, ReLU), top-2,
    dispatch, then the 7 projections' applies (y = y0 + delta, bf16)."""
    import synth
    c = synth.qwen_layer()
    N, K, k = c.N, c.K, c.k
    r = c.router
    xs = {}
    for t in c.targets:  # q/k/v/gate/up share x
        key = id(t.x)
        if key not in xs:
            xs[key] = bf(t.x)
    tx = [xs[id(t.x)] for t in c.targets]
    y0 = [bf(t.y0) for t in c.targets]
    y = [torch.empty(N, t.d_out, dtype=torch.bfloat16, device=dev) for t in c.targets]
    hs = m.molora_hotset_init([(bf(t.A), bf(t.B)) for t in c.targets], c.scale)
    W1 = bf(np.ascontiguousarray(r["W1"].T))
    W2 = bf(np.ascontiguousarray(r["W2"].T))
    b1, b2 = f32(r["b1"]), f32(r["b2"])
    logits = torch.empty(N, K, dtype=torch.float32, device=dev)
    idx = torch.empty(N * k, dtype=torch.int32, device=dev)
    w = torch.empty(N * k, dtype=torch.float32, device=dev)
    flags = torch.empty(N, dtype=torch.uint8, device=dev)
    # the router's first layer split over d (a workspace; the same bits as one launch)
    rws = torch.empty(max(256, m.molora_route_topk_workspace(N, c.targets[0].d_in)), dtype=torch.uint8, device=dev)
    meta = (torch.empty(K, dtype=torch.int32, device=dev), torch.empty(K + 1, dtype=torch.int32, device=dev),
            torch.empty(N * k, dtype=torch.int32, device=dev), torch.empty(N * k, dtype=torch.float32, device=dev),
            torch.empty(N * k, dtype=torch.int32, device=dev))
    compulsory = (sum(v.numel() * 2 for v in xs.values()) + sum(2 * N * t.d_out * 2 for t in c.targets)
                  + sum(K * (t.d_in + t.d_out) * c.r * 2 for t in c.targets)
                  + (W1.numel() + W2.numel()) * 2 + (b1.numel() + b2.numel()) * 4)
    d = c.targets[0].d_in
    flops = sum(N * k * c.r * (t.d_in + t.d_out) * 2 for t in c.targets) + N * (2 * d * 64 + 2 * 64 * K)
    out = {"workload": "Qwen3-1.7B-shaped layer N=4096 d=2048 7 targets K=4 r=16 k=2, router MLP 2048->64->4",
           "compulsory_bytes": compulsory, "flops": flops, "paths": {}}
    for name, path in (("auto", m.PATH_AUTO), ("grouped", m.PATH_GROUPED), ("tile", m.PATH_TILE),
                       ("block", m.PATH_BLOCK)):
        wss = [torch.zeros(max(1, m.molora_apply_workspace(hs, ti, N, k, path, torch.bfloat16)), dtype=torch.uint8, device=dev)
               for ti in range(len(c.targets))]

        def step():
            m.molora_route_topk(k, K, x=tx[0], W1=W1, b1=b1, W2=W2, b2=b2, logits=logits, idx=idx, w=w, flags=flags,
                                ws=rws)
            m.molora_dispatch(idx, w, K, k, out=meta)
            for ti in range(len(c.targets)):
                m.molora_apply(hs, tx[ti], y0[ti], meta[1], meta[2], meta[3], meta[4], k=k, target=ti, y=y[ti],
                               path=path, ws=wss[ti])

        ms, g, _ = graph_ms(torch, step, reps)
        out["paths"][name] = {"ms_per_step": ms, "routed_tokens_per_s": N / (ms * 1e-3),
                              "pairs_per_s": N * k / (ms * 1e-3),
                              "roofline_frac": compulsory / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)}
        del g, wss
    # the 7 projections in one multi-target apply (one launch per phase on the fused paths)
    tids = list(range(len(c.targets)))
    for name, path in (("multi_auto", m.PATH_AUTO), ("multi_skinny", m.PATH_SKINNY)):
        mws = torch.zeros(max(1, m.molora_apply_multi_workspace(hs, tids, N, k, path, torch.bfloat16)),
                          dtype=torch.uint8, device=dev)

        def step():
            m.molora_route_topk(k, K, x=tx[0], W1=W1, b1=b1, W2=W2, b2=b2, logits=logits, idx=idx, w=w, flags=flags,
                                ws=rws)
            m.molora_dispatch(idx, w, K, k, out=meta)
            m.molora_apply_multi(hs, tx, y0, meta[1], meta[2], meta[3], meta[4], k=k, ys=y, path=path, ws=mws)

        ms, g, _ = graph_ms(torch, step, reps)
        out["paths"][name] = {"ms_per_step": ms, "routed_tokens_per_s": N / (ms * 1e-3),
                              "pairs_per_s": N * k / (ms * 1e-3),
                              "roofline_frac": compulsory / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)}
        del g, mws
    # dispatch and the 7 projections in one call (the dispatch rides in the block shrink's launch)
    fws = torch.zeros(max(1, m.molora_dispatch_apply_multi_workspace(hs, tids, N, k, m.PATH_AUTO, torch.bfloat16)),
                      dtype=torch.uint8, device=dev)

    def step():
        m.molora_route_topk(k, K, x=tx[0], W1=W1, b1=b1, W2=W2, b2=b2, logits=logits, idx=idx, w=w, flags=flags,
                            ws=rws)
        m.molora_dispatch_apply_multi(hs, tx, y0, idx, w, K, k, ys=y, path=m.PATH_AUTO, meta=meta, ws=fws)

    ms, g, _ = graph_ms(torch, step, reps)
    out["paths"]["multi_fused_dispatch"] = {"ms_per_step": ms, "routed_tokens_per_s": N / (ms * 1e-3),
                                            "pairs_per_s": N * k / (ms * 1e-3),
                                            "roofline_frac": compulsory / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)}
    del g, fws
    best = min(out["paths"].items(), key=lambda kv: kv[1]["ms_per_step"])
    out["best_path"] = best[0]
    out["routed_tokens_per_s"] = best[1]["routed_tokens_per_s"]
    out["roofline_frac"] = best[1]["roofline_frac"]
    return out


def row_decode(m, torch, dev, bf, i32, reps):
    """Decode sweep: B tokens, 64 hot-set adapters of rank 16, one uniformly random adapter
    per token (idx given): dispatch + apply on the skinny, grouped and AUTO paths (AUTO's choice
    as the library reports it); then the slab layouts (direct vs indirect, identical operations,
    AUTO path) at every B for 4 .. 64 adapters."""
    import synth
    names = {m.PATH_GROUPED: "grouped", m.PATH_SKINNY: "skinny", m.PATH_TILE: "tile", m.PATH_BLOCK: "block"}
    batches = (1, 16, 64, 160, 512, 2048)
    out = {"workload": "decode B in {1,16,64,160,512,2048}, d=4096, K=64 r=16 k=1; 20 steps per graph",
           "sweep": {}, "layouts": {}}
    per_adapter = 2 * 4096 * 16 * 2
    cache = {}
    for B in batches:
        c = synth.decode_batch(B)
        t = c.targets[0]
        if "hs" not in cache:
            cache["hs"] = m.molora_hotset_init([(bf(t.A), bf(t.B))], c.scale)
        hs = cache["hs"]
        x, y0 = bf(t.x), bf(t.y0)
        y = torch.empty(B, t.d_out, dtype=torch.bfloat16, device=dev)
        idx = i32(c.idx)
        w = torch.ones(B, dtype=torch.float32, device=dev)
        meta = (torch.empty(c.K, dtype=torch.int32, device=dev), torch.empty(c.K + 1, dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.float32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))
        used = len(np.unique(c.idx))
        nbytes = B * (t.d_in + 2 * t.d_out) * 2 + used * per_adapter
        entry = {"distinct_adapters": used, "compulsory_bytes": nbytes,
                 "auto_path": names[m.molora_apply_path(hs, B, 1, m.PATH_AUTO)]}
        for name, path in (("skinny", m.PATH_SKINNY), ("grouped", m.PATH_GROUPED), ("auto", m.PATH_AUTO)):
            ws = torch.zeros(max(1, m.molora_apply_workspace(hs, 0, B, 1, path, torch.bfloat16)), dtype=torch.uint8, device=dev)

            def step():
                m.molora_dispatch(idx, w, c.K, 1, out=meta)
                m.molora_apply(hs, x, y0, meta[1], meta[2], meta[3], meta[4], k=1, y=y, path=path, ws=ws)

            ms, g, _ = graph_ms(torch, step, reps, inner=20)
            entry[name] = {"us_per_step": ms * 1e3, "GBps": nbytes / (ms * 1e-3) / 1e9}
            del g
        out["sweep"][str(B)] = entry
    sk = [int(b) for b, e in out["sweep"].items() if e["grouped"]["us_per_step"] < e["skinny"]["us_per_step"]]
    out["grouped_faster_from_B"] = min(sk) if sk else None
    del cache
    # direct vs indirect slab at 4/8/16/32/64 adapters and every B, identical operations (AUTO path)
    for Kh in (4, 8, 16, 32, 64):
        c0 = synth.decode_batch(1, K=Kh, case_id=30 + Kh)
        t0 = c0.targets[0]
        hss = {lay: m.molora_hotset_init([(bf(t0.A), bf(t0.B))], c0.scale, layout=lay) for lay in (0, 1)}
        per_k = {}
        for B in batches:
            c = synth.decode_batch(B, K=Kh, case_id=30 + Kh)
            t = c.targets[0]
            x, y0 = bf(t.x), bf(t.y0)
            y = torch.empty(B, t.d_out, dtype=torch.bfloat16, device=dev)
            meta = m.molora_dispatch(i32(c.idx), torch.ones(B, dtype=torch.float32, device=dev), Kh, 1)
            ent = {"path": names[m.molora_apply_path(hss[0], B, 1, m.PATH_AUTO)]}
            for lay, name in ((0, "direct"), (1, "indirect")):
                hs = hss[lay]
                ms, g, _ = graph_ms(torch, lambda: m.molora_apply(hs, x, y0, meta[1], meta[2], meta[3], meta[4], k=1,
                                                                  y=y), reps, inner=20)
                ent[name + "_us"] = ms * 1e3
                del g
            ent["indirect_over_direct"] = ent["indirect_us"] / ent["direct_us"]
            per_k[str(B)] = ent
        out["layouts"][str(Kh)] = per_k
        del hss
    out["layout_mean_indirect_over_direct"] = statistics.mean(
        e["indirect_over_direct"] for pk in out["layouts"].values() for e in pk.values())
    return out


def row_stress(m, torch, dev, bf, f32, reps):
    """Stress: N=16384, d=4096, K=16 adapters of rank 64, Zipf(1.1) biased random router
    (logits given), top-k for k = 1..4: route_topk -> dispatch -> apply."""
    import synth
    c = synth.stress(1)
    t = c.targets[0]
    N, K = c.N, c.K
    x, y0 = bf(t.x), bf(t.y0)
    y = torch.empty(N, t.d_out, dtype=torch.bfloat16, device=dev)
    logits = f32(c.logits)
    hs = m.molora_hotset_init([(bf(t.A), bf(t.B))], c.scale)
    compulsory = 3 * N * t.d_in * 2 + K * (t.d_in + t.d_out) * c.r * 2 + logits.numel() * 4
    out = {"workload": "stress N=16384 d=4096 K=16 r=64 Zipf(1.1) logits", "compulsory_bytes": compulsory, "k": {}}
    for k in (1, 2, 3, 4):
        idx = torch.empty(N * k, dtype=torch.int32, device=dev)
        w = torch.empty(N * k, dtype=torch.float32, device=dev)
        meta = (torch.empty(K, dtype=torch.int32, device=dev), torch.empty(K + 1, dtype=torch.int32, device=dev),
                torch.empty(N * k, dtype=torch.int32, device=dev), torch.empty(N * k, dtype=torch.float32, device=dev),
                torch.empty(N * k, dtype=torch.int32, device=dev))
        ws = torch.zeros(max(1, m.molora_apply_workspace(hs, 0, N, k, m.PATH_AUTO, torch.bfloat16)), dtype=torch.uint8, device=dev)

        def step():
            m.molora_route_topk(k, K, logits=logits, idx=idx, w=w, want_flags=False)
            m.molora_dispatch(idx, w, K, k, out=meta)
            m.molora_apply(hs, x, y0, meta[1], meta[2], meta[3], meta[4], k=k, y=y, ws=ws)

        ms, g, _ = graph_ms(torch, step, reps)
        flops = N * k * c.r * (t.d_in + t.d_out) * 2
        out["k"][str(k)] = {"ms_per_step": ms, "routed_tokens_per_s": N / (ms * 1e-3),
                            "pairs_per_s": N * k / (ms * 1e-3),
                            "roofline_frac": compulsory / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                            "mfma_utilisation_bf16": flops / (ms * 1e-3) / 2.5e15}
        del g, ws
    return out


def row_tiling(m, torch, dev, bf, f32, i32, reps):
    """Fixed against adaptive tiling of the 64-row grouped kernel (the pages' Table 9): adapter
    usage mixes 25% each, 80/10/5/5 and 95/2/2/1 (one adapter per token, 4 adapters of rank 64,
    d=4096) at 512, 2048 and 16384 tokens (the adaptive bound is 16 rows at 512 tokens, 64 from
    2048 on), and the stress workload's Zipf top-k (16 adapters of rank 64, 16384 tokens,
    k = 1..4).  Each entry: dispatch (and top-k) + apply as one graph."""
    import synth
    out = {"workload": "grouped 64-row kernel, MOLORA_PATH_GROUPED (adaptive) vs MOLORA_PATH_GROUPED_FIXED",
           "mixes": {}, "zipf_stress": {}}
    mixes = {"uniform_25": (0.25, 0.25, 0.25, 0.25), "80_10_5_5": (0.8, 0.1, 0.05, 0.05),
             "95_2_2_1": (0.95, 0.02, 0.02, 0.01)}
    for N in (512, 2048, 16384):
        for name, probs in mixes.items():
            c = synth.mixed_batch(N, probs, case_id=6, sub=N)
            t = c.targets[0]
            hs = m.molora_hotset_init([(bf(t.A), bf(t.B))], c.scale)
            x, y0 = bf(t.x), bf(t.y0)
            y = torch.empty(N, t.d_out, dtype=torch.bfloat16, device=dev)
            idx = i32(c.idx)
            w = torch.ones(N, dtype=torch.float32, device=dev)
            meta = m.molora_dispatch(idx, w, c.K, 1)
            ent = {"segment_rows": [int(v) for v in np.bincount(c.idx, minlength=c.K)]}
            for tname, path in (("adaptive", m.PATH_GROUPED), ("fixed64", m.PATH_GROUPED_FIXED)):
                def step():
                    m.molora_dispatch(idx, w, c.K, 1, out=meta)
                    m.molora_apply(hs, x, y0, meta[1], meta[2], meta[3], meta[4], k=1, y=y, path=path)
                ms, g, _ = graph_ms(torch, step, reps)
                ent[tname + "_us"] = ms * 1e3
                del g
            ent["fixed_over_adaptive"] = ent["fixed64_us"] / ent["adaptive_us"]
            out["mixes"][f"{name}_N{N}"] = ent
            del hs
    c = synth.stress(1)
    t = c.targets[0]
    N, K = c.N, c.K
    x, y0 = bf(t.x), bf(t.y0)
    y = torch.empty(N, t.d_out, dtype=torch.bfloat16, device=dev)
    logits = f32(c.logits)
    hs = m.molora_hotset_init([(bf(t.A), bf(t.B))], c.scale)
    for k in (1, 2, 3, 4):
        idx = torch.empty(N * k, dtype=torch.int32, device=dev)
        w = torch.empty(N * k, dtype=torch.float32, device=dev)
        meta = (torch.empty(K, dtype=torch.int32, device=dev), torch.empty(K + 1, dtype=torch.int32, device=dev),
                torch.empty(N * k, dtype=torch.int32, device=dev), torch.empty(N * k, dtype=torch.float32, device=dev),
                torch.empty(N * k, dtype=torch.int32, device=dev))
        ent = {}
        for tname, path in (("adaptive", m.PATH_GROUPED), ("fixed64", m.PATH_GROUPED_FIXED)):
            ws = torch.zeros(max(1, m.molora_apply_workspace(hs, 0, N, k, path, torch.bfloat16)), dtype=torch.uint8,
                             device=dev)

            def step():
                m.molora_route_topk(k, K, logits=logits, idx=idx, w=w, want_flags=False)
                m.molora_dispatch(idx, w, K, k, out=meta)
                m.molora_apply(hs, x, y0, meta[1], meta[2], meta[3], meta[4], k=k, y=y, path=path, ws=ws)

            ms, g, _ = graph_ms(torch, step, reps)
            ent[tname + "_us"] = ms * 1e3
            del g, ws
        ent["fixed_over_adaptive"] = ent["fixed64_us"] / ent["adaptive_us"]
        out["zipf_stress"][f"k{k}"] = ent
    del hs
    return out


def row_backward(m, torch, dev, bf, f32, reps):
    """Backward of the routed LoRA (dx through the transposed hot set, dA, dB, dL/dw) on the
    4-modality shape and the stress shape, and the router chain (dL/dlogits, router MLP
    gradients) on the Qwen-shaped layer; each one graph replayed.  Compulsory bytes: read x,
    dL/dy and dx0, write dx (bf16), read A and B, write dA, dB (fp32) and dL/dw."""
    import synth
    out = {}

    def lora(name, N, d, K, r, k, cid, idx=None, w=None):
        A = bf(synth.normal_bf16(cid, synth.T_A, (K, d, r), std=1.0 / np.sqrt(d)))
        B = bf(synth.normal_bf16(cid, synth.T_B, (K, r, d), std=1.0 / np.sqrt(r)))
        x = bf(synth.normal_bf16(cid, synth.T_X, (N, d)))
        gy_b, dx0_b = synth.grad_case(cid, N, d, d)
        gy, dx0 = bf(gy_b), bf(dx0_b)
        if idx is None:
            g = np.random.default_rng(cid)
            idx = g.integers(0, K, size=N * k).astype(np.int32)
            w = np.full(N * k, 1.0 / k, np.float32)
        hs = m.molora_hotset_init([(A, B)], 2.0)
        hs_t = m.molora_hotset_init_transposed([(A, B)], 2.0)
        meta = m.molora_dispatch(torch.from_numpy(idx).to(dev), torch.from_numpy(w).to(dev), K, k)
        dx = torch.empty(N, d, dtype=torch.bfloat16, device=dev)
        dA = torch.empty(K, d, r, dtype=torch.float32, device=dev)
        dB = torch.empty(K, r, d, dtype=torch.float32, device=dev)
        dw = torch.empty(N * k, dtype=torch.float32, device=dev)
        ws = torch.zeros(m.molora_backward_workspace(hs, hs_t, N, k), dtype=torch.uint8, device=dev)

        def step():
            m.molora_backward(hs, hs_t, x, gy, meta[1], meta[2], meta[3], meta[4], k=k, dx0=dx0, dx=dx, dA=dA, dB=dB,
                              dw=dw, ws=ws)

        ms, g, _ = graph_ms(torch, step, reps)
        compulsory = 4 * N * d * 2 + K * 2 * d * r * (2 + 4) + N * k * 4
        out[name] = {"workload": f"backward N={N} d={d} K={K} r={r} k={k}", "us": ms * 1e3,
                     "compulsory_bytes": compulsory,
                     "roofline_frac": compulsory / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                     "workspace_bytes": int(ws.numel())}
        del g

    lora("modality4_k1", 2048, 4096, 4, 16, 1, 54)
    c = synth.stress(1)
    for k in (1, 2):
        lg = c.logits.astype(np.float64)
        order = np.argsort(-lg, axis=1, kind="stable")[:, :k]
        sel = np.sort(order, axis=1)
        ex = np.exp(np.take_along_axis(lg, sel, 1) - np.take_along_axis(lg, sel, 1).max(1, keepdims=True))
        w = (ex / ex.sum(1, keepdims=True)).astype(np.float32)
        lora(f"stress_k{k}", c.N, 4096, 16, 64, k, 4, sel.reshape(-1).astype(np.int32), w.reshape(-1))
    # router chain on the Qwen-shaped layer
    q = synth.qwen_layer()
    r = q.router
    N, K, k, d = q.N, q.K, q.k, q.targets[0].d_in
    xq = bf(q.targets[0].x)
    W1, W2 = bf(np.ascontiguousarray(r["W1"].T)), bf(np.ascontiguousarray(r["W2"].T))
    b1 = f32(r["b1"])
    g = np.random.default_rng(9)
    idx = torch.from_numpy(np.sort(np.stack([g.choice(K, k, replace=False) for _ in range(N)]), axis=1).astype(np.int32)).to(dev)
    wq = torch.full((N, k), 1.0 / k, dtype=torch.float32, device=dev)
    dwq = f32(g.standard_normal((N, k)).astype(np.float32))
    dl = torch.empty(N, K, dtype=torch.float32, device=dev)
    o = {n: torch.empty(sh, dtype=torch.float32, device=dev) for n, sh in (("dW1", (64, d)), ("db1", (64,)),
                                                                            ("dW2", (K, 64)), ("db2", (K,)),
                                                                            ("dx", (N, d)))}
    wsr = torch.zeros(m.molora_router_backward_workspace(N, d, K), dtype=torch.uint8, device=dev)

    def rstep():
        m.molora_route_topk_backward(idx, wq, dwq, K, dlogits=dl)
        m.molora_router_backward(xq, W1, b1, W2, dl, want=(), out=o, ws=wsr)

    ms, gr, _ = graph_ms(torch, rstep, reps)
    rbytes = N * d * 2 + 64 * d * 2 + N * d * 4 + 64 * d * 4 + N * K * 4 * 2
    out["router_qwen"] = {"workload": f"router backward N={N} d={d} K={K} k={k} (dlogits, dW1, db1, dW2, db2, dx fp32)",
                          "us": ms * 1e3, "compulsory_bytes": rbytes,
                          "roofline_frac": rbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)}
    del gr
    return out


def row_xf(m, torch, dev, reps):
    """The synthetic decoder with per-token LoRA on all seven projections (the pages' Table 7:
    d = 1024 / 2048 / 4096, L = 2 / 4, batches 16x512, 4x512, 16x512, K = 4; Table 8: d = 2048,
    L = 4, K = 2, interleaved modalities), rank 16, vocabulary routing of interleaved modality
    runs (mean run 64 tokens).  Per token: one forward with the per-token routing.  Per
    sequence (the pages' simulation): K forwards, pass e with every token on adapter e.  Base:
    one forward without adapters.  Eager launches (the base GEMMs are rocBLAS calls), timed
    with events around `reps` repetitions after a warmup."""
    import synth
    gen = torch.Generator(device=dev)
    out = {}
    configs = [("table7_d1024_L2", 1024, 2, 16, 512, 4), ("table7_d2048_L4", 2048, 4, 4, 512, 4),
               ("table7_d4096_L4", 4096, 4, 16, 512, 4), ("table8_d2048_L4_K2", 2048, 4, 4, 512, 2)]
    for name, d, L, n_seq, seq_len, K in configs:
        gen.manual_seed(1000 + d + L + K)
        f = synth.xf_mlp_width(d)
        r = 16
        dims = synth.xf_dims(d, f)

        def randn(*shape, std):
            return (torch.randn(*shape, generator=gen, device=dev) * std).to(torch.bfloat16)

        layers, bare = [], []
        for _ in range(L):
            W = [randn(dout, din, std=din ** -0.5) for din, dout in dims]
            n1 = (1 + randn(d, std=0.1).float()).to(torch.bfloat16)
            n2 = (1 + randn(d, std=0.1).float()).to(torch.bfloat16)
            hs = m.molora_hotset_init([(randn(K, din, r, std=din ** -0.5), randn(K, r, dout, std=0.25 / r ** 0.5))
                                       for din, dout in dims], 2.0)
            layers.append({"norm1": n1, "norm2": n2, "W": W, "lora": hs})
            bare.append({"norm1": n1, "norm2": n2, "W": W, "lora": None})
        model, base = m.XfModel(d, f, layers), m.XfModel(d, f, bare)
        N = n_seq * seq_len
        labels = synth.modality_runs(1000 + d, N, [1.0 / K] * K, 64.0)
        bounds = synth.vocab_bounds(K)
        ids = torch.from_numpy(synth.ids_for_labels(1000 + d, labels, bounds)).to(dev)
        idx, w = m.molora_route_vocab(ids, [int(b) for b in bounds])
        route = m.molora_dispatch(idx, w, K, 1)[1:]
        passes = []
        for e in range(K):
            ie = torch.full((N,), e, dtype=torch.int32, device=dev)
            passes.append(m.molora_dispatch(ie, torch.ones(N, device=dev), K, 1)[1:])
        x = randn(N, d, std=1.0)
        y = torch.empty_like(x)
        ws = torch.empty(m.molora_xf_workspace(model, n_seq, seq_len), dtype=torch.uint8, device=dev)

        def timed(fn):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        per_token = timed(lambda: m.molora_xf_forward(model, x, n_seq, seq_len, route=route, out=y, ws=ws))
        per_seq = timed(lambda: [m.molora_xf_forward(model, x, n_seq, seq_len, route=p, out=y, ws=ws) for p in passes])
        base_ms = timed(lambda: m.molora_xf_forward(base, x, n_seq, seq_len, out=y, ws=ws))
        flops = 2 * N * L * sum(a * b for a, b in dims) + 4 * n_seq * L * (d // 128) * seq_len * seq_len * 128
        out[name] = {"workload": f"decoder d={d} f={f} L={L} batch {n_seq}x{seq_len} K={K} r={r} (7 LoRA targets)",
                     "per_token_ms": per_token, "per_sequence_sim_ms": per_seq, "speedup": per_seq / per_token,
                     "base_only_ms": base_ms, "lora_overhead_frac": per_token / base_ms - 1.0,
                     "base_tflops_per_token_pass": flops / (per_token * 1e-3) / 1e12}
        del ws, layers, bare, model, base
        torch.cuda.empty_cache()
    return out


def row_stack(m, torch, dev, layers=28, B=256, K=16, r=64, k=2, replays=1000):
    """A hipGraph of 28 layers x 7 Qwen3-1.7B projections at decode batch 256 (K=16 adapters of
    rank 64 per projection, top-2 over Zipf logits per layer, in-place y += delta); step
    latency percentiles over single-graph replays.  Adapters are random device tensors."""
    import synth
    targets = synth.QWEN3_1P7B_TARGETS
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260316)
    layer_objs = []
    nbytes = 0
    for L in range(layers):
        tg = []
        for (_, d_in, d_out) in targets:
            A = (torch.randn(K, d_in, r, device=dev, generator=gen) / d_in ** 0.5).to(torch.bfloat16)
            Bm = (torch.randn(K, r, d_out, device=dev, generator=gen) / r ** 0.5).to(torch.bfloat16)
            tg.append((A, Bm))
        hs = m.molora_hotset_init(tg, 2.0)
        del tg
        x = torch.randn(B, 2048, device=dev, generator=gen).to(torch.bfloat16)
        o_in = torch.randn(B, 2048, device=dev, generator=gen).to(torch.bfloat16)
        d_in6 = torch.randn(B, 6144, device=dev, generator=gen).to(torch.bfloat16)
        ins = {"o": o_in, "down": d_in6}
        xs = [ins.get(name, x) for (name, _, _) in targets]
        ys = [torch.randn(B, d_out, device=dev, generator=gen).to(torch.bfloat16) for (_, _, d_out) in targets]
        logits = torch.from_numpy(synth.zipf_logits(5, B, K, sub=L)).to(dev)
        idx = torch.empty(B * k, dtype=torch.int32, device=dev)
        w = torch.empty(B * k, dtype=torch.float32, device=dev)
        meta = (torch.empty(K, dtype=torch.int32, device=dev), torch.empty(K + 1, dtype=torch.int32, device=dev),
                torch.empty(B * k, dtype=torch.int32, device=dev), torch.empty(B * k, dtype=torch.float32, device=dev),
                torch.empty(B * k, dtype=torch.int32, device=dev))
        tids = list(range(len(targets)))
        ws = torch.zeros(max(1, m.molora_apply_multi_workspace(hs, tids, B, k, m.PATH_AUTO, torch.bfloat16)),
                         dtype=torch.uint8, device=dev)
        layer_objs.append((hs, xs, ys, logits, idx, w, meta, ws))
        nbytes += (3 * B * 2048 + B * 6144) * 2 + sum(2 * B * d_out * 2 for (_, _, d_out) in targets)
        nbytes += sum(K * (d_in + d_out) * r * 2 for (_, d_in, d_out) in targets) + logits.numel() * 4
    torch.cuda.synchronize()

    def step():
        # per layer: routing, dispatch, then the 7 projections in one multi-target apply
        for (hs, xs, ys, logits, idx, w, meta, ws) in layer_objs:
            m.molora_route_topk(k, K, logits=logits, idx=idx, w=w, want_flags=False)
            m.molora_dispatch(idx, w, K, k, out=meta)
            m.molora_apply_multi(hs, xs, ys, meta[1], meta[2], meta[3], meta[4], k=k, ys=ys, ws=ws)

    ms, g, stream = graph_ms(torch, step, 20)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    with torch.cuda.stream(stream):
        for a, b in evs:
            a.record(stream)
            g.replay()
            b.record(stream)
    torch.cuda.synchronize()
    lat = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    out = {"workload": f"{layers} layers x 7 Qwen3-1.7B projections, decode batch {B}, K={K} r={r} k={k}",
           "p50_us": lat[len(lat) // 2], "p99_us": lat[min(len(lat) - 1, int(0.99 * len(lat)))],
           "cv": statistics.pstdev(lat) / statistics.mean(lat), "replays": replays,
           "mean_us": statistics.mean(lat), "compulsory_bytes": nbytes,
           "roofline_frac_at_p50": nbytes / (lat[len(lat) // 2] * 1e-6) / (HBM_PEAK_GBS * 1e9)}
    del g, layer_objs
    return out


def cpu_baseline(case, seconds, threads=None):
    """The CPU oracle as it stands (fp64 numpy), timed on this host on the same workload:
    route_vocab -> dispatch -> apply for the full batch, repeated for about `seconds`, with the
    BLAS pool at `threads` threads (None: as configured, normally all cores)."""
    import contextlib
    from oracle import apply, bf16_to_f64, dispatch, route_vocab
    t = case.targets[0]
    x, A, B, y0 = (bf16_to_f64(v) for v in (t.x, t.A, t.B, t.y0))  # conversion excluded
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover - threadpoolctl is installed here
        threadpool_info = threadpool_limits = None
    limit = threadpool_limits(limits=threads) if (threads and threadpool_limits) else contextlib.nullcontext()
    with limit:
        if threadpool_info is not None:
            used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        else:
            used = threads or os.cpu_count()

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
    return {"value": case.N / med, "unit": "routed tokens/s", "cores": used, "kind": "oracle",
            "sample": f"full batch (N={case.N}) route+dispatch+apply, {len(times)} runs, median {med * 1e3:.1f} ms",
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
