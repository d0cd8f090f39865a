#!/usr/bin/env python3
"""Benchmark of the DMS decode hot path on one MI355X.

One step = one decode step of every sequence of the workload through the C
ABI: dms_decode_step (decide, retire, store, then attention over the visible
tokens; in whole-unit mode a single launch, in split mode the attention and
the split merge that also appends).  `--path calls` times dms_append_step +
dms_decode_attention instead.  Inputs are synthetic, generated in HBM before
the timed region; after the prompt's compression dms_cache_balance plans the
attention's work split.  The default workload is the Qwen-R1-32B-shaped
layer: 64 chains at 32768 tokens, 40 query / 8 KV heads, head_dim 128, bf16,
w = 256, logit mean for CR 4 below position 10240 and CR 12 beyond (overall
about 8).

Prints one JSON line.  `value` is decode tokens per second (batch sequences
per step); the live-KV bandwidth of the step's kernels is in `roofline`,
timed on every 8th step of the timed region with HIP events that the runtime
stamps at the call's own kernels (dms_decode_step_timed).  A workload whose
live KV per step would fit in the MALL rotates over enough independent caches
that every step reads HBM, and reports the one-cache figure beside it.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --workload qwen-r1-32b-layer-dense --no-cpu-baseline
        # the dense baseline (nothing evicted, CR 1) through the same kernels
    python bench.py --workload qwen-r1-32b-layer-head-skew [--no-balance]
        # per-head compression 2 ... 16 (split mode after balancing)
    python bench.py --workload qwen-r1-7b-layer | llama-3.2-1b-layer
        # MALL-sized layers, caches rotated
    python bench.py --prefill-attention --steps 5 --warmup 1
        # attention of every prompt query (after the prompt's compression)
    python bench.py --chunk 16 --steps 30 --warmup 3
        # several decode steps per call (dms_decode_chunk)
    python bench.py --workload qwen-r1-32b-64-layer-step --steps 16 --warmup 4
        # the whole 64-layer step (256 chains, prompts of 1K-32K tokens)
    python bench.py --hyper-scaling
        # KV budgets of a vanilla generation spent on longer / more DMS chains
    python bench.py --soft-attention
        # training-time relaxed attention, forward + backward
    python bench.py --calib-copy-bytes N    # plain copy, for scaling the HBM byte counters
    python bench.py --calib-read-bytes N    # plain streaming read: the HBM read ceiling
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attention tokens/sec + live-KV HBM GB/s (% of peak) at CR=8, 32K ctx"
HBM_PEAK_GBPS = 8000.0
# MI355X Infinity Cache (MALL): a step whose live KV fits in it is reported as
# cache-resident, its rate is not an HBM rate
MALL_BYTES = 256 * 2**20
# live KV read between two visits of one cache when the bench rotates caches
ROTATE_BYTES = 2**30
# MI355X dense bf16 matrix-core peak (no sparsity)
MFMA_BF16_PEAK_TFLOPS = 2500.0
# the sources that decide a decode call's HBM traffic: the decode kernels, the
# device helpers they share and the runtime that plans their launches
KERNEL_SRCS = [os.path.join(ROOT, "learned_kv_cache_dms_amd", "csrc", f)
               for f in ("dms_device.h", "dms_decode.hip", "dms_runtime.cpp")]


def kernel_source_hash() -> str:
    """First 16 hex digits of the SHA-256 of the decode kernels, their shared
    device helpers and the runtime that plans their launches (together they
    decide the traffic of a decode call)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, path_kind: str = "calls"):
    """HBM bytes per timed call (the fused step, or the attention) from the
    committed counter summary, or None when it is missing or was taken on
    another version of the kernels."""
    name = "decode_step_traffic" if path_kind == "step" else "attention_traffic"
    path = os.path.join(ROOT, "profiles", f"{name}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def calib_copy(nbytes: int):
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": nbytes, "launches": 5}), flush=True)


def calib_read(nbytes: int, reps: int = 20):
    """The HBM read ceiling: a plain streaming read (synth's read_kernel, 16
    bytes per lane, nontemporal, four loads in flight per thread) of nbytes,
    run back to back; for each grid size the mean time per launch over
    `reps` launches bracketed by one event pair, and the best single launch
    (an event pair each).  One JSON line per grid size."""
    import torch
    from synth import device as dsynth
    n = nbytes // 16 * 16
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    for grid in (512, 1024, 2048, 4096):
        sink = torch.empty(grid, dtype=torch.int32, device="cuda")
        for _ in range(3):
            dsynth.stream_read(src, grid, sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            dsynth.stream_read(src, grid, sink)
        b.record()
        torch.cuda.synchronize()
        mean_s = a.elapsed_time(b) / reps / 1e3
        single = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dsynth.stream_read(src, grid, sink)
            e1.record()
            single.append((e0, e1))
        torch.cuda.synchronize()
        best_s = min(x.elapsed_time(y) for x, y in single) / 1e3
        print(json.dumps({"calib_read_bytes": n, "grid": grid, "launches": reps,
                          "mean_us": round(mean_s * 1e6, 2), "mean_gbps": round(n / mean_s / 1e9, 1),
                          "best_us": round(best_s * 1e6, 2), "best_gbps": round(n / best_s / 1e9, 1)}), flush=True)


def cpu_baseline(wl, steps_per_unit: int, n_units: int, layers: int = 1, budget_s: float = 20.0):
    """The oracle, as it is, on a sample of the workload's (layer, sequence,
    KV head) units over its first `layers` layers: `steps_per_unit` decode
    steps each at full context, for up to `n_units` units or until the
    oracle has run `budget_s` seconds (at least one unit).  Input generation
    is outside the timed part."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import dms_oracle as O
    from synth import synth

    rng = np.random.default_rng(wl.seed + 17)
    U = wl.batch * wl.num_kv_heads
    # in the sample's random order, so that a budget cut keeps it unbiased
    units = rng.choice(U * layers, size=min(n_units, U * layers), replace=False).tolist()
    lengths = wl.prompt_lengths()
    G = wl.group
    elapsed = 0.0
    live = 0  # live tokens attended over the sampled steps
    done = 0
    for lu in units:
        if done and elapsed >= budget_s:
            break
        done += 1
        layer, u = divmod(lu, U)
        b, h = divmod(u, wl.num_kv_heads)
        P = int(lengths[b])
        pos = np.arange(P + steps_per_unit)
        K = synth.tensor(wl.seed, synth.STREAM_K, layer, [b], [h], pos, wl.head_dim, wl.dtype)[0, 0]
        V = synth.tensor(wl.seed, synth.STREAM_V, layer, [b], [h], pos, wl.head_dim, wl.dtype)[0, 0]
        lg = synth.logits(wl.seed, layer, [b], [h], pos, *wl.layer_mu(layer), wl.pos_threshold)[0, 0]
        Q = synth.tensor(wl.seed, synth.STREAM_Q, layer, [b], list(range(h * G, (h + 1) * G)),
                         np.arange(P, P + steps_per_unit), wl.head_dim, wl.dtype)[0].transpose(1, 0, 2)
        t0 = time.perf_counter()
        recs = O.decode_unit(Q, K, V, lg, P, steps_per_unit, wl.window, O.default_scale(wl.head_dim))
        elapsed += time.perf_counter() - t0
        live += sum(len(r.visible) for r in recs)
    units = units[:done]
    per_unit_step = elapsed / (len(units) * steps_per_unit)
    step_s = per_unit_step * U * layers             # a full decode step of the workload
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": wl.batch / step_s,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(units)} of {U * layers} ({'layer, ' if layers > 1 else ''}sequence, KV head) units x "
                  f"{steps_per_unit} decode steps at full context ({elapsed:.1f} s of oracle time), "
                  f"scaled to all units",
        "seconds_per_step": step_s,
        # the live K/V bytes of the workload's dtype attended per second, as the metric counts them
        "live_kv_gbps": live * 2 * wl.head_dim * (2 if wl.dtype == "bf16" else 4) / elapsed / 1e9,
        "host_cores_available": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
    }


def cpu_baseline_prompt(wl, n_units: int, n_queries: int):
    """The oracle's prompt attention (each query over its visible set, the
    oracle's own visible + attend) on sampled (sequence, KV head) units and
    sampled prompt queries of each, every query head of the group: algorithmic
    TFLOP/s at 4 d flops per visible (query, key) pair and head."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import dms_oracle as O
    from synth import synth

    rng = np.random.default_rng(wl.seed + 23)
    U = wl.batch * wl.num_kv_heads
    units = sorted(rng.choice(U, size=min(n_units, U), replace=False).tolist())
    lengths = wl.prompt_lengths()
    G, d = wl.group, wl.head_dim
    scale = O.default_scale(d)
    elapsed, pairs, nq = 0.0, 0, 0
    for u in units:
        b, h = divmod(u, wl.num_kv_heads)
        P = int(lengths[b])
        pos = np.arange(P)
        K = synth.tensor(wl.seed, synth.STREAM_K, 0, [b], [h], pos, d, wl.dtype)[0, 0]
        V = synth.tensor(wl.seed, synth.STREAM_V, 0, [b], [h], pos, d, wl.dtype)[0, 0]
        lg = synth.logits(wl.seed, 0, [b], [h], pos, *wl.layer_mu(0), wl.pos_threshold)[0, 0]
        qs = np.sort(rng.choice(P, size=min(n_queries, P), replace=False))
        Q = synth.tensor(wl.seed, synth.STREAM_Q, 0, [b], list(range(h * G, (h + 1) * G)), qs, d,
                         wl.dtype)[0]                       # [G, n, d]
        alpha = O.eviction_decision(lg)
        t0 = time.perf_counter()
        for i, q in enumerate(qs):
            vis = O.visible(alpha, int(q), wl.window)
            O.attend(Q[:, i], K[vis], V[vis], scale)
            pairs += len(vis) * G
        elapsed += time.perf_counter() - t0
        nq += len(qs)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": 4.0 * d * pairs / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{nq} prompt queries (x {G} query heads) from {len(units)} of {U} (sequence, KV head) "
                  f"units, {pairs} visible (query, key) pairs ({elapsed:.1f} s of oracle time)",
        "host_cores_available": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def visible_pairs(Ld, lengths, w: int, G: int) -> int:
    """Visible (query, key) pairs of every prompt query of every query head:
    for query q, the unmarked positions below q - w plus the min(q + 1, w + 1)
    positions of its window (counted from the logits on the device)."""
    import torch
    B, Hkv, T = Ld.shape
    L = torch.as_tensor(lengths, device=Ld.device).view(B, 1, 1)
    pos = torch.arange(T, device=Ld.device).view(1, 1, T)
    unmarked = ((Ld <= 0) | torch.isnan(Ld)) & (pos < L)
    cu = torch.cumsum(unmarked.to(torch.int64), dim=-1)            # unmarked in [0, i]
    # far part of query q: cu[q - w - 1]; summed over q < P: sum of cu[i], i <= P - w - 2
    far = torch.where(pos <= L - w - 2, cu, torch.zeros_like(cu)).sum()
    near = torch.where(pos < L, torch.clamp(pos + 1, max=w + 1), torch.zeros_like(pos)).sum() * Hkv
    return int((far + near).item()) * G


def bench_prefill_attention(args):
    """dms_prefill_attention on the workload's prompt (after its compression):
    algorithmic TFLOP/s = 4 d flops per visible (query, key) pair (q.k and
    p.v, 2 d each) over the mean event time of the call."""
    import numpy as np
    import torch
    from learned_kv_cache_dms_amd import dms
    from synth import device as dsynth
    from synth import synth, workloads

    torch.cuda.set_device(0)
    wl = workloads.ALL[args.workload]()
    B, Hq, Hkv, d = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    lengths = wl.prompt_lengths()
    max_len = int(lengths.max())
    cache = dms.Cache(B, Hq, Hkv, d, wl.window, wl.max_tokens(), wl.pool_blocks(0), dtype=wl.dtype)
    Kd = torch.empty((B, Hkv, max_len, d), dtype=tdt, device="cuda")
    Vd = torch.empty_like(Kd)
    Ld = torch.empty((B, Hkv, max_len), dtype=torch.float32, device="cuda")
    Qd = torch.empty((B, Hq, max_len, d), dtype=tdt, device="cuda")
    mb, ma = wl.layer_mu(0)
    dsynth.fill(Kd, wl.seed, synth.STREAM_K, 0, 0)
    dsynth.fill(Vd, wl.seed, synth.STREAM_V, 0, 0)
    dsynth.fill(Qd, wl.seed, synth.STREAM_Q, 0, 0)
    dsynth.logits(Ld, wl.seed, 0, 0, mb, ma, wl.pos_threshold)
    cache.prefill(Kd, Vd, Ld, lengths)
    out = torch.empty((B, Hq, max_len, d), dtype=torch.float32, device="cuda")
    pairs = visible_pairs(Ld, lengths, wl.window, Hq // Hkv)
    causal = int(sum(int(P) * (int(P) + 1) // 2 for P in lengths)) * Hq
    flops = 4.0 * d * pairs
    torch.cuda.synchronize()
    W, K = args.warmup, args.steps
    for _ in range(W):
        cache.prefill_attention(Qd, Kd, Vd, out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        cache.prefill_attention(Qd, Kd, Vd, out)
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    mean_s = sum(ms) / K / 1e3
    tflops = flops / mean_s / 1e12
    res = {
        "metric": "DMS-masked prompt attention, algorithmic TFLOP/s (every prompt query over its visible set)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(mean_s * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "prompt": max_len, "window": wl.window},
        "visible_pairs": pairs, "causal_pairs": causal, "visible_fraction": round(pairs / causal, 4),
        "prompt_tokens_per_s": round(float(np.sum(lengths)) / mean_s, 1),
        "ms_median": round(statistics.median(ms), 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "dms_prefill_attention = prefill_attention_kernel",
                     "algorithmic_flops_per_launch": flops},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prompt(wl, 8, 512)
    print(json.dumps(res), flush=True)


def bench_soft_attention(args):
    """Training-time relaxed attention (dms_soft_attention_forward, then
    dms_soft_attention_backward) on the Qwen-R1-32B-shaped training layer.
    Algorithmic flops per causal (query, key) pair and head: 4 d forward (q.k,
    p.v) and 8 d backward (dP = dO v^T, dq, dk, dv; the recomputed scores are
    not counted).  Forward and backward are timed with HIP events on the
    stream the library launches on; the step is one of each."""
    import numpy as np
    import torch
    from learned_kv_cache_dms_amd import dms
    from synth import workloads

    torch.cuda.set_device(0)
    wl = workloads.qwen_32b_train()
    B, Hq, Hkv, T, d, w = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.seq_len, wl.head_dim, wl.window
    q, k, v, do, logit, noise = wl.device_inputs()
    out = torch.empty((B, Hq, T, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(dms.dms_soft_attention_backward_workspace_bytes(B, Hq, Hkv, T, d), dtype=torch.uint8,
                     device="cuda")
    fws = torch.empty(dms.dms_soft_attention_forward_workspace_bytes(B, Hq, Hkv, T, d), dtype=torch.uint8,
                      device="cuda")
    pairs = wl.causal_pairs()
    f_fwd, f_bwd = 4.0 * d * pairs, 8.0 * d * pairs

    def fwd():
        dms.soft_attention_forward(q, k, v, logit, noise, w, wl.gamma, wl.tau, out=out, lse=lse, workspace=fws)

    def bwd():
        return dms.soft_attention_backward(q, k, v, logit, noise, out, lse, do, w, wl.gamma, wl.tau, workspace=ws)

    W, K = args.warmup, args.steps
    for _ in range(W):
        fwd()
        bwd()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(s)
        fwd()
        e[1].record(s)
        bwd()
        e[2].record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_f = [a.elapsed_time(b) for a, b, _ in ev]
    ms_b = [b.elapsed_time(c) for _, b, c in ev]
    mf, mb = sum(ms_f) / K / 1e3, sum(ms_b) / K / 1e3
    tf_f, tf_b = f_fwd / mf / 1e12, f_bwd / mb / 1e12
    tf_all = (f_fwd + f_bwd) / (mf + mb) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import dms_oracle as O
        sample = [(b, h) for b in (0, B - 1) for h in range(0, Hkv, 2)]
        t1 = time.perf_counter()
        for (b, h) in sample:
            Q, K_, V, dO, lg, g = wl.host_slice([b], [h])
            O.soft_attention(Q, K_, V, lg, g, w, wl.gamma, wl.tau)
            O.soft_attention_grads(Q, K_, V, lg, g, dO, w, wl.gamma, wl.tau)
        secs = time.perf_counter() - t1
        G = Hq // Hkv
        cpu_flops = 12.0 * d * len(sample) * G * T * (T + 1) // 2
        cpu = {"value": round(cpu_flops / secs / 1e12, 5), "unit": "TFLOP/s", "cores": torch.get_num_threads(),
               "kind": "oracle",
               "sample": f"forward + gradients of {len(sample)} KV heads x {G} query heads x {T} tokens "
                         f"(float64 numpy, {secs:.1f} s incl. input generation)"}
    res = {
        "metric": "relaxed DMS attention forward + backward, algorithmic TFLOP/s (training layer)",
        "value": round(tf_all, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round((mf + mb) * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "seq_len": T, "window": w, "tau": wl.tau, "gamma": wl.gamma},
        "forward_ms": round(mf * 1e3, 4), "backward_ms": round(mb * 1e3, 4),
        "forward_tflops": round(tf_f, 2), "backward_tflops": round(tf_b, 2),
        "tokens_per_s": round(B * T / (mf + mb), 1), "causal_pairs": pairs, "wall_s": round(wall, 3),
        "roofline": {"bound": "mfma", "achieved": round(tf_b, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_b / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "dms_soft_attention_backward (pack, dq, dkv launches)",
                     "algorithmic_flops_per_launch": f_bwd},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_hyper_scaling(args):
    """The hyper-scaling harness: the vanilla generation (8 chains x 16384
    tokens after a 1024-token prompt, nothing evicted) sets a KV memory-read
    budget and a peak-token budget; the DMS budget model picks the longest
    generation per chain count within each; the vanilla run and three DMS
    frontier points run end to end on the GPU, and their device-counted reads
    are checked against the count implied by their decisions."""
    import numpy as np
    import torch
    from learned_kv_cache_dms_amd import hyperscale as H
    from synth import workloads

    torch.cuda.set_device(0)
    wl = workloads.ALL["qwen-r1-32b-hyperscale"]()
    P, L0, W0 = wl.prompt_len, wl.decode_steps, wl.batch
    max_len = 4 * L0
    vanilla_model = H.BudgetModel(lambda pos: np.zeros(len(pos)), wl.window, P, max_len)
    dms_model = H.BudgetModel(lambda pos: wl.marked_prob(0, pos), wl.window, P, max_len)
    base = vanilla_model.config(W0, L0)
    widths = [8, 16, 32, 64, 128, 256]
    fr = {kind: H.frontier(dms_model, budget, kind, widths)
          for kind, budget in (("reads", base.reads), ("peak", base.peak))}
    picks = [("reads", 8), ("reads", 64), ("peak", 32)]
    dense = dataclasses.replace(wl, mu_before=[-8.0], mu_after=None, pos_threshold=wl.pos_threshold)
    runs = []
    r = H.run_config(dense, W0, L0)
    runs.append(("vanilla", W0, L0, r))
    print(f"# vanilla {W0} x {L0}: {r.seconds:.3f} s, reads {r.reads_device} (exact {r.reads_exact})",
          file=sys.stderr, flush=True)
    for kind, wd in picks:
        c = next(x for x in fr[kind] if x.width == wd)
        r = H.run_config(wl, c.width, c.length)
        runs.append((f"dms-{kind}-budget", c.width, c.length, r))
        print(f"# dms {kind} {c.width} x {c.length}: {r.seconds:.3f} s, reads {r.reads_device} "
              f"(exact {r.reads_exact})", file=sys.stderr, flush=True)
    Hkv = wl.num_kv_heads
    van = runs[0][3]
    out_runs = []
    for name, wd, ln, rr in runs:
        out_runs.append({
            "run": name, "chains": wd, "tokens_per_chain": ln, "tokens": wd * ln,
            "decode_s": round(rr.seconds, 4), "tokens_per_s": round(rr.tokens_per_s, 1),
            "reads_per_kv_head": rr.reads_device / Hkv, "reads_exact_match": rr.reads_device == rr.reads_exact,
            "peak_per_kv_head": rr.peak_device / Hkv, "peak_exact_match": rr.peak_device == rr.peak_exact,
            "reads_vs_budget": round(rr.reads_device / Hkv / base.reads, 4),
            "peak_vs_budget": round(rr.peak_device / Hkv / base.peak, 4),
            "kv_gbps": round(rr.kv_bytes_read / rr.seconds / 1e9, 1),
            "tokens_vs_vanilla": round(wd * ln / (W0 * L0), 3),
            "time_vs_vanilla": round(rr.seconds / van.seconds, 3),
        })
    best = out_runs[2]   # 64 chains within the vanilla read budget
    res = {
        "metric": "hyper-scaling: tokens generated within the vanilla KV memory-read budget, DMS / vanilla",
        "value": best["tokens_vs_vanilla"], "unit": "x", "n_gpus": 1, "steps": int(sum(x["tokens_per_chain"] for x in out_runs)),
        "warmup": 0, "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "prompt": P, "vanilla_chains": W0, "vanilla_tokens_per_chain": L0,
                   "q_heads": wl.num_q_heads, "kv_heads": Hkv, "head_dim": wl.head_dim, "window": wl.window},
        "budget_reads_per_kv_head": base.reads, "budget_peak_per_kv_head": base.peak,
        "frontier": {k: [{"chains": c.width, "tokens_per_chain": c.length, "tokens": c.tokens,
                          "tokens_vs_vanilla": round(c.tokens / base.tokens, 3)} for c in v] for k, v in fr.items()},
        "runs": out_runs,
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def bench_chunk(args):
    """dms_decode_chunk on the workload: after the prompt, chunks of C
    tokens per sequence, each call timed with HIP events.  Live-KV bytes of a
    call = the cached tokens it reads (the live count before the chunk) plus
    the chunk's own rows, 2 d sizeof(dtype) each."""
    import torch
    from learned_kv_cache_dms_amd import dms
    from synth import device as dsynth
    from synth import synth, workloads

    torch.cuda.set_device(0)
    wl0 = workloads.ALL[args.workload]()
    C, W, K = args.chunk, args.warmup, args.steps
    wl = dataclasses.replace(wl0, decode_steps=C * (W + K))
    B, Hq, Hkv, d = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    esize = 2 if wl.dtype == "bf16" else 4
    lengths = wl.prompt_lengths()
    max_len = int(lengths.max())
    cache = dms.Cache(B, Hq, Hkv, d, wl.window, wl.max_tokens(), wl.pool_blocks(0), dtype=wl.dtype)
    Kd = torch.empty((B, Hkv, max_len, d), dtype=tdt, device="cuda")
    Vd = torch.empty_like(Kd)
    Ld = torch.empty((B, Hkv, max_len), dtype=torch.float32, device="cuda")
    mb, ma = wl.layer_mu(0)
    dsynth.fill(Kd, wl.seed, synth.STREAM_K, 0, 0)
    dsynth.fill(Vd, wl.seed, synth.STREAM_V, 0, 0)
    dsynth.logits(Ld, wl.seed, 0, 0, mb, ma, wl.pos_threshold)
    cache.prefill(Kd, Vd, Ld, lengths)
    torch.cuda.synchronize()
    del Kd, Vd, Ld
    n_calls = W + K
    base = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    qs = torch.empty((n_calls, B, Hq, C, d), dtype=tdt, device="cuda")
    ks = torch.empty((n_calls, B, Hkv, C, d), dtype=tdt, device="cuda")
    vs = torch.empty_like(ks)
    lgs = torch.empty((n_calls, B, Hkv, C), dtype=torch.float32, device="cuda")
    for i in range(n_calls):
        dsynth.fill(qs[i], wl.seed, synth.STREAM_Q, 0, 0, pos_base=base + i * C)
        dsynth.fill(ks[i], wl.seed, synth.STREAM_K, 0, 0, pos_base=base + i * C)
        dsynth.fill(vs[i], wl.seed, synth.STREAM_V, 0, 0, pos_base=base + i * C)
        dsynth.logits(lgs[i], wl.seed, 0, 0, mb, ma, wl.pos_threshold, pos_base=base + i * C)
    out = torch.empty((B, Hq, C, d), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for i in range(W):
        cache.decode_chunk(qs[i], ks[i], vs[i], lgs[i], out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    live_before = []
    torch.cuda.synchronize()
    for i in range(K):
        live_before.append(cache.stats()["live_tokens"])
        ev[i][0].record()
        cache.decode_chunk(qs[W + i], ks[W + i], vs[W + i], lgs[W + i], out)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    mean_s = sum(ms) / K / 1e3
    kv_bytes = (sum(live_before) / K + B * Hkv * C) * 2 * d * esize
    gbps = kv_bytes / mean_s / 1e9
    res = {
        "metric": "chunked decode tokens/sec (dms_decode_chunk, C tokens per sequence per call)",
        "value": round(B * C / mean_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(mean_s * 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "context": max_len, "window": wl.window, "chunk": C},
        "ms_median": round(statistics.median(ms), 5),
        "live_kv_gbps": round(gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "dms_decode_chunk = chunk_attention_kernel + append_chunk_kernel",
                     "algorithmic_bytes_per_launch": round(kv_bytes)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        # a chunk of C tokens computes what C decode steps do: the oracle's
        # step-by-step decode is the baseline, in tokens/s
        cpu = cpu_baseline(wl0, args.cpu_steps, args.cpu_units, budget_s=args.cpu_seconds)
        cpu["sample"] += f" (a chunk of {C} tokens = {C} decode steps)"
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


def bench_full_step(args):
    """A multi-layer decode step: one cache per layer, every timed step runs
    the decode step of every layer in order (as a model would): one
    dms_decode_step per layer (--path step) or dms_append_step +
    dms_decode_attention (--path calls).  Each layer's cache is balanced once
    after its prompt.  Tokens/s = batch / (time of one step over all layers)."""
    import torch
    from learned_kv_cache_dms_amd import dms
    from synth import device as dsynth
    from synth import synth, workloads

    torch.cuda.set_device(0)
    wl0 = workloads.ALL[args.workload]()
    W, K = args.warmup, args.steps
    wl = dataclasses.replace(wl0, decode_steps=W + K)
    B, Hq, Hkv, d, NL = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_layers
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    esize = 2 if wl.dtype == "bf16" else 4
    lengths = wl.prompt_lengths()
    max_len = int(lengths.max())
    caches = []
    for l in range(NL):
        c = dms.Cache(B, Hq, Hkv, d, wl.window, wl.max_tokens(), wl.pool_blocks(l, slack=1.1), dtype=wl.dtype)
        Kd = torch.empty((B, Hkv, max_len, d), dtype=tdt, device="cuda")
        Vd = torch.empty_like(Kd)
        Ld = torch.empty((B, Hkv, max_len), dtype=torch.float32, device="cuda")
        mb, ma = wl.layer_mu(l)
        dsynth.fill(Kd, wl.seed, synth.STREAM_K, l, 0)
        dsynth.fill(Vd, wl.seed, synth.STREAM_V, l, 0)
        dsynth.logits(Ld, wl.seed, l, 0, mb, ma, wl.pos_threshold)
        c.prefill(Kd, Vd, Ld, lengths)
        c.balance()
        del Kd, Vd, Ld
        caches.append(c)
        if l % 16 == 15:
            torch.cuda.synchronize()
            print(f"# {l + 1} layers prefilled", file=sys.stderr, flush=True)
    S = W + K
    base = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    qs = torch.empty((S, NL, B, Hq, d), dtype=tdt, device="cuda")
    ks = torch.empty((S, NL, B, Hkv, d), dtype=tdt, device="cuda")
    vs = torch.empty_like(ks)
    lgs = torch.empty((S, NL, B, Hkv), dtype=torch.float32, device="cuda")
    for t in range(S):
        for l in range(NL):
            mb, ma = wl.layer_mu(l)
            dsynth.fill(qs[t, l], wl.seed, synth.STREAM_Q, l, 0, pos_base=base + t)
            dsynth.fill(ks[t, l], wl.seed, synth.STREAM_K, l, 0, pos_base=base + t)
            dsynth.fill(vs[t, l], wl.seed, synth.STREAM_V, l, 0, pos_base=base + t)
            dsynth.logits(lgs[t, l], wl.seed, l, 0, mb, ma, wl.pos_threshold, pos_base=base + t)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    def layer_step(t, l, timer=None):
        c = caches[l]
        if args.path == "step":
            if timer is None:
                c.step(qs[t, l], ks[t, l], vs[t, l], lgs[t, l], out)
            else:
                c.step_timed(qs[t, l], ks[t, l], vs[t, l], lgs[t, l], timer, out)
        else:
            c.append(ks[t, l], vs[t, l], lgs[t, l])
            if timer is None:
                c.attend(qs[t, l], out)
            else:
                c.attend_timed(qs[t, l], timer, out)

    for t in range(W):
        for l in range(NL):
            layer_step(t, l)
    st0 = [c.stats() for c in caches]
    # every layer call of every N-th step timed by kernel-stamped events
    N = max(1, args.event_every)
    sampled = list(range(0, K, N))
    ev = {(i, l): dms.KernelTimer() for i in sampled for l in range(NL)}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        t = W + i
        for l in range(NL):
            layer_step(t, l, ev.get((i, l)))
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st1 = [c.stats() for c in caches]
    if any(x["sticky_error"] for x in st1):
        raise SystemExit("device error during the run")
    total_ms = start.elapsed_time(end)
    attn_s = sum(tm.elapsed_ms() for tm in ev.values()) / 1e3 * K / len(sampled)  # timed calls, scaled to K steps
    for tm in ev.values():
        tm.close()
    split_layers = sum(1 for c in caches if c.split_mode())
    live_tokens = sum(b["live_token_steps"] - a["live_token_steps"] for a, b in zip(st0, st1)) / K
    live_bytes = live_tokens * 2 * d * esize                        # per step, all layers
    step_s = total_ms / K / 1e3
    achieved = live_bytes * K / attn_s / 1e9
    seen = sum(x["seen_tokens"] for x in st1)
    live_now = sum(x["live_tokens"] for x in st1)
    res = {
        "metric": METRIC, "value": round(B / step_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(total_ms / K, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "layers": NL, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "prompt_lengths": [int(lengths.min()), int(lengths.max())], "window": wl.window,
                   "decode_steps": S},
        "live_kv_gbps": round(achieved, 1), "live_kv_gbps_per_step": round(live_bytes / step_s / 1e9, 1),
        "pct_peak_hbm": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "timed_kernels_ms_per_layer": round(attn_s / (K * NL) * 1e3, 5),
        "path": args.path, "layers_in_split_mode": split_layers,
        "live_bytes_per_step": round(live_bytes), "realized_cr": round(seen / live_now, 3),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": ("dms_decode_step per layer (fused append + attention launch in whole-unit mode)"
                                if args.path == "step" else
                                "dms_decode_attention per layer = attention_kernel (+ reduce_kernel in split mode)"),
                     "algorithmic_bytes_per_launch": round(live_bytes / NL)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        # (layer, sequence, KV head) units drawn from every layer, scaled to all
        # layers' units: the oracle's time for one decode step of the model
        res["cpu_baseline"] = cpu_baseline(wl0, args.cpu_steps, args.cpu_units, layers=NL, budget_s=args.cpu_seconds)
    print(json.dumps(res), flush=True)


def _mu_json(mu):
    import numpy as np
    a = np.asarray(mu, dtype=np.float64)
    return round(float(a), 4) if a.ndim == 0 else [round(float(x), 4) for x in a]


def bench_decode(args):
    """The decode step of a one-layer workload: every timed step is one
    dms_decode_step (--path step: the append fused into the attention launch
    in whole-unit mode) or dms_append_step + dms_decode_attention (--path
    calls), on every sequence.  After the prompt's compression the cache is
    balanced once (dms_cache_balance).  A step whose live KV would fit in the
    MALL rotates over k independent caches (k x live bytes >= 1 GB), so that
    every step reads its cache from HBM; the same workload without rotation is
    reported beside it as the cache-resident figure."""
    import math

    import torch

    from learned_kv_cache_dms_amd import dms
    from synth import device as dsynth
    from synth import synth, workloads

    wl0 = workloads.ALL[args.workload]()
    W, K = args.warmup, args.steps
    B, Hq, Hkv, d = wl0.batch, wl0.num_q_heads, wl0.num_kv_heads, wl0.head_dim
    tdt = torch.bfloat16 if wl0.dtype == "bf16" else torch.float32
    esize = 2 if wl0.dtype == "bf16" else 4
    lengths = wl0.prompt_lengths()
    max_len = int(lengths.max())
    # expected live bytes of a step, for the rotation count
    est_bytes = sum(wl0.expected_live(0, int(lengths[b]) + wl0.decode_steps // 2, h)
                    for b in range(B) for h in range(Hkv)) * 2 * d * esize
    rot = args.rotate if args.rotate > 0 else (1 if est_bytes >= MALL_BYTES else
                                               int(math.ceil(ROTATE_BYTES / est_bytes)))
    S = W + K
    local_steps = -(-S // rot)  # steps each cache takes
    wl = dataclasses.replace(wl0, decode_steps=local_steps)
    src, ch = args.logit_source, args.logit_channel
    G = Hq // Hkv
    if src != "array" and args.path != "calls":
        raise SystemExit("--logit-source k|q is timed with --path calls")
    print(f"# workload {wl.name}: prompt {max_len}, {W}+{K} steps over {rot} cache(s), pool {wl.pool_blocks(0)} "
          f"blocks each, path {args.path}", file=sys.stderr, flush=True)
    mb, ma = wl.layer_mu(0)
    Kd = torch.empty((B, Hkv, max_len, d), dtype=tdt, device="cuda")
    Vd = torch.empty_like(Kd)
    Ld = torch.empty((B, Hkv, max_len), dtype=torch.float32, device="cuda")
    dsynth.fill(Kd, wl.seed, synth.STREAM_K, 0, 0)
    dsynth.fill(Vd, wl.seed, synth.STREAM_V, 0, 0)
    dsynth.logits(Ld, wl.seed, 0, 0, mb, ma, wl.pos_threshold)
    if src == "k":
        Kd[..., ch] = Ld.to(tdt)
    Qp = None
    if src == "q":
        Qp = torch.zeros((B, Hq, max_len, d), dtype=tdt, device="cuda")
        Qp[:, ::G, :, ch] = Ld.to(tdt)
    caches = []
    for r in range(rot):
        c = dms.Cache(B, Hq, Hkv, d, wl.window, wl.max_tokens(), wl.pool_blocks(0), dtype=wl.dtype,
                      split_wgs=args.split_wgs)
        if src == "array":
            c.prefill(Kd, Vd, Ld, lengths)
        elif src == "k":
            c.prefill_channel(Kd, Vd, lengths, source="k", channel=ch, zero=True)
        else:
            c.prefill_channel(Kd, Vd, lengths, source="q", channel=ch, q=Qp)
        if not args.no_balance:
            c.balance()
        caches.append(c)
    torch.cuda.synchronize()
    # The dense prompt stays in torch's cache: returning 17 GB to the HIP runtime
    # (empty_cache) was measured to lower HBM streaming rates by 4-5% for the
    # rest of the process on this platform.
    del Kd, Vd, Ld, Qp

    qs = torch.empty((local_steps, B, Hq, d), dtype=tdt, device="cuda")
    ks = torch.empty((local_steps, B, Hkv, d), dtype=tdt, device="cuda")
    vs = torch.empty_like(ks)
    lgs = torch.empty((local_steps, B, Hkv), dtype=torch.float32, device="cuda")
    base = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    for t in range(local_steps):
        pb = base + t
        dsynth.fill(qs[t], wl.seed, synth.STREAM_Q, 0, 0, pos_base=pb)
        dsynth.fill(ks[t], wl.seed, synth.STREAM_K, 0, 0, pos_base=pb)
        dsynth.fill(vs[t], wl.seed, synth.STREAM_V, 0, 0, pos_base=pb)
        dsynth.logits(lgs[t], wl.seed, 0, 0, mb, ma, wl.pos_threshold, pos_base=pb)
    if src == "k":
        ks[..., ch] = lgs.to(tdt)
    elif src == "q":
        qs[:, :, ::G, ch] = lgs.to(tdt)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step(s, timer=None):
        c, t = caches[s % rot], s // rot
        if args.path == "step":
            if timer is None:
                c.step(qs[t], ks[t], vs[t], lgs[t], out)
            else:
                c.step_timed(qs[t], ks[t], vs[t], lgs[t], timer, out)
            return
        if src == "array":
            c.append(ks[t], vs[t], lgs[t])
        else:
            c.append_channel(ks[t], vs[t], source=src, channel=ch, zero=(src == "k"),
                             q=qs[t] if src == "q" else None)
        if timer is None:
            c.attend(qs[t], out)
        else:
            c.attend_timed(qs[t], timer, out)

    for s in range(W):
        step(s)
    st0 = [c.stats() for c in caches]

    # Every N-th step of the timed region is timed by a pair of HIP events that
    # the runtime stamps with the start and the end of that call's own kernels
    # (the step's launches, or the attention's with --path calls); the steps in
    # between run exactly as the sampled ones.  (Event pairs recorded around
    # the call instead read 1-10 us more than the kernels themselves.)
    N = max(1, args.event_every)
    sampled = list(range(0, K, N))
    ev = {i: dms.KernelTimer() for i in sampled}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        step(W + i, ev.get(i))
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st1 = [c.stats() for c in caches]
    if any(x["sticky_error"] != 0 for x in st1):
        raise SystemExit(f"device error during the run: {st1}")

    total_ms = start.elapsed_time(end)
    kern_ms = [ev[i].elapsed_ms() for i in sampled]
    kern_avg_s = sum(kern_ms) / len(kern_ms) / 1e3
    period_ms = [dms.KernelTimer.between(ev[a], ev[b]) / (b - a) for a, b in zip(sampled, sampled[1:])]
    for tm in ev.values():
        tm.close()
    live_tokens = sum(b["live_token_steps"] - a["live_token_steps"] for a, b in zip(st0, st1)) / K
    live_bytes = live_tokens * 2 * d * esize   # per step: the K/V rows of every visible token
    step_s = total_ms / K / 1e3
    achieved = live_bytes / kern_avg_s / 1e9
    # per call; the same whichever of the rotated caches a call reads
    traffic = measured_traffic(wl.name, args.path)
    seen = sum(x["seen_tokens"] for x in st1)
    live_now = sum(x["live_tokens"] for x in st1)
    kernel = ("dms_decode_step = attention_kernel<fused> (the append inside the attention launch; split mode: "
              "attention_kernel<split step> + reduce_kernel<step>, the merge and the appends)" if args.path == "step" else
              "dms_decode_attention = attention_kernel (+ reduce_kernel in split mode)")
    res = {
        "metric": METRIC,
        "value": round(B / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
            "context": max_len, "window": wl.window, "block_tokens": 16,
            "decode_steps": S, "logit_mean": [_mu_json(mb), _mu_json(ma)], "logit_mean_switch": wl.pos_threshold,
            "logit_source": {"array": "array", "k": f"key channel {ch} (stored zeroed)",
                             "q": f"query channel {ch} of each group's first head"}[src],
            "path": args.path, "caches_rotated": rot, "balanced": not args.no_balance,
        },
        "live_kv_gbps": round(achieved, 1),
        "live_kv_gbps_per_step": round(live_bytes / step_s / 1e9, 1),
        "pct_peak_hbm": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "timed_kernels_ms": round(kern_avg_s * 1e3, 5),
        "timed_kernels_ms_median": round(statistics.median(kern_ms), 5),
        "timed_calls": len(kern_ms),
        "ms_per_step_median": round(statistics.median(period_ms), 5) if period_ms else None,
        "cache_resident": bool(rot == 1 and live_bytes < MALL_BYTES),
        "attention_mode": "split" if caches[0].split_mode() else "whole units",
        "live_tokens_per_step": round(live_tokens, 1),
        "realized_cr": round(seen / live_now, 3),
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None if traffic is None else round(traffic),
            "kernel": kernel,
            "algorithmic_bytes_per_launch": round(live_bytes),
        },
        "cpu_baseline": None,
    }
    for c in caches:
        c.close()
    del caches
    if rot > 1 and not args.no_resident:
        res["cache_resident_run"] = resident_figure(args, wl0)
    if not args.no_cpu_baseline and src == "array":
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_steps, args.cpu_units, budget_s=args.cpu_seconds)
    print(json.dumps(res), flush=True)


def resident_figure(args, wl0):
    """The same decode steps on one cache (its live KV stays in the MALL)."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", wl0.name, "--steps", str(args.steps),
           "--warmup", str(args.warmup), "--rotate", "1", "--path", args.path, "--no-cpu-baseline",
           "--event-every", str(args.event_every)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True, timeout=600)
    if r.returncode != 0:
        return None
    line = json.loads(r.stdout.strip().splitlines()[-1])
    return {"value": line["value"], "ms_per_step": line["ms_per_step"], "live_kv_gbps": line["live_kv_gbps"],
            "note": "one cache, its live KV resident in the 256 MB MALL: not an HBM rate"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="qwen-r1-32b-layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=24)
    ap.add_argument("--cpu-steps", type=int, default=256)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="the oracle baseline stops taking units after this many seconds of oracle time")
    ap.add_argument("--calib-copy-bytes", type=int, default=0,
                    help="plain copy of this many bytes (to scale the HBM byte counters)")
    ap.add_argument("--calib-read-bytes", type=int, default=0,
                    help="plain streaming read of this many bytes: the HBM read ceiling")
    ap.add_argument("--event-every", type=int, default=8,
                    help="decode bench: time every N-th attention call of the timed region with its own "
                         "kernel-stamped event pair (roofline.achieved is their mean)")
    ap.add_argument("--logit-source", choices=("array", "k", "q"), default="array",
                    help="where the append reads the eviction logit: the logit array, or the workload's "
                         "logits (bf16-rounded) planted in channel --logit-channel of the keys (stored "
                         "zeroed) or of each group's first query head")
    ap.add_argument("--logit-channel", type=int, default=0)
    ap.add_argument("--chunk", type=int, default=0,
                    help="time dms_decode_chunk with this many tokens per sequence per call")
    ap.add_argument("--hyper-scaling", action="store_true",
                    help="run the hyper-scaling harness (vanilla budget, DMS frontier, end-to-end runs)")
    ap.add_argument("--soft-attention", action="store_true",
                    help="training-time relaxed attention forward + backward on the 32B-shaped training layer")
    ap.add_argument("--path", choices=("step", "calls"), default="step",
                    help="decode bench: dms_decode_step (step) or dms_append_step + dms_decode_attention (calls)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="decode bench: independent caches used in turn (0: enough for 1 GB of live KV "
                         "when one step's live KV would fit in the MALL, else 1)")
    ap.add_argument("--no-balance", action="store_true",
                    help="decode bench: keep the cache's default work split (skip dms_cache_balance after the prompt)")
    ap.add_argument("--split-wgs", type=int, default=0,
                    help="decode bench: dms_config.split_wgs (0 = the library's choice, 1 = whole units, "
                         ">= 2 = split over that many work-groups at most)")
    ap.add_argument("--no-resident", action="store_true",
                    help="skip the cache-resident (one cache) figure that goes with a rotated run")
    ap.add_argument("--prefill-attention", action="store_true",
                    help="time dms_prefill_attention on the workload's prompt instead of the decode step "
                         "(use small --steps / --warmup: one call is a whole prompt)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the DMS path here runs on one GPU only; "
              f"--gpus {args.gpus} (WORLD_SIZE {world}) is not supported.", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    if args.calib_copy_bytes:
        calib_copy(args.calib_copy_bytes)
        return
    if args.calib_read_bytes:
        calib_read(args.calib_read_bytes)
        return
    if args.prefill_attention:
        bench_prefill_attention(args)
        return
    if args.hyper_scaling:
        bench_hyper_scaling(args)
        return
    if args.soft_attention:
        bench_soft_attention(args)
        return
    if args.chunk:
        bench_chunk(args)
        return

    from synth import workloads

    wl0 = workloads.ALL[args.workload]()
    if wl0.num_layers != 1:
        bench_full_step(args)
        return
    bench_decode(args)


if __name__ == "__main__":
    main()
