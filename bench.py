#!/usr/bin/env python3
"""Sparse decode-step benchmark on one MI355X.

A step is one decode token through a stack of OPT-175B-shaped layers (d 12288, 49152
neurons, 96 heads of 128, 2048 cached positions, predictor width 1024, fp16 weights,
batch 1): per layer LayerNorm, the two sparsity predictors and top-k selection (5% of
neurons, 20% of heads; layer l+1's sets predicted inside layer l's launches),
head-sparse Q/K/V with the KV append, attention over the kept heads, the head-sparse
output projection, LayerNorm, and the sparse MLP.  Every layer has its own weights and
cache, all resident in HBM before timing starts.

Prints one JSON line: HBM GB/s on the bytes the step touches (the value), microseconds
per layer, the dense path on the same stack, the roofline of the dominant kernel
(head-sparse Q/K/V GEMV) measured with HIP events around its launches, and the CPU
oracle timed on a bounded sample of the same workload.

--ablation times the fused sparse MLP against gather-then-dense (the pages' kernel-fusion
claim) at a few keep-percentages.  --sweep instead times OPT-175B-shaped layers over
neuron keep-percentages
{1..100}, head keep-percentages {10..100} and batches {1..32} (union index sets),
with the vector-ALU and the matrix-core kernel forms where both apply and the dense path
per batch, and prints one JSON line per point.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
HEADLINE_METRIC = "sparse decode-layer µs and HBM GB/s (% of peak), OPT-175B shape, 5% MLP/20% heads"
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qkv_p1_launch_opt175b_traffic.txt")
KERNEL_SOURCES = ["common.hpp", "gemv.hpp", "select.hpp", "attn.hpp", "gemv_f16_side.hip", "gemv_own_f16.hip"]


def kernel_sources_sha():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "contextual_sparsity_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter summary
    (rocprofv3 FETCH_SIZE and WRITE_SIZE, calibrated on a copy), or None when the kernel
    sources changed since it was taken."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith(("#", " ", "|")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("sources_sha256") != kernel_sources_sha():
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="opt175b-24layers-fp16")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0: the workload's)")
    ap.add_argument("--batch", type=int, default=0, help="override the batch size (0: the workload's)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget")
    ap.add_argument("--breakdown", action="store_true", help="time every kernel family")
    ap.add_argument("--no-lookahead", action="store_true", help="serial schedule for any workload")
    ap.add_argument("--flush", dest="flush", action="store_true", default=None,
                    help="write a 1 GiB buffer before every timed step (outside its timing) so that no "
                         "weights are served from the 256 MB Infinity Cache or L2 (default for one-layer "
                         "workloads, whose weights would otherwise stay cached between steps)")
    ap.add_argument("--no-flush", dest="flush", action="store_false")
    ap.add_argument("--deterministic", action="store_true",
                    help="bitwise-reproducible lookahead stack (fixed-order reductions, finalize launches)")
    ap.add_argument("--lookahead", action="store_true",
                    help="lookahead schedule for any workload (the single-layer workloads default to "
                         "the serial one: head set from LN(x), neuron set from LN(x'))")
    ap.add_argument("--sweep", action="store_true", help="the keep-percentage x batch sweep")
    ap.add_argument("--sweep-layers", type=int, default=8, help="distinct layers per sweep step")
    ap.add_argument("--sweep-steps", type=int, default=5)
    ap.add_argument("--sweep-batches", default="", help="comma list overriding the sweep's batches")
    ap.add_argument("--sweep-pct-a", default="", help="comma list overriding the head keep-percentages")
    ap.add_argument("--sweep-pct-m", default="", help="comma list overriding the neuron keep-percentages")
    ap.add_argument("--threshold", action="store_true",
                    help="threshold-mode selection: t calibrated on layer 0's scores to the keep "
                         "percentages; one JSON line with the kept-count spread")
    ap.add_argument("--recall", action="store_true",
                    help="the true selection by output norm on every layer of one step: probe time "
                         "and recall of the predicted sets; one JSON line")
    ap.add_argument("--tp", type=int, default=1,
                    help="time one tensor-parallel shard of the workload split over this many GPUs "
                         "(full predictors, the shard's heads and neurons); one JSON line")
    ap.add_argument("--tp-rank", type=int, default=0, help="which shard --tp times")
    ap.add_argument("--ablation", action="store_true",
                    help="the fusion ablation: fused sparse MLP vs gather-then-dense, OPT-175B shape")
    ap.add_argument("--lazy-kv", action="store_true",
                    help="decode steps with n advancing, with and without lazy K/V of skipped heads")
    ap.add_argument("--lazy-steps", type=int, default=16, help="decode steps of --lazy-kv")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB three times (reference for HBM byte "
                         "counters) and exit")
    return ap.parse_args(argv)


def device_facts(torch) -> dict:
    """What the run measured on: name, architecture, compute units, HBM capacity."""
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "compute_units": pr.multi_processor_count,
            "hbm_GiB": round(pr.total_memory / 2**30, 1)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------------ algorithmic bytes
def layer_bytes(s, k_A, k_M):
    """Bytes one sparse layer must touch (weights of the kept units, predictors, the kept
    heads' KV rows); activations are a few KiB and left out."""
    e = 2 if s.dtype == "f16" else 4
    pred = (2 * s.d * s.r + s.r * s.N + s.r * s.h) * e
    qkv = 3 * s.d * s.dh * k_A * e
    o = k_A * s.dh * s.d * e
    kv = s.B * 2 * (s.n + 1) * s.dh * k_A * e
    mlp = 2 * k_M * s.d * e + k_M * e
    return {"pred": pred, "qkv": qkv, "o_proj": o, "kv": kv, "mlp": mlp,
            "total": pred + qkv + o + kv + mlp}


def dense_layer_bytes(s):
    e = 2 if s.dtype == "f16" else 4
    return 4 * s.d * s.h * s.dh * e + 2 * s.N * s.d * e + s.N * e + s.B * 2 * (s.n + 1) * s.h * s.dh * e


# ------------------------------------------------------------------------ CPU oracle baseline
def _cpu_threads_cap() -> int:
    """Host threads the baseline may use: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, s, layers_gpu, preds_gpu, x0, k_A, k_M, budget_s, lb, dense_lb, lookahead=True):
    """The float64 oracle on the host, timed on a bounded sample of the same step, in three
    legs (numpy's BLAS pool held at one thread in each, so a leg uses exactly the threads
    it starts):
      * one core: the stack's layers in order (lookahead or serial sets, as on the GPU),
        until a third of the budget;
      * all cores: P threads (P = the host CPUs this process may use, at most 16), thread i
        running the oracle on layer i % L' of the step from the step's input, L' = min(P, L)
        layers held on the host (fewer threads if host memory is short); numpy releases the interpreter lock inside its array loops, so
        the threads run in parallel.  Throughput = P layers / wall time; the effective
        cores are the process CPU time over the wall time;
      * dense: the dense oracle layer 0 on one core.
    `value` is the faster leg's rate on the sparse layer's touched bytes, `cores` its threads."""
    import numpy as np
    import oracle as O
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    host = lambda t: t.detach().cpu().numpy()
    weights = lambda l: (O.LayerWeights(**{k: host(v) for k, v in layers_gpu[l].items()}),
                         O.PredictorWeights(**{k: host(v) for k, v in preds_gpu[l].items()}))
    sel = O.Selection(O.TOPK, k_A=k_A, k_M=k_M)
    x_in = host(x0).astype(np.float64)

    def sparse_one(x, Lw, Pw, y_src):
        if not lookahead:  # head set from LN(x), neuron set from LN(x') in between
            return O.serial_layer(x, Lw, Pw, sel, s.n, wl.scale)[0]
        S_A, S_M = O.predict_sets(y_src, Pw, sel)
        return O.sparse_layer(x, Lw, S_A, S_M, s.n, wl.scale)[0]

    with threadpool_limits(limits=1):
        # one core: layers in order (the sets of layer l come from LN(x_{l-1})), from layer 0
        # again after the last one while the budget lasts; small layers keep their host copy
        x, prev_y, done, t1 = x_in, None, 0, 0.0
        small = sum(v.numel() * v.element_size() for v in layers_gpu[0].values()) < 2**30
        kept = {}
        while t1 < budget_s / 3 and done < 100000:
            l = done % len(layers_gpu)
            Lw, Pw = kept[l] if l in kept else weights(l)
            if small:
                kept[l] = (Lw, Pw)
            t0 = time.perf_counter()
            y_src = O.layernorm(x) if prev_y is None else prev_y
            prev_y = O.layernorm(x)
            x = sparse_one(x, Lw, Pw, y_src)
            t1 += time.perf_counter() - t0
            done += 1
            del Lw, Pw
        kept.clear()
        one_us = t1 / done * 1e6

        # all cores: thread i runs layer i % L, all host copies made before the clock starts
        P = _cpu_threads_cap()
        nl = min(P, len(layers_gpu))
        try:
            import psutil
            per_layer = sum(v.numel() * v.element_size() for v in layers_gpu[0].values()) * 1.6
            fit = int(psutil.virtual_memory().available * 0.6 // per_layer)
            if fit < nl:
                nl = P = max(1, fit)
        except ImportError:  # pragma: no cover
            pass
        ws = [weights(l) for l in range(nl)]
        y0 = O.layernorm(x_in)
        reps = max(1, round(budget_s / 3 / (one_us * 1e-6) / P))  # layers per thread

        def run(i):
            for _ in range(reps):
                sparse_one(x_in, ws[i % nl][0], ws[i % nl][1], y0)

        c0, w0 = time.process_time(), time.perf_counter()
        with ThreadPoolExecutor(P) as ex:
            list(ex.map(run, range(P)))
        wall = time.perf_counter() - w0
        eff = (time.process_time() - c0) / wall
        del ws
        all_us = wall / (P * reps) * 1e6

        # dense layer 0 on one core
        Lw, _ = weights(0)
        t0 = time.perf_counter()
        O.dense_layer(x_in, Lw, s.n, wl.scale)
        dense_us = (time.perf_counter() - t0) * 1e6
        del Lw
    # the faster leg is the baseline (small layers are interpreter-bound, and their threads
    # mostly wait for one another)
    best_us, best_p = (all_us, P) if all_us < one_us else (one_us, 1)
    return {
        "value": round(lb / (best_us * 1e-6) / 1e9, 4), "unit": "GB/s", "kind": "oracle",
        "cores": best_p, "cores_used": best_p, "all_cores_threads": P,
        "all_cores_effective_cores": round(eff, 2), "host_cpus": os.cpu_count(),
        "us_per_layer": round(best_us, 1),
        "one_core_us_per_layer": round(one_us, 1),
        "all_cores_us_per_layer": round(all_us, 1),
        "dense_us_per_layer": round(dense_us, 1),
        "dense_GBps": round(dense_lb / (dense_us * 1e-6) / 1e9, 4),
        "sample": f"float64 numpy oracle ({'lookahead' if lookahead else 'serial'} sets), BLAS at one "
                  f"thread per thread: {done} layers of the step in "
                  f"order (from layer 0 again after the last) on one core ({t1:.1f} s); {P} threads at once, "
                  f"thread i running layer i % {nl} {reps} times from the step's input ({wall:.1f} s wall, {eff:.1f} cores "
                  f"busy on average); the dense "
                  f"layer 0 on one core ({dense_us * 1e-6:.1f} s)",
    }


# ------------------------------------------------------------------------ fusion ablation
def ablation(args) -> int:
    """Fused gather-and-multiply (the library's sparse MLP, kept rows read in place) against
    the unfused form: kept W1 rows, b1 entries and W2 rows gathered into contiguous copies,
    then the dense MLP over the copies (three passes over the kept bytes instead of one)."""
    import torch
    from contextual_sparsity_amd import configs, synth
    from contextual_sparsity_amd import dejavu as dj

    base = configs.WORKLOADS["opt175b-1layer-fp16"]
    s = base.shape
    dev = "cuda"
    w = synth.make_layer(s, args.seed, 0, dev)
    x = synth.make_input(s, args.seed, dev)
    y = torch.empty_like(x)
    dj.dejavu_layernorm(1, s.d, x, y, 1e-5)
    ws = dj.workspace(dj.dejavu_workspace_bytes(1, s.d, s.N, s.h, s.dh, s.r, s.cap), dev)
    out = torch.empty_like(x)
    e = 2
    for pct in (1, 5, 10, 25):
        k = configs.keep(pct, s.N)
        g = torch.Generator(device="cpu").manual_seed(args.seed + pct)
        S = torch.randperm(s.N, generator=g)[:k].sort().values.to(torch.int32).to(dev)
        cnt = torch.tensor([k], dtype=torch.int32, device=dev)
        W1g = torch.empty(k, s.d, dtype=torch.float16, device=dev)
        W2g = torch.empty_like(W1g)
        b1g = torch.empty(k, dtype=torch.float16, device=dev)

        def fused():
            dj.dejavu_sparse_mlp(dj.DJV_F16, 1, s.d, s.N, y, w["W1"], w["b1"], w["W2"], S, cnt, k, x, out, ws)

        def unfused():
            dj.dejavu_gather_rows(dj.DJV_F16, 1, s.d, s.N, w["W1"], S, cnt, k, W1g)
            dj.dejavu_gather_rows(dj.DJV_F16, 1, 1, s.N, w["b1"], S, cnt, k, b1g)
            dj.dejavu_gather_rows(dj.DJV_F16, 1, s.d, s.N, w["W2"], S, cnt, k, W2g)
            dj.dejavu_dense_mlp(dj.DJV_F16, 1, s.d, k, y, W1g, b1g, W2g, x, out, ws)

        def gather_only():
            dj.dejavu_gather_rows(dj.DJV_F16, 1, s.d, s.N, w["W1"], S, cnt, k, W1g)
            dj.dejavu_gather_rows(dj.DJV_F16, 1, 1, s.N, w["b1"], S, cnt, k, b1g)
            dj.dejavu_gather_rows(dj.DJV_F16, 1, s.d, s.N, w["W2"], S, cnt, k, W2g)

        def timed(f, n=30):
            for _ in range(3):
                f()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                f()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / n

        kept = 2 * k * s.d * e + k * e
        t_f, t_u, t_g = timed(fused), timed(unfused), timed(gather_only)
        pt = {"ablation": "fused gather-multiply vs gather then dense", "workload": "opt175b MLP, fp16, B 1",
              "pct_M": pct, "k_M": k, "kept_bytes": kept,
              "fused_us": round(t_f, 2), "fused_bytes": kept, "fused_GBps": round(kept / (t_f * 1e-6) / 1e9, 1),
              "unfused_us": round(t_u, 2), "unfused_bytes": 3 * kept, "gather_us": round(t_g, 2),
              "speedup_fused": round(t_u / t_f, 3)}
        print(json.dumps(pt), flush=True)
    return 0


# ------------------------------------------------------------------------ sparsity x batch sweep
def union_bytes(s, B, uA, uM):
    """Bytes a layer touches with union sets of uA heads and uM neurons at batch B."""
    e = 2 if s.dtype == "f16" else 4
    pred = (2 * s.d * s.r + s.r * s.N + s.r * s.h) * e
    return pred + 4 * s.d * s.dh * uA * e + B * 2 * (s.n + 1) * s.dh * uA * e + 2 * uM * s.d * e + uM * e


def union_weight_elems(s, uA, uM):
    """Weight elements of the products (predictors, Q/K/V, O, MLP) at union sizes uA, uM:
    each carries one multiply-add per batch row, on the matrix cores in their form."""
    pred = 2 * s.d * s.r + s.r * s.N + s.r * s.h
    return pred + 4 * s.d * s.dh * uA + 2 * uM * s.d


MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak, AMD published


def sweep(args) -> int:
    import torch
    from contextual_sparsity_amd import configs, synth
    from contextual_sparsity_amd import dejavu as dj

    base = configs.WORKLOADS["opt175b-1layer-fp16"]
    batches = [int(b) for b in args.sweep_batches.split(",")] if args.sweep_batches else \
        list(configs.SWEEP_BATCH)
    Bmax = max(batches)
    L = args.sweep_layers
    s = base.shape.with_(B=Bmax)
    dev = "cuda"
    t0 = time.time()
    layers = [synth.make_layer(s, args.seed, l, dev) for l in range(L)]
    preds = [synth.make_predictors(s, args.seed, l, dev) for l in range(L)]
    torch.cuda.synchronize()
    log(f"sweep: {L} OPT-175B-shaped layers with caches for {Bmax} sequences "
        f"({time.time() - t0:.1f} s, {torch.cuda.memory_allocated() / 2**30:.1f} GiB)")
    desc = [dj.make_layer(layers[l], preds[l]) for l in range(L)]
    big = dj.make_model(dj.DJV_F16, Bmax, s.d, s.N, s.h, s.dh, s.r, s.n, s.cap, base.scale, dj.DJV_TOPK,
                        s.h, s.N)
    ws = dj.workspace(max(dj.dejavu_workspace_bytes_model(big),
                          dj.dejavu_workspace_bytes_model(dj.make_model(
                              dj.DJV_F16, Bmax, s.d, s.N, s.h, s.dh, s.r, s.n, s.cap, base.scale))), dev)
    stream = torch.cuda.current_stream()
    counts = torch.zeros(L, 2, dtype=torch.int32, device=dev)
    trace = dj.make_trace(counts=counts)
    default_min = dj.dejavu_set_mfma_min_batch(dj.DJV_MAX_VALU_BATCH + 1)

    def run(m, x, x0, dense, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            x.copy_(x0)
            dj.dejavu_stack_decode(m, desc, x, True, dense, None, ws, stream)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(n):
            x.copy_(x0)
            dj.dejavu_stack_decode(m, desc, x, True, dense, None, ws, stream)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n / L

    rows = []
    for B in batches:
        sb = s.with_(B=B)
        x0 = synth.make_input(sb, args.seed, dev)
        x = x0.clone()
        m_dense = dj.make_model(dj.DJV_F16, B, s.d, s.N, s.h, s.dh, s.r, s.n, s.cap, base.scale)
        forms = ["valu", "mfma"] if B <= dj.DJV_MAX_VALU_BATCH else ["mfma"]
        dense_us = {}
        for form in forms:
            dj.dejavu_set_mfma_min_batch(1 if form == "mfma" else dj.DJV_MAX_VALU_BATCH + 1)
            dense_us[form] = run(m_dense, x, x0, True, max(2, args.sweep_steps // 2))
        pcts_A = [int(p) for p in args.sweep_pct_a.split(",")] if args.sweep_pct_a else list(configs.SWEEP_PCT_A)
        pcts_M = [int(p) for p in args.sweep_pct_m.split(",")] if args.sweep_pct_m else list(configs.SWEEP_PCT_M)
        for pA in pcts_A:
            for pM in pcts_M:
                kA, kM = configs.keep(pA, s.h), configs.keep(pM, s.N)
                m = dj.make_model(dj.DJV_F16, B, s.d, s.N, s.h, s.dh, s.r, s.n, s.cap, base.scale,
                                  dj.DJV_TOPK, kA, kM)
                # union sizes of this point (the sets do not depend on the kernel form)
                x.copy_(x0)
                dj.dejavu_stack_decode(m, desc, x, True, False, trace, ws, stream)
                c = counts.cpu().numpy().astype(float)
                uA, uM = float(c[:, 0].mean()), float(c[:, 1].mean())
                nbytes = union_bytes(s, B, uA, uM)
                pt = {"batch": B, "pct_M": pM, "pct_A": pA, "k_M": kM, "k_A": kA,
                      "union_M": round(uM, 1), "union_A": round(uA, 1),
                      "bytes_per_layer": int(nbytes)}
                for form in forms:
                    dj.dejavu_set_mfma_min_batch(1 if form == "mfma" else dj.DJV_MAX_VALU_BATCH + 1)
                    us = run(m, x, x0, False, args.sweep_steps)
                    pt[f"{form}_us"] = round(us, 2)
                    pt[f"{form}_GBps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
                    if form == "mfma":
                        # algorithmic matrix rate of the layer: 2*B flops per weight element
                        tf = 2 * B * union_weight_elems(s, uA, uM) / (us * 1e-6) / 1e12
                        pt["mfma_TFLOPs_alg"] = round(tf, 2)
                        pt["mfma_pct_of_peak_alg"] = round(100 * tf / MFMA_F16_PEAK_TFLOPS, 3)
                    pt[f"{form}_dense_us"] = round(dense_us[form], 2)
                best = min(forms, key=lambda f: pt[f"{f}_us"])
                pt["best"] = best
                pt["speedup_vs_dense"] = round(min(dense_us.values()) / pt[f"{best}_us"], 3)
                rows.append(pt)
                print(json.dumps(pt), flush=True)
    dj.dejavu_set_mfma_min_batch(default_min)
    log(f"sweep done: {len(rows)} points")
    return 0


def lazy_kv(args) -> int:
    """Decode steps at positions n0, n0+1, ... through the stack (a fresh seeded token each
    step), once without and once with lazy K/V: with it, each step saves its attention
    inputs and a selected head first recomputes the K/V of the positions it skipped.
    Reports µs per layer per step for both, and the K/V positions recomputed per step."""
    import torch
    from contextual_sparsity_amd import configs, synth
    from contextual_sparsity_amd import dejavu as dj

    wl = configs.WORKLOADS[args.workload]
    T = args.lazy_steps
    L = args.layers or wl.layers
    s = wl.shape.with_(n_cap=wl.shape.n + T + 1)
    n0, dev = s.n, "cuda"
    t0 = time.time()
    layers, preds = [], []
    for l in range(L):
        layers.append(synth.make_layer(s, args.seed, l, dev))
        preds.append(synth.make_predictors(s, args.seed, l, dev))
    for w in layers:
        w["Y"] = torch.zeros(s.B, s.cap, s.d, dtype=torch.float32, device=dev)
        w["kv_len"] = torch.full((2, s.h), n0, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"lazy K/V: {L} layers, cache capacity {s.cap} ({time.time() - t0:.1f} s, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB)")
    wt = dj.DJV_F16 if s.dtype == "f16" else dj.DJV_F32
    plain = [dj.make_layer({k: v for k, v in layers[l].items() if k not in ("Y", "kv_len")}, preds[l])
             for l in range(L)]
    lazy = [dj.make_layer(layers[l], preds[l]) for l in range(L)]
    tokens = [synth.make_input(s, args.seed + 1000 + t, dev) for t in range(T)]
    models = [dj.make_model(wt, s.B, s.d, s.N, s.h, s.dh, s.r, n0 + t, s.cap, wl.scale, dj.DJV_TOPK,
                            wl.k_A, wl.k_M) for t in range(T)]
    ws = dj.workspace(dj.dejavu_workspace_bytes_model(models[-1]), dev)
    stream = torch.cuda.current_stream()
    x = tokens[0].clone()
    out = {"mode": "lazy K/V decode", "workload": wl.name, "layers": L, "steps": T, "n0": n0}
    for name, desc in (("plain", plain), ("lazy", lazy)):
        for w in layers:
            w["kv_len"].fill_(n0)
        x.copy_(tokens[0])
        dj.dejavu_stack_decode(models[0], desc, x, True, False, None, ws, stream)  # warm-up
        for w in layers:
            w["kv_len"].fill_(n0)
        us, recomputed, heads_back = [], [], []
        for t in range(T):
            # a step at position n reads the lengths in half n % 2 and writes half (n + 1) % 2
            n = n0 + t
            before = torch.stack([w["kv_len"][n % 2] for w in layers]) if name == "lazy" else None
            x.copy_(tokens[t])
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dj.dejavu_stack_decode(models[t], desc, x, True, False, None, ws, stream)
            b.record(stream)
            torch.cuda.synchronize()
            us.append(a.elapsed_time(b) * 1e3 / L)
            if name == "lazy":
                # heads selected at step t: valid length n0+t+1 after it; each recomputed
                # the positions between its previous valid length and n0+t
                after = torch.stack([w["kv_len"][(n + 1) % 2] for w in layers])
                sel = after == n + 1
                recomputed.append(int(((n - before).clamp(min=0) * sel).sum().item()))
                heads_back.append(int((((n - before) > 0) & sel).sum().item()))
        out[f"{name}_us_per_layer"] = round(sum(us) / T, 2)
        out[f"{name}_us_per_layer_first_last"] = [round(us[0], 2), round(us[-1], 2)]
        if name == "lazy":
            out["kv_positions_recomputed_per_step"] = round(sum(recomputed) / T, 1)
            out["kv_positions_recomputed_by_step"] = recomputed
            out["heads_caught_up_per_step"] = round(sum(heads_back) / T, 1)
            # algorithmic bytes of the lazy launches of a step: W^K and W^V rows of every head
            # that catches up, the saved input of every recomputed position and batch row, the
            # recomputed cache rows, and the save of the step's own input (every layer)
            e = 2 if s.dtype == "f16" else 4
            step_bytes = [hb * 2 * s.dh * s.d * e + rc * s.B * (s.d * 4 + 2 * s.dh * e) + L * s.B * s.d * 4
                          for hb, rc in zip(heads_back, recomputed)]
            out["lazy_bytes_per_layer"] = round(sum(step_bytes) / T / L)
    out["lazy_overhead_us_per_layer"] = round(out["lazy_us_per_layer"] - out["plain_us_per_layer"], 2)
    # the lazy launches' bytes over the time they add to the step (their own launch included)
    out["lazy_overhead_GBps"] = round(out["lazy_bytes_per_layer"] / (out["lazy_overhead_us_per_layer"] * 1e-6)
                                      / 1e9, 1) if out["lazy_overhead_us_per_layer"] > 0 else None
    out["lazy_overhead_frac_of_8TBs"] = round(out["lazy_overhead_GBps"] / HBM_PEAK_GBS, 4) \
        if out["lazy_overhead_GBps"] else None
    print(json.dumps(out), flush=True)
    return 0


def recall_probe(args, wl, s, L, layers, m, desc, ws, x0, lookahead, s_main, k_A, k_M) -> int:
    """One traced step, then per layer the true sets from output norms (neuron activations
    on LN(x'), head outputs on LN(x)) and the recall of the predicted sets."""
    import torch
    from contextual_sparsity_amd import dejavu as dj
    import numpy as np
    dev = "cuda"
    f = lambda *shape: torch.zeros(*shape, dtype=torch.float32, device=dev)
    i = lambda *shape: torch.full(shape, -1, dtype=torch.int32, device=dev)
    t = dict(x_in=f(L, s.B, s.d), x_mid=f(L, s.B, s.d), sets_A=i(L, s.h), sets_M=i(L, s.N), counts=i(L, 2))
    x = x0.clone()
    dj.dejavu_stack_decode(m, desc, x, lookahead, False, dj.make_trace(**t), ws, s_main)
    torch.cuda.synchronize()
    wt = dj.DJV_F16 if s.dtype == "f16" else dj.DJV_F32
    pws = dj.workspace(dj.dejavu_workspace_bytes(s.B, s.d, s.N, s.h, s.dh, s.r, s.cap), dev)
    sws = dj.workspace(4 * ((s.N + 31) // 32) + 256, dev)
    y = torch.empty(s.B, s.d, device=dev)
    sc_M, sc_A = torch.empty(s.N, device=dev), torch.empty(s.h, device=dev)
    idx, cnt = torch.empty(s.N, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    rec_A, rec_M, us_M, us_A = [], [], [], []

    def true_set(scores, n, k):
        dj.dejavu_select(1, n, scores.view(1, n), dj.DJV_TOPK, k, 0.5, idx, cnt, sws)
        torch.cuda.synchronize()
        return set(idx[: int(cnt.item())].cpu().tolist())

    counts = t["counts"].cpu()
    for l in range(L):
        w = layers[l]
        dj.dejavu_layernorm(s.B, s.d, t["x_mid"][l], y, 1e-5)
        ev[0].record()
        dj.dejavu_neuron_norms(wt, s.B, s.d, s.N, y, w["W1"], w["b1"], sc_M, pws)
        ev[1].record()
        torch.cuda.synchronize()
        us_M.append(ev[0].elapsed_time(ev[1]) * 1e3)
        tM = true_set(sc_M, s.N, k_M)
        dj.dejavu_layernorm(s.B, s.d, t["x_in"][l], y, 1e-5)
        ev[0].record()
        dj.dejavu_head_norms(wt, s.B, s.d, s.h, s.dh, s.n, s.cap, y, w["Wqkv"], w["K"], w["V"], wl.scale,
                             sc_A, pws)
        ev[1].record()
        torch.cuda.synchronize()
        us_A.append(ev[0].elapsed_time(ev[1]) * 1e3)
        tA = true_set(sc_A, s.h, k_A)
        pA = set(t["sets_A"][l, : int(counts[l, 0])].cpu().tolist())
        pM = set(t["sets_M"][l, : int(counts[l, 1])].cpu().tolist())
        rec_A.append(len(pA & tA) / max(1, len(tA)))
        rec_M.append(len(pM & tM) / max(1, len(tM)))
    e = 2 if s.dtype == "f16" else 4
    bytes_M = s.N * s.d * e
    bytes_A = 3 * s.h * s.dh * s.d * e + s.B * 2 * s.h * (s.n + 1) * s.dh * e
    mean = lambda v: float(np.mean(v))
    out = {"mode": "true-selection recall", "workload": wl.name, "layers": L, "k_A": k_A, "k_M": k_M,
           "recall_heads": round(mean(rec_A), 4), "recall_neurons": round(mean(rec_M), 4),
           "chance_heads": round(k_A / s.h, 4), "chance_neurons": round(k_M / s.N, 4),
           "neuron_norms_us": round(mean(us_M[1:] or us_M), 2),
           "neuron_norms_GBps": round(bytes_M / (mean(us_M[1:] or us_M) * 1e-6) / 1e9, 1),
           "head_norms_us": round(mean(us_A[1:] or us_A), 2),
           "head_norms_GBps": round(bytes_A / (mean(us_A[1:] or us_A) * 1e-6) / 1e9, 1),
           "note": "untrained synthetic weights: recall near chance is the expected outcome"}
    print(json.dumps(out), flush=True)
    return 0


def main(argv=None) -> int:
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        return 2
    if args.deterministic:
        import torch  # noqa: F401  (torch's HIP runtime is loaded before the library's)
        from contextual_sparsity_amd import dejavu as dj
        dj.dejavu_set_deterministic(True)
    if args.sweep:
        return sweep(args)
    if args.lazy_kv:
        return lazy_kv(args)
    if args.ablation:
        return ablation(args)
    import torch
    from contextual_sparsity_amd import configs, synth
    from contextual_sparsity_amd import dejavu as dj

    if args.calibrate_copy:
        # a copy kernel of known size: its FETCH_SIZE / WRITE_SIZE per dispatch calibrate the
        # byte counters (1 GiB read and 1 GiB written per copy)
        src = torch.empty(2**30 // 4, dtype=torch.float32, device="cuda").normal_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": 2**30, "bytes_written": 2**30,
                          "dispatches": 3}), flush=True)
        return 0

    wl = configs.WORKLOADS[args.workload]
    s = wl.shape.with_(B=args.batch) if args.batch else wl.shape
    L = args.layers or wl.layers
    k_A, k_M = wl.k_A, wl.k_M
    dev = "cuda"
    log(f"{dj.dejavu_version()}  device {torch.cuda.get_device_name(0)}  workload {wl.name} L={L}")
    # a tensor-parallel shard: the predictors (and the selection) stay whole, the layer
    # weights and caches are the shard's heads and neurons
    if not (1 <= args.tp <= s.h and 0 <= args.tp_rank < args.tp):
        print(f"--tp {args.tp} --tp-rank {args.tp_rank}: need 1 <= tp <= h and 0 <= rank < tp",
              file=sys.stderr)
        return 2
    shard = None
    s_loc = s
    if args.tp > 1:
        hr = configs.shard_range(s.h, args.tp, args.tp_rank)
        nr = configs.shard_range(s.N, args.tp, args.tp_rank)
        s_loc = s.with_(h=hr[1] - hr[0], N=nr[1] - nr[0])
        shard = (s.h, hr[0], s.N, nr[0])
        log(f"shard {args.tp_rank} of {args.tp}: heads {hr}, neurons {nr}")

    # ---- seeded weights, all resident before timing
    t0 = time.time()
    layers, preds = [], []
    for l in range(L):
        layers.append(synth.make_layer(s_loc, args.seed, l, dev))
        preds.append(synth.make_predictors(s, args.seed, l, dev))
        if l % 4 == 3 or l == L - 1:
            torch.cuda.synchronize()
            log(f"generated layer {l + 1}/{L} ({time.time() - t0:.1f} s, "
                f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB)")
    x0 = synth.make_input(s, args.seed, dev)
    wt = dj.DJV_F16 if s.dtype == "f16" else dj.DJV_F32
    sl = s_loc
    m = dj.make_model(wt, s.B, s.d, sl.N, sl.h, s.dh, s.r, s.n, s.cap, wl.scale, dj.DJV_TOPK, k_A, k_M,
                      shard=shard)
    thr = None
    if args.threshold:
        # t_A, t_M: sigmoid of the score quantiles that keep pct_A / pct_M of layer 0's units
        # (calibrated once on the host from the library's own scores; the step then selects
        # by threshold on the device, so the kept count varies per layer and token)
        import torch.nn.functional as F
        xn = torch.empty_like(x0)
        dj.dejavu_layernorm(s.B, s.d, x0, xn, 1e-5)
        ts = []
        for P1, P2, n_out, pct in ((preds[0]["P1_A"], preds[0]["P2_A"], s.h, wl.pct_A),
                                   (preds[0]["P1_M"], preds[0]["P2_M"], s.N, wl.pct_M)):
            z = torch.empty(s.B, n_out, dtype=torch.float32, device=dev)
            idx = torch.empty(n_out, dtype=torch.int32, device=dev)
            cnt = torch.empty(1, dtype=torch.int32, device=dev)
            pws = dj.workspace(dj.dejavu_workspace_bytes(s.B, s.d, s.N, s.h, s.dh, s.r, s.cap), dev)
            dj.dejavu_predict(wt, s.B, s.d, s.r, n_out, xn, P1, P2, dj.DJV_TOPK, 1, 0.5, idx, cnt, z, pws)
            q = torch.quantile(z.flatten().double().cpu(), 1.0 - pct / 100.0).item()
            ts.append(float(torch.sigmoid(torch.tensor(q)).item()))
        m = dj.make_model(wt, s.B, s.d, sl.N, sl.h, s.dh, s.r, s.n, s.cap, wl.scale, dj.DJV_THRESHOLD, 0,
                          0, t_A=ts[0], t_M=ts[1], shard=shard)
        thr = {"t_A": ts[0], "t_M": ts[1]}
    desc = [dj.make_layer(layers[l], preds[l]) for l in range(L)]
    ws = dj.workspace(dj.dejavu_workspace_bytes_model(m), dev)
    x = x0.clone()
    s_main = torch.cuda.current_stream()
    lookahead = (wl.lookahead or args.lookahead) and not args.no_lookahead

    def step(dense=False):
        x.copy_(x0)
        dj.dejavu_stack_decode(m, desc, x, lookahead, dense, None, ws, s_main)

    # cache flush between timed steps: a stack of distinct layers streams past the caches by
    # itself, one layer run again and again would be partly served from them
    flush = (L == 1) if args.flush is None else args.flush
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if flush else None
    flush_val = [0]

    def do_flush():
        if flush_buf is not None:
            flush_val[0] ^= 0x5A
            flush_buf.fill_(flush_val[0])

    def timed(n, dense=False):
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        if not flush:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(s_main)
            for _ in range(n):
                step(dense)
            b.record(s_main)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n, (time.perf_counter() - w0) * 1e3 / n
        # each step between its own events, after a flush outside them; the wall time holds
        # the flushes too
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            do_flush()
            a.record(s_main)
            step(dense)
            b.record(s_main)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / n, (time.perf_counter() - w0) * 1e3 / n

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warm-up done")
    ms_step, wall_ms = timed(args.steps)
    log(f"sparse step {ms_step:.3f} ms (wall {wall_ms:.3f} ms)")

    # spread of single steps (a separate pass after the timed region): each step between
    # its own pair of events on the main stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        do_flush()
        a.record(s_main)
        step()
        b.record(s_main)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    pick = lambda q: per[min(len(per) - 1, int(round(q * (len(per) - 1))))]
    step_spread = {"median_ms": round(pick(0.5), 4), "p10_ms": round(pick(0.1), 4),
                   "p90_ms": round(pick(0.9), 4), "steps": len(per)}

    def family_time(fam, n_steps):
        cap = n_steps * L + 4
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * cap)]
        dj.dejavu_profile_kernel(fam, evs)
        for _ in range(n_steps):
            do_flush()
            step()
        used = dj.dejavu_profile_count()
        torch.cuda.synchronize()
        dj.dejavu_profile_kernel("off")
        d = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(used)]
        return sum(d) / max(1, len(d)), used

    if args.recall:
        return recall_probe(args, wl, s, L, layers, m, desc, ws, x0, lookahead, s_main, k_A, k_M)

    if thr is not None or shard is not None:
        # kept counts vary by layer: bytes from each layer's own counts
        counts = torch.zeros(L, 2, dtype=torch.int32, device=dev)
        x.copy_(x0)
        dj.dejavu_stack_decode(m, desc, x, lookahead, False, dj.make_trace(counts=counts), ws, s_main)
        c = counts.cpu().double()
        e = 2 if s.dtype == "f16" else 4
        pred_b = (2 * s.d * s.r + s.r * s.N + s.r * s.h) * e  # whole predictors, on every shard
        lbs = [pred_b + 4 * s.d * s.dh * int(c[l, 0]) * e + s.B * 2 * (s.n + 1) * s.dh * int(c[l, 0]) * e
               + (2 * s.d + 1) * int(c[l, 1]) * e for l in range(L)]
        step_bytes_t = sum(lbs)
        out = {"mode": "threshold" if thr else "top-k", "workload": wl.name, "layers": L}
        if thr:
            out.update({"t_A": round(thr["t_A"], 6), "t_M": round(thr["t_M"], 6)})
        if shard:
            out.update({"tp": args.tp, "tp_rank": args.tp_rank, "shard_heads": sl.h, "shard_neurons": sl.N,
                        "predictor_share_of_bytes": round(pred_b * L / step_bytes_t, 3)})
        out.update({"ms_per_step": round(ms_step, 4),
                    "us_per_layer": round(ms_step * 1e3 / L, 2),
                    "GBps": round(step_bytes_t / (ms_step * 1e-3) / 1e9, 1),
                    "pct_of_peak": round(100 * step_bytes_t / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                    "kept_heads": {"mean": round(c[:, 0].mean().item(), 2), "min": int(c[:, 0].min()),
                                   "max": int(c[:, 0].max())},
                    "kept_neurons": {"mean": round(c[:, 1].mean().item(), 1), "min": int(c[:, 1].min()),
                                     "max": int(c[:, 1].max())},
                    "bytes_per_layer_mean": round(step_bytes_t / L)})
        if args.breakdown:
            out["kernels_us"] = {fam: round(family_time(fam, max(3, args.steps // 4))[0] * 1e3, 2)
                                 for fam in ("qkv", "mlp_up", "mlp_down", "o_proj", "attn", "pred_1",
                                             "pred_2", "select")}
        print(json.dumps(out), flush=True)
        return 0
    lb = layer_bytes(s, k_A, k_M)
    unions = None
    if s.B > 1:
        # a batch reads the union of its tokens' sets: bytes from each layer's union sizes
        counts = torch.zeros(L, 2, dtype=torch.int32, device=dev)
        x.copy_(x0)
        dj.dejavu_stack_decode(m, desc, x, lookahead, False, dj.make_trace(counts=counts), ws, s_main)
        c = counts.cpu().tolist()
        per = [layer_bytes(s, cA, cM) for cA, cM in c]
        lb = {key: round(sum(p[key] for p in per) / L) for key in lb}
        unions = {"heads_mean": round(sum(r[0] for r in c) / L, 2),
                  "neurons_mean": round(sum(r[1] for r in c) / L, 1)}
    step_bytes = lb["total"] * L
    gbs = step_bytes / (ms_step * 1e-3) / 1e9

    # ---- dominant kernel: the Q/K/V launch of each layer (kept heads' Q/K/V rows and the
    # next layer's first predictor layers, one GEMV launch; the neuron selection of the
    # layer runs in a side block of it), timed with events around each of its launches
    e = 2 if s.dtype == "f16" else 4
    p1_bytes = 2 * s.r * s.d * e
    # with lookahead the launch also reads the next layer's first predictor layers (the last
    # layer has no next layer); in the serial schedule those run in a launch of their own
    k1_bytes = lb["qkv"] + (p1_bytes * (L - 1) / L if lookahead else 0)


    qkv_ms, qkv_n = family_time("qkv", args.steps)
    qkv_gbs = k1_bytes / (qkv_ms * 1e-3) / 1e9
    log(f"Q/K/V+P1 launch {qkv_ms * 1e3:.1f} us/launch over {qkv_n} launches -> {qkv_gbs:.0f} GB/s")
    kernels = {}
    if args.breakdown:
        # the MLP launches read the kept (at B > 1: the union's) W1 and W2 rows
        mlp_half = lb["mlp"] * s.d / (2 * s.d + 1)
        fam_bytes = {"qkv": k1_bytes, "mlp_up": mlp_half, "mlp_down": mlp_half,
                     "o_proj": lb["o_proj"], "attn": lb["kv"], "pred_1": p1_bytes,
                     "pred_2": (s.N + s.h) * s.r * e, "select": None}
        for fam in ("qkv", "mlp_up", "mlp_down", "o_proj", "attn", "pred_1", "pred_2", "select"):
            ms_f, n_f = family_time(fam, max(3, args.steps // 4))
            ent = {"us": round(ms_f * 1e3, 2), "launches": n_f}
            if fam_bytes.get(fam):
                ent["GBps"] = round(fam_bytes[fam] / (ms_f * 1e-3) / 1e9, 1)
            kernels[fam] = ent
            log(f"  {fam:9s} {ms_f * 1e3:8.1f} us  {ent.get('GBps', '')}")

    # ---- dense path on the same stack
    dense = None
    if not args.no_dense:
        step(dense=True)
        torch.cuda.synchronize()
        ms_dense, _ = timed(args.dense_steps, dense=True)
        db = dense_layer_bytes(s) * L
        dense = {"ms_per_step": round(ms_dense, 3), "us_per_layer": round(ms_dense * 1e3 / L, 2),
                 "GBps": round(db / (ms_dense * 1e-3) / 1e9, 1),
                 "pct_of_peak": round(100 * db / (ms_dense * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                 "bytes_per_layer": dense_layer_bytes(s)}
        log(f"dense step {ms_dense:.3f} ms")

    # achievable HBM rate on this device: a plain device copy of 2 GiB (read + write bytes)
    src = torch.empty(2**29, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record()
    for _ in range(5):
        dst.copy_(src)
    eb.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 5 / (ea.elapsed_time(eb) * 1e-3) / 1e9
    # plain read rate: the library's streaming-read kernel over the same 2 GiB
    probe_out = torch.zeros(1, dtype=torch.int32, device=dev)
    dj.dejavu_read_probe(src, probe_out, stream=s_main)
    torch.cuda.synchronize()
    ea.record(s_main)
    for _ in range(5):
        dj.dejavu_read_probe(src, probe_out, stream=s_main)
    eb.record(s_main)
    torch.cuda.synchronize()
    read_gbs = src.numel() * 4 * 5 / (ea.elapsed_time(eb) * 1e-3) / 1e9
    del src, dst
    log(f"device copy reference {copy_gbs:.0f} GB/s (read + write), plain read {read_gbs:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle sample ...")
        cpu = cpu_baseline(wl, s, layers, preds, x0, k_A, k_M, args.cpu_seconds, lb["total"],
                           dense_layer_bytes(s), lookahead)
        log(f"CPU oracle {cpu['us_per_layer']} us/layer on {cpu['cores']} threads "
            f"({cpu['one_core_us_per_layer']} on one core; dense {cpu['dense_us_per_layer']} on one core)")

    headline = wl.name == "opt175b-24layers-fp16" and s.B == 1 and L == wl.layers
    metric = HEADLINE_METRIC if headline else (
        f"sparse decode-layer µs and HBM GB/s (% of peak), {wl.name}{f', batch {s.B}' if s.B > 1 else ''}"
        f"{f', {L} layers' if L != wl.layers else ''}, {wl.pct_M}% MLP/{wl.pct_A}% heads")
    out = {
        "metric": metric,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if s.dtype == "f16" else "f32",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,0.05) predictors, N(0,1) input)",
        "config": {"workload": wl.name, "layers": L, "d": s.d, "N": s.N, "h": s.h, "dh": s.dh,
                   "n": s.n, "r": s.r, "batch": s.B, "keep_neurons_pct": wl.pct_M,
                   "keep_heads_pct": wl.pct_A, "k_M": k_M, "k_A": k_A, "lookahead": lookahead,
                   "deterministic": args.deterministic, "union_sets": unions, "cache_flush": flush},
        "us_per_layer": round(ms_step * 1e3 / L, 2),
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "copy_ref_GBps": round(copy_gbs, 1),
        "pct_of_copy_ref": round(100 * gbs / copy_gbs, 2),
        "read_ref_GBps": round(read_gbs, 1),
        "pct_of_read_ref": round(100 * gbs / read_gbs, 2),
        "tokens_per_s": round(1e3 / ms_step, 1),
        "bytes_per_layer": lb,
        "wall_ms_per_step": round(wall_ms, 4),
        "step_spread": step_spread,
        "device": device_facts(torch),
        "dense": dense,
        "speedup_vs_dense": round(dense["ms_per_step"] / ms_step, 3) if dense else None,
        "roofline": {"kernel": ("Q/K/V of the kept heads + next layer's predictor first layers "
                                "(gemv_kernel, one launch per layer)") if lookahead and L > 1 else
                               "Q/K/V of the kept heads (gemv_kernel, one launch per layer)", "bound": "hbm",
                     "achieved": round(qkv_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(qkv_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic() if headline else None,
                     "bytes_per_launch": round(k1_bytes), "us_per_launch": round(qkv_ms * 1e3, 2),
                     "launches": qkv_n},
        "kernels": kernels or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
