#!/usr/bin/env python3
"""Throughput of the orthonormalized optimizer step on one MI355X.

One bench step on the 4096 x 4096 bf16 workload (fp32 momentum, gradient with a
planted rank-32 part of 10x norm) is the whole hot path once:
    dion_step at r = 1024 (rank fraction 1/4)
    dion_step at r = 256  (rank fraction 1/16)
    newton_schulz, 5 iterations, on the same matrix.
The three are independent and run on three streams; the same steps on one
stream are reported beside the headline.
Inputs are synthetic, seeded and resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sizes] [--workload 1|2|3|4]

Prints ONE JSON line.  Besides the headline step it carries a per-size table
(time per call, modeled GB/s and TFLOP/s and their fraction of peak) for square
matrices from 1024 to 8192 at rank fractions 1/4 and 1/16 and for the
Llama-405B weight shapes, with the whole Muon step (momentum, NS x5, update)
and the Dion2 step (rows of largest norm, fractions 1/4 and 1/16) beside NS, and the time per step of the other named workloads (256 x 256 fp32,
the 12-layer GPT parameter groups, per-head NS), measured after the timed region.  The oracle is timed on the host cores on a bounded
sample (one step of the same workload) as the reported CPU baseline.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "optimizer steps/sec & ms/step vs matrix size, rank frac 1/4,1/16; % HBM/MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
# HBM bytes per launch of the product kernel (mean over the Gram, polynomial
# and apply launches on 4096 x 4096), from rocprofv3 FETCH_SIZE and WRITE_SIZE
# passes over `bench.py --counter-sample`, each scaled by the same counter's
# reading for a 256 MiB elementwise copy (fetch factor 2.0, write factor 1.0).
# Set to None whenever the kernel changes, until the passes are taken again.
TRAFFIC_BYTES_PER_LAUNCH = 2.412e8


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--one-stream", action="store_true",
                   help="time the step with its paths one after another on one stream (kernel "
                        "profiles: every launch then runs alone)")
    p.add_argument("--no-sizes", action="store_true",
                   help="skip the per-size table (square 1024-8192 and the Llama-405B shapes) "
                        "and the other workloads (256x256 fp32, GPT-12 groups, per-head NS)")
    p.add_argument("--counter-sample", action="store_true",
                   help="run 2 Newton-Schulz iterations, one Dion step at each rank and a "
                        "256 MiB device copy, print nothing else (for rocprofv3 --pmc passes)")
    return p.parse_args()


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.s.record(self.torch.cuda.current_stream())
        return self

    def __exit__(self, *a):
        self.e.record(self.torch.cuda.current_stream())
        self.e.synchronize()
        self.ms = self.s.elapsed_time(self.e)


def workload2(torch, api, synth):
    """State and closures for the 4096 x 4096 workload."""
    wl = synth.WORKLOADS[2]
    m = n = 4096
    dev = "cuda"
    S = synth.planted(2, m, n, 32, wl["planted_ratio"])
    Gs = [torch.from_numpy(synth.gradient(2, m, n, t, "bf16", planted_part=S)).to(dev).to(torch.bfloat16)
          for t in (1, 2, 3)]
    X0 = torch.from_numpy(synth.weight(2, m, n, "bf16")).to(dev).to(torch.bfloat16)
    paths = {}
    for r in wl["ranks"]:
        st = dict(X=X0.clone(), M=torch.zeros(m, n, device=dev),
                  Q=torch.from_numpy(synth.right_factor0(2, n, r)).to(dev),
                  ws=api.workspace(api.dion_workspace_size(m, n, r), dev))
        paths[f"dion_r{r}"] = st
    ns_ws = api.workspace(api.ns_workspace_size(m, n), dev)
    ns_out = torch.empty(m, n, device=dev, dtype=torch.bfloat16)
    mu, lr = wl["mu"], wl["lr"]

    def run_path(name, i):
        G = Gs[i % len(Gs)]
        if name == "ns5":
            api.newton_schulz(G, out=ns_out, steps=5, ws=ns_ws)
        else:
            st = paths[name]
            api.dion_step(st["X"], G, st["M"], st["Q"], mu, lr, ws=st["ws"])

    names = [f"dion_r{r}" for r in wl["ranks"]] + ["ns5"]

    def ns_steps(k):
        api.newton_schulz(Gs[0], out=ns_out, steps=k, ws=ns_ws)

    info = dict(workload=wl["name"], m=m, n=n, ranks=wl["ranks"], ns_iterations=5,
                mu=mu, lr=lr, x_dtype="bf16", momentum_dtype="f32")
    return names, run_path, ns_steps, info, (m, n)


# Per-size table, outside the timed region: time per call of each path on
# square matrices and on the Llama-405B weight shapes.  Inputs are drawn on the
# device from a seeded generator (X ~ N(0, 0.02^2), G ~ N(0, 1), Q0 Gaussian with
# unit columns), bf16 weights and gradients, fp32 momentum.
SIZE_CASES = [
    # (name, m, n, ranks, ns, timed calls)
    ("square-1024", 1024, 1024, (256, 64), True, 10),
    ("square-2048", 2048, 2048, (512, 128), True, 10),
    ("square-4096", 4096, 4096, (1024, 256), True, 10),
    ("square-8192", 8192, 8192, (2048, 512), True, 5),
    ("llama405b-16384x16384", 16384, 16384, (4096, 1024), True, 2),
    ("llama405b-16384x53248", 16384, 53248, (4096, 1024), False, 2),
]


def dion_model(m, n, r):
    """Algorithmic bytes (bf16 X and G, fp32 M, fp32 factors) and flops of one
    Dion step: three sweeps of M + G, the weight read and written once; four
    rank-r products (8 m n r), the Householder-count QR of the m x r power
    iterate (2 m r^2) and the column norms (3 n r)."""
    return 26.0 * m * n + 16.0 * (m + n) * r, 8.0 * m * n * r + 2.0 * m * r * r + 3.0 * n * r


def ns_model(m, n, iters=5):
    a, b = min(m, n), max(m, n)
    return (3.0 * 2 * a * b + 12.0 * a * a) * iters, (4.0 * a * a * b + 2.0 * a ** 3) * iters


def size_table(torch, api, warmup=1):
    dev = "cuda"
    out = {}
    for ci, (name, m, n, ranks, ns, calls) in enumerate(SIZE_CASES):
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 + ci)
        X = (torch.randn(m, n, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        G = torch.randn(m, n, generator=gen, device=dev).to(torch.bfloat16)
        row = {}

        def timed(fn):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            with Timer(torch) as t:
                for _ in range(calls):
                    fn()
            return t.ms / calls

        for r in ranks:
            M = torch.zeros(m, n, device=dev)
            Q = torch.randn(n, r, generator=gen, device=dev)
            Q /= Q.norm(dim=0, keepdim=True)
            ws = api.workspace(api.dion_workspace_size(m, n, r), dev)
            ms = timed(lambda: api.dion_step(X, G, M, Q, 0.95, 0.01, ws=ws))
            nbytes, flops = dion_model(m, n, r)
            gbs, tfs = nbytes / (ms * 1e-3) / 1e9, flops / (ms * 1e-3) / 1e12
            row[f"dion_r{r}"] = {"ms": ms, "steps_per_s": 1000.0 / ms, "rank_frac": f"1/{min(m, n) // r}",
                                 "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
                                 "TFLOP/s": tfs, "mfma_frac": tfs / PEAK_BF16_TFLOPS}
            del M, Q, ws
        if ns:
            ws = api.workspace(api.ns_workspace_size(m, n), dev)
            o = torch.empty_like(G)
            ms = timed(lambda: api.newton_schulz(G, out=o, steps=5, ws=ws))
            nbytes, flops = ns_model(m, n)
            tfs = flops / (ms * 1e-3) / 1e12
            row["ns5"] = {"ms": ms, "steps_per_s": 1000.0 / ms, "TFLOP/s": tfs,
                          "mfma_frac": tfs / PEAK_BF16_TFLOPS}
            del ws, o
            # the whole Muon step: momentum buffer, NS x5 of it, weight update
            M = torch.zeros(m, n, device=dev)
            ws = api.workspace(api.muon_workspace_size(m, n), dev)
            ms = timed(lambda: api.muon_step(X, G, M, 0.95, 0.02, ws=ws))
            tfs = flops / (ms * 1e-3) / 1e12
            row["muon5"] = {"ms": ms, "steps_per_s": 1000.0 / ms, "TFLOP/s": tfs,
                            "mfma_frac": tfs / PEAK_BF16_TFLOPS}
            del M, ws
            # NorMuon: the Muon step with the orthogonalised rows normalised
            M = torch.zeros(m, n, device=dev)
            ws = api.workspace(api.normuon_workspace_size(m, n), dev)
            ms = timed(lambda: api.normuon_step(X, G, M, 0.95, 0.02, ws=ws))
            tfs = flops / (ms * 1e-3) / 1e12
            row["normuon5"] = {"ms": ms, "steps_per_s": 1000.0 / ms, "TFLOP/s": tfs,
                               "mfma_frac": tfs / PEAK_BF16_TFLOPS}
            del M, ws
        if m <= 65535:
            # Dion2: the rows of largest norm (fractions 1/4 and 1/16 of the
            # rows), Newton-Schulz x5 of that block, error feedback
            for frac in (4, 16):
                k = m // frac
                M = torch.zeros(m, n, device=dev)
                ws = api.workspace(api.dion2_workspace_size(m, n, k), dev)
                ms = timed(lambda: api.dion2_step(X, G, M, k, 0.95, 0.01, ws=ws))
                _, fl = ns_model(k, n)
                tfs = fl / (ms * 1e-3) / 1e12
                row[f"dion2_k{k}"] = {"ms": ms, "steps_per_s": 1000.0 / ms, "row_frac": f"1/{frac}",
                                      "TFLOP/s": tfs, "mfma_frac": tfs / PEAK_BF16_TFLOPS}
                del M, ws
        out[name] = row
        del X, G
        torch.cuda.empty_cache()
    return out


def workload_table(torch, api, synth, calls=10, only=None):
    """Time per step of the other named workloads (all of them, or workload
    ``only``): the 256 x 256 fp32 weight (Dion r = 64), the 12-layer d = 2048
    GPT parameter set (three shape-grouped Dion calls at r = 1/4 of the small
    side) and the per-head split of a 4096 x 4096 projection (32 row blocks of
    128 x 4096, batched Newton-Schulz x5).  Inputs are drawn on the device from
    a seeded generator with the workloads' distributions."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(2000)
    out = {}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        with Timer(torch) as t:
            for _ in range(calls):
                fn()
        return t.ms / calls

    def unit_cols(n, r):
        q = torch.randn(n, r, generator=gen, device=dev)
        return q / q.norm(dim=0, keepdim=True)

    if only in (None, 1):  # single 256 x 256 fp32 weight, r = 64
        wl = synth.WORKLOADS[1]
        X = torch.randn(256, 256, generator=gen, device=dev) * 0.02
        G = torch.randn(256, 256, generator=gen, device=dev)
        M = torch.zeros(256, 256, device=dev)
        Q = unit_cols(256, 64)
        ws = api.workspace(api.dion_workspace_size(256, 256, 64), dev)
        ms = timed(lambda: api.dion_step(X, G, M, Q, wl["mu"], wl["lr"], ws=ws))
        # the same call captured once into a HIP graph and replayed: the step
        # is a chain of small launches, and replay removes their host-side cost
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            api.dion_step(X, G, M, Q, wl["mu"], wl["lr"], ws=ws)
        ms_graph = timed(graph.replay)
        del graph
        out[wl["name"]] = {"dion_r64_ms": ms, "steps_per_s": 1000.0 / ms,
                           "dion_r64_graph_replay_ms": ms_graph}

    if only in (None, 3):  # 12-layer d = 2048 GPT parameter set, one call per shape group
        wl = synth.WORKLOADS[3]
        groups = []
        nbytes = flops = 0.0
        for count, m, n in wl["groups"]:
            r = min(m, n) // 4
            Xs = [(torch.randn(m, n, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
                  for _ in range(count)]
            Gs = [torch.randn(m, n, generator=gen, device=dev).to(torch.bfloat16) for _ in range(count)]
            Ms = [torch.zeros(m, n, device=dev) for _ in range(count)]
            Qs = [unit_cols(n, r) for _ in range(count)]
            ws = api.workspace(api.dion_workspace_size(m, n, r, count), dev)
            groups.append((Xs, Gs, Ms, Qs, ws))
            b, f = dion_model(m, n, r)
            nbytes += count * b
            flops += count * f

        def gpt_step():
            for Xs, Gs, Ms, Qs, ws in groups:
                api.dion_step_batched(Xs, Gs, Ms, Qs, wl["mu"], wl["lr"], ws=ws)
        ms = timed(gpt_step)
        # The same step with each shape group's calls on streams of their own
        # (separate workspaces, no shared state): one call's latency-bound
        # phases (the Cholesky chains, the small launches) run beside another
        # call's products.
        main = torch.cuda.current_stream()
        # a group of more than 32 matrices splits into calls of at most 32 (the
        # library's launch chunk), each on its own stream, with its own workspace
        chunks = []
        for Xs, Gs, Ms, Qs, ws in groups:
            if len(Xs) <= 32:
                chunks.append((Xs, Gs, Ms, Qs, ws))
                continue
            m, n, r = Xs[0].size(0), Xs[0].size(1), Qs[0].size(1)
            for c0 in range(0, len(Xs), 32):
                sl = slice(c0, c0 + 32)
                chunks.append((Xs[sl], Gs[sl], Ms[sl], Qs[sl],
                              api.workspace(api.dion_workspace_size(m, n, r, len(Xs[sl])), dev)))
        side = [torch.cuda.Stream() for _ in chunks]

        def gpt_step_streams():
            fork = torch.cuda.Event()
            fork.record(main)
            done = []
            for st, (Xs, Gs, Ms, Qs, ws) in zip(side, chunks):
                st.wait_event(fork)
                with torch.cuda.stream(st):
                    api.dion_step_batched(Xs, Gs, Ms, Qs, wl["mu"], wl["lr"], ws=ws)
                ev = torch.cuda.Event()
                ev.record(st)
                done.append(ev)
            for ev in done:
                main.wait_event(ev)
        ms_streams = timed(gpt_step_streams)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[wl["name"]] = {"dion_r_quarter_ms": ms, "steps_per_s": 1000.0 / ms, "matrices": 72,
                           "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
                           "TFLOP/s": flops / (ms * 1e-3) / 1e12,
                           "dion_r_quarter_group_streams_ms": ms_streams,
                           "group_streams": len(chunks)}
        del groups
        torch.cuda.empty_cache()

    if only in (None, 4):  # per-head: 32 row blocks of 128 x 4096 of one 4096 x 4096 projection
        wl = synth.WORKLOADS[4]
        G = torch.randn(4096, 4096, generator=gen, device=dev).to(torch.bfloat16)
        O = torch.empty_like(G)
        heads = [G[128 * h:128 * (h + 1)] for h in range(32)]
        outs = [O[128 * h:128 * (h + 1)] for h in range(32)]
        ws = api.workspace(api.ns_workspace_size(128, 4096, 32), dev)
        ms = timed(lambda: api.newton_schulz_batched(heads, outs, steps=5, ws=ws))
        nb, _ = ns_model(128, 4096)
        gbs = 32 * nb / (ms * 1e-3) / 1e9
        out[wl["name"]] = {"ns5_per_head_ms": ms, "steps_per_s": 1000.0 / ms, "heads": 32,
                           "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}
    return out


def host_info():
    """Cores available to this process, the CPU model and numpy's BLAS."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f'{i.get("internal_api")} {i.get("version")}'
                threads = int(i.get("num_threads", 1))
                break
    except Exception:  # pragma: no cover
        pass
    return cores, model, blas, threads


def cpu_baseline(synth, oracle):
    """One oracle step of the same workload on the host (bounded sample)."""
    cores, model, blas, threads = host_info()
    wl = synth.WORKLOADS[2]
    m = n = 4096
    S = synth.planted(2, m, n, 32, wl["planted_ratio"])
    G = synth.gradient(2, m, n, 1, "bf16", planted_part=S)
    X = synth.weight(2, m, n, "bf16")
    t0 = time.perf_counter()
    for r in wl["ranks"]:
        oracle.dion_step(X, G, np.zeros((m, n)), synth.right_factor0(2, n, r), wl["mu"], wl["lr"])
    oracle.newton_schulz(G, 5)
    dt = time.perf_counter() - t0
    return {"value": 1.0 / dt, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": "one full step (Dion r=1024, Dion r=256, Newton-Schulz x5) of the "
                      "4096x4096 workload, fp64 numpy, first step's inputs",
            "seconds": dt, "cpu_model": model, "blas": blas, "blas_threads": threads}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); multi-GPU sharding "
              "is not implemented.", file=sys.stderr)
        sys.exit(2)
    if args.workload not in (1, 2, 3, 4):
        print("--workload 1, 2 (the bench line), 3 or 4; the Llama-405B shapes are in the per-size "
              "table of the default run", file=sys.stderr)
        sys.exit(2)
    import torch
    from orthonormal_optimizer_update_amd import api, synth
    api.lib()
    torch.cuda.set_device(0)
    if args.workload != 2:
        # one named workload alone, after one warm-up (for kernel profiles of it)
        table = workload_table(torch, api, synth, calls=args.steps, only=args.workload)
        name, row = next(iter(table.items()))
        print(json.dumps({"workload": name, **row}))
        return
    names, run_path, ns_steps, info, (m, n) = workload2(torch, api, synth)

    if args.counter_sample:
        # The product kernel's HBM traffic per launch, and a plain copy of
        # known size (256 MiB read + 256 MiB written) that calibrates the
        # FETCH_SIZE / WRITE_SIZE counters.
        ns_steps(2)
        for nm in names:  # one Dion step at each rank (the streaming and 256 x 256 updates)
            if nm.startswith("dion"):
                run_path(nm, 0)
        src = torch.ones(64 * 1024 * 1024, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)  # elementwise copy kernel: 256 MiB in, 256 MiB out
        torch.cuda.synchronize()
        print("counter sample done", flush=True)
        return

    # The paths of a step are independent (each has its own weight, momentum,
    # right factor and workspace; the gradient is only read), so each runs on
    # its own stream (default priority), forked from the main stream and joined
    # back to it every step: the idle CUs of one path's narrow launches (the
    # Cholesky chain, the small orthonormalisation products) take the other
    # paths' work.
    main = torch.cuda.current_stream()
    side = {nm: torch.cuda.Stream() for nm in names}

    def step(i):
        if args.one_stream:
            for nm in names:
                run_path(nm, i)
            return
        fork = torch.cuda.Event()
        fork.record(main)
        done = []
        for nm in names:
            side[nm].wait_event(fork)
            with torch.cuda.stream(side[nm]):
                run_path(nm, i)
            ev = torch.cuda.Event()
            ev.record(side[nm])
            done.append(ev)
        for ev in done:
            main.wait_event(ev)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly K whole steps.  An event on the main stream after
    # each step (every path has joined it by then) splits the region into
    # per-step times for the median and the 10th/90th percentiles.
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with Timer(torch) as t:
        bounds[0].record(main)
        for i in range(args.steps):
            step(i)
            bounds[i + 1].record(main)
    torch.cuda.synchronize()
    ms_step = t.ms / args.steps
    per_step = sorted(bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps))

    def pct(q):
        return per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]

    # The same steps with the paths one after another on one stream.
    with Timer(torch) as ts:
        for i in range(args.steps):
            for nm in names:
                run_path(nm, i)
    ms_serial = ts.ms / args.steps

    # Each optimizer step on its own (one stream, back to back): its own
    # steps/s, and the step's algorithmic bytes and flops over its time as
    # fractions of the HBM and bf16 matrix-core peaks.
    per_path = {}
    for nm in names:
        with Timer(torch) as tp:
            for i in range(args.steps):
                run_path(nm, i)
        ms_p = tp.ms / args.steps
        if nm == "ns5":
            nbytes, fl = ns_model(m, n)
            what = "Newton-Schulz x5 (bf16 products, fp32 iterate)"
        else:
            r = int(nm.split("_r")[1])
            nbytes, fl = dion_model(m, n, r)
            what = f"Dion step, r = {r} (rank fraction 1/{min(m, n) // r})"
        gbs, tfs = nbytes / (ms_p * 1e-3) / 1e9, fl / (ms_p * 1e-3) / 1e12
        per_path[nm] = {"optimizer": what, "ms": ms_p, "steps_per_s": 1000.0 / ms_p,
                        "GB/s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
                        "TFLOP/s": tfs, "mfma_frac": tfs / PEAK_BF16_TFLOPS,
                        "model_bytes": nbytes, "model_flops": fl}

    # Dominant kernel: the Newton-Schulz MFMA products (three launches per
    # iteration).  Work per iteration is counted densely, 4 m m n + 2 m^3 (Gram,
    # polynomial, apply).  The Gram and the polynomial are symmetric and their
    # kernel computes only the blocks on and above the diagonal, so the
    # products executed are reported beside the dense rate.  The average
    # launch time is
    # (time of 6 iterations - time of 1 iteration) / 15, on the same stream:
    # both runs launch the same normalisation kernels, and both keep the GPU
    # busy for far longer than the host needs to issue a call, so the
    # difference holds only the 15 product launches.
    reps = max(3, args.steps // 2)
    ns_steps(1)
    ns_steps(6)
    torch.cuda.synchronize()
    with Timer(torch) as t6:
        for _ in range(reps):
            ns_steps(6)
    with Timer(torch) as t1:
        for _ in range(reps):
            ns_steps(1)
    gemm_ms = (t6.ms - t1.ms) / reps / 15.0
    flops = (4.0 * m * m * n + 2.0 * m ** 3) / 3.0  # dense count, mean per launch
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    # products computed by the Gram and the polynomial (gemm_bf16_sym): the
    # T (T - 1) upper 256 x 128 half tiles whole, and 36 of the 64 32 x 32
    # blocks of each of the T diagonal tiles, out of T^2 tiles
    tiles = m // 256
    sym_frac = (tiles * (tiles - 1) * 0.5 + tiles * 36.0 / 64.0) / float(tiles * tiles)
    executed = (2.0 * m * m * n * sym_frac + 2.0 * m ** 3 * sym_frac + 2.0 * m * m * n) / 3.0
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": TRAFFIC_BYTES_PER_LAUNCH,
                "kernel": "Newton-Schulz products: X X^T and b A + c A^2 on gemm_bf16_sym (the upper "
                          "256x256 tiles as 256x128 halves and the diagonal tiles' upper 32x32 "
                          "blocks, one workgroup per CU), a X + Bp X on gemm_bf16_256; bf16 MFMA "
                          "32x32x16, direct-to-LDS operand copies",
                "avg_launch_ms": gemm_ms, "flops_per_launch": flops,
                "executed_flops_per_launch": executed,
                "executed_tflops": executed / (gemm_ms * 1e-3) / 1e12}

    sizes = None if args.no_sizes else size_table(torch, api)
    workloads = None if args.no_sizes else workload_table(torch, api, synth)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import dion_ref as oracle  # reported CPU baseline only
        cpu = cpu_baseline(synth, oracle)

    line = {
        "metric": METRIC, "value": 1000.0 / ms_step, "unit": "steps/s",
        "value_is": ("bench steps/s; one bench step = Dion r=1024 + Dion r=256 + Newton-Schulz x5 "
                     "on the 4096x4096 matrix (three optimizer steps, one per stream); each "
                     "optimizer's own rate is in 'optimizers'"),
        "optimizers": per_path, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "ms_per_step_median": pct(0.5), "ms_per_step_p10": pct(0.1), "ms_per_step_p90": pct(0.9),
        "streams": 1 if args.one_stream else len(names),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": info, "ms_per_step_one_stream": ms_serial,
        "roofline": roofline,
        "cpu_baseline": cpu, "sizes": sizes, "workloads": workloads,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
