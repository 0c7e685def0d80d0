#!/usr/bin/env python3
"""DP-SGD-RC step throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is the whole hot path over one batch: per-sample norm estimation of
every linear layer (summed over layers), clip factors, the clipped-sum
contraction and the fused noise + SGD update of every layer.  Inputs are
synthetic, generated on the device before timing and already resident in
HBM; several input copies are rotated so that the 256 MB last-level cache
cannot serve one step's inputs from the previous step.

Prints ONE JSON line: tokens/s of the timed steps, the roofline of the
dominant kernel (duration from HIP events recorded by the library around
that kernel, inside the timed steps), and the CPU oracle timed on a bounded
sample of the same workload on this host.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DP-SGD-RC step tokens/sec (norm-est+clip+noisy agg); % HBM / MFMA peak"
EV_STRIDE = 10  # timed steps between two that bracket the dominant kernel with events


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama1b_stack_b8_t4096")
    ap.add_argument("--method", default=None, help="override the workload's estimator")
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-step", action="store_true",
                    help="time the steps only: no side measurements and no CPU baseline (for "
                         "profiler passes whose per-kernel means must cover the step alone)")
    ap.add_argument("--rademacher", action="store_true",
                    help="sign (+-1) probes instead of Gaussian ones for Hutch / Hutch++")
    ap.add_argument("--unfused", action="store_true",
                    help="aggregate and update with two calls per layer (S materialised)")
    ap.add_argument("--per-layer", action="store_true",
                    help="one norm call and one update call per layer instead of the batched "
                         "calls over all layers")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


KERNEL_SOURCES = {"aggregate": "sample_gradient_clipping_amd/csrc/mfma_gemm.hip",
                  "norm_est": "sample_gradient_clipping_amd/csrc/mfma_hutch.hip",
                  "noise_update": "sample_gradient_clipping_amd/csrc/rng_kernels.hip"}


def source_hash(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on this workload with the kernel source as it is now; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k_, v = line.split("=", 1)
            kv[k_.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_inputs(wl, copies, dev):
    import torch
    from sample_gradient_clipping_amd.inputs import linear_inputs, linear_inputs_device
    out = []
    for c in range(copies):
        layers = []
        for l in wl.layers:
            seed = wl.data_seed + 7919 * c
            if wl.tokens * (l.d + l.p) <= (1 << 22):
                A, G = linear_inputs(wl.B, wl.T, l.d, l.p, wl.dtype, wl.recipe, seed, l.layer_id)
                A, G = A.to(dev), G.to(dev)
            else:
                A, G = linear_inputs_device(wl.B, wl.T, l.d, l.p, wl.dtype, wl.recipe, seed,
                                            l.layer_id, dev)
            layers.append((A, G))
        out.append(layers)
    torch.cuda.synchronize()
    return out


def _cpu_threads():
    """Host threads this process may use: its CPU affinity, capped by OMP_NUM_THREADS."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(cap))) if cap.isdigit() and int(cap) > 0 else max(1, n)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, method, target_s=15.0, rademacher=False):
    """The CPU oracle on a bounded sample of the workload: the plain C++ fp64
    oracle (std::thread, no BLAS) for Hutch with Gaussian probes, else the numpy
    fp64 oracle.  One sampled step = Bs samples of the first block's linear
    layers (all of them for a single layer) through norms, clip factors,
    clipped sums, noise and update; a layer stack's time is scaled to all of
    its blocks."""
    import numpy as np
    from sample_gradient_clipping_amd.inputs import linear_inputs
    layers = wl.layers
    scale_blocks = 1
    if len(layers) > 7:  # a layer stack: time block 0, extrapolate to all blocks
        scale_blocks = len(layers) // 7
        layers = layers[:7]
    use_cpp = method == "hutch" and not rademacher
    threads = _cpu_threads()
    if use_cpp:
        from oracle import cpp_oracle as co
        co.load()
        kind = "oracle (plain C++17 fp64, std::thread, no BLAS)"
    else:
        import oracle
        kind = "oracle (numpy fp64)"

    def run(Bs):
        data = []
        for l in layers:
            A, G = linear_inputs(Bs, wl.T, l.d, l.p, wl.dtype, wl.recipe, wl.data_seed, l.layer_id)
            data.append((l, A, G))
        t = {"norms": 0.0, "clip": 0.0, "aggregate": 0.0, "noise_update": 0.0}
        if not use_cpp:
            t0 = time.perf_counter()
            oracle.dp_step([(l.layer_id, A, G, np.zeros((l.p, l.d))) for l, A, G in data], method,
                           wl.k, wl.C, wl.sigma, wl.eta, wl.method_seed, wl.noise_seed,
                           rademacher=rademacher)
            return time.perf_counter() - t0, None
        n = None
        t0 = time.perf_counter()
        for l, A, G in data:
            n = co.hutch_norms(A, G, wl.k, wl.method_seed, l.layer_id, n=n, threads=threads)
        t1 = time.perf_counter()
        c, _ = co.clip_factors(n, wl.C)
        t2 = time.perf_counter()
        t["norms"], t["clip"] = t1 - t0, t2 - t1
        for l, A, G in data:
            t3 = time.perf_counter()
            S = co.aggregate(A, G, c, threads=threads)
            t4 = time.perf_counter()
            co.noise_update(np.zeros((l.p, l.d)), S, wl.sigma, wl.C, wl.eta, Bs, wl.noise_seed,
                            l.layer_id, threads=threads)
            t["aggregate"] += t4 - t3
            t["noise_update"] += time.perf_counter() - t4
        return sum(t.values()), t

    # one sample first, then as many samples as fill about `target_s`
    Bs = 1
    t, stages = run(1)
    if t < target_s and wl.B > 1:
        Bs = int(min(wl.B, max(2, target_s // max(t, 1e-3))))
        t, stages = run(Bs)
    t_step = t * scale_blocks
    sample = (f"{Bs} of {wl.B} samples x {wl.T} tokens, {len(layers)} of {len(wl.layers)} linear "
              f"layers, one step (norms, clip, clipped sums, noise + update) in {t:.2f} s"
              + (f"; time x{scale_blocks} (extrapolated to all blocks)" if scale_blocks > 1 else ""))
    out = {"value": Bs * wl.T / t_step, "unit": "tokens/s", "cores": threads if use_cpp else None,
           "kind": "oracle", "implementation": kind, "sample": sample, "cpu_model": _cpu_model()}
    if use_cpp:
        out["stage_seconds"] = stages
        out["hardware_concurrency"] = co.hardware_concurrency()
    else:
        try:
            from threadpoolctl import threadpool_info
            out["cores"] = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:  # threadpoolctl missing: numpy's BLAS default
            out["cores"] = os.cpu_count() or 1
    return out


def estimator_accuracy(dp, wl, layer_inputs, dev, nseeds=8, rademacher=False):
    """Relative RMS error of Hutch and Hutch++ (k = the workload's k) against the
    exact norms (the FGC contraction on the GPU) on the first layer, over
    ``nseeds`` probe seeds and all samples, with each estimator's time per
    call.  Outside the timed steps; not part of the throughput."""
    import torch
    A, G = layer_inputs
    B = A.shape[0]
    l = wl.layers[0]
    exact = torch.zeros(B, dtype=torch.float32, device=dev)
    dp.dp_norm_est("fgc", A, G, 0, 0, 0, exact)
    flags = dp.DP_PROBE_RADEMACHER if rademacher else 0
    out = {"layer": l.name, "k": wl.k, "seeds": nseeds, "exact": "FGC contraction on the GPU",
           "probes": "rademacher" if rademacher else "gaussian"}
    for m in ("hutch", "hutchpp"):
        ws = torch.empty(dp.dp_norm_est_workspace(m, wl.dtype, B, wl.T, l.d, l.p, wl.k),
                         dtype=torch.uint8, device=dev)
        n = torch.zeros(B, dtype=torch.float32, device=dev)
        dp.dp_norm_est(m, A, G, wl.k, 0, l.layer_id, n, flags=flags, ws=ws)  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        errs = []
        ms = 0.0
        for sd in range(nseeds):
            e0.record()
            dp.dp_norm_est(m, A, G, wl.k, 9000 + sd, l.layer_id, n, flags=flags, ws=ws)
            e1.record()
            torch.cuda.synchronize()
            ms += e0.elapsed_time(e1)
            errs.append((n.double() / exact.double() - 1.0).cpu())
        e = torch.stack(errs)
        out[f"{m}_rel_rms"] = float(torch.sqrt(torch.mean(e * e)))
        out[f"{m}_us_per_call"] = ms / nseeds * 1e3
    return out


def estimator_costs(dp, dev, reps=5):
    """Time and device memory of every estimator on one layer, outside the timed
    steps: the long-context layer (B 2, T 16384, d 2048, p 8192) for ghost-exact,
    Hutch (k 32), Hutch++ (k 32) and FGC, and the MLP up projection (B 8,
    T 4096, d 2048, p 8192) for the Hutch / Hutch++ latency ratio.

    Memory per estimator: the library allocates nothing, so a call's device
    memory beyond its inputs and n is its workspace (the *_workspace query);
    ``peak_bytes_measured`` is torch's peak-allocation increase over a call
    with that workspace allocated inside the measured window.  Beside them the
    summary's memory accounting (section 主要な貢献, 1. 複雑性の削減):
    O(B k T + k p) for randomized clipping, O(B min(d^2, T^2)) for the exact
    methods, here as fp32 bytes: B k T + k p for Hutch, B T^2 for materialised
    ghost Grams (two per sample), B d p for FGC's per-sample gradients."""
    import torch
    from sample_gradient_clipping_amd import roofline as rf
    from sample_gradient_clipping_amd.configs import workloads
    from sample_gradient_clipping_amd.inputs import linear_inputs_device
    W = workloads()
    out = {}
    for wname, methods in (("long_ctx_b2_t16384_d2048_p8192", ("ghost", "hutch", "hutchpp", "fgc")),
                           ("mlp_up_b8_t4096_d2048_p8192", ("hutch", "hutchpp"))):
        wl = W[wname]
        l = wl.layers[0]
        B, T, d, p, k = wl.B, wl.T, l.d, l.p, wl.k
        A, G = linear_inputs_device(B, T, d, p, wl.dtype, wl.recipe, wl.data_seed, l.layer_id, dev)
        n = torch.zeros(B, dtype=torch.float32, device=dev)
        res = {"B": B, "T": T, "d": d, "p": p, "k": k}
        for m in methods:
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats(dev)
            base = torch.cuda.memory_allocated(dev)
            wsb = dp.dp_norm_est_workspace(m, wl.dtype, B, T, d, p, k)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
            dp.dp_norm_est(m, A, G, k, 11, l.layer_id, n, ws=ws)
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated(dev) - base
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for r in range(reps):
                dp.dp_norm_est(m, A, G, k, 12 + r, l.layer_id, n, ws=ws)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            del ws
            if m == "ghost":
                pages = 4 * B * T * T * 2
            elif m == "fgc":
                pages = 4 * B * d * p
            else:
                pages = 4 * (B * k * T + k * p)
            flops = (rf.ghost_flops(B, T, d, p) if m == "ghost" else
                     rf.gemm_flops(B, T, d, p) if m == "fgc" else
                     rf.hutch_flops(B, T, d, p, k) if m == "hutch" else
                     rf.hutchpp_flops(B, T, d, p, k))
            res[m] = {"us_per_call": us, "workspace_bytes": int(wsb),
                      "peak_bytes_measured": int(peak), "pages_accounting_bytes": int(pages),
                      "flops": flops, "big_o_flops": rf.big_o_flops(m, B, T, d, p, k)}
        if "hutchpp" in res and "hutch" in res:
            res["hutchpp_over_hutch_time"] = res["hutchpp"]["us_per_call"] / res["hutch"]["us_per_call"]
        if "fgc" in res:
            res["hutch_workspace_over_fgc"] = res["hutch"]["workspace_bytes"] / res["fgc"]["workspace_bytes"]
            res["ghost_over_hutch_time"] = res["ghost"]["us_per_call"] / res["hutch"]["us_per_call"]
        out[wname] = res
        del A, G
        torch.cuda.empty_cache()
    return out


def read_ceiling(dp, dev, nbytes=512 << 20, reps=10):
    """The practical HBM read ceiling of this GPU: dp_stream_read (a plain streaming
    read with 16-byte loads) over a 512 MiB buffer (twice the MALL), the best of
    two grid sizes, HIP events over ``reps`` back-to-back reads."""
    import torch
    from sample_gradient_clipping_amd import roofline as rf
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    best = 0.0
    for nblocks in (1024, 2048):
        out = torch.zeros(nblocks, dtype=torch.int32, device=dev)
        for _ in range(3):
            dp.dp_stream_read(buf, out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            dp.dp_stream_read(buf, out)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del buf
    return {"GBps": best, "bytes": nbytes, "frac_of_spec": best / rf.PEAK_HBM_GBPS,
            "kernel": "dp_stream_read: 16-byte loads, 8 in flight per thread, 1024 or 2048 "
                      "workgroups of 256"}


def poisson_timing(dp, dev, reps=20):
    """Time the Poisson subsampling call (step 1 of DP-SGD) for two training-set
    sizes, with q chosen so that the expected minibatch is 8 sequences.
    Outside the timed steps."""
    import torch
    out = []
    for N in (1 << 20, 1 << 26):
        q = 8.0 / N
        idx = torch.empty(1024, dtype=torch.int64, device=dev)
        count = torch.empty(1, dtype=torch.int64, device=dev)
        ws = torch.empty(dp.dp_poisson_sample_workspace(N), dtype=torch.uint8, device=dev)
        dp.dp_poisson_sample(1, 0, N, q, idx, count, ws=ws)  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(reps):
            dp.dp_poisson_sample(1, t, N, q, idx, count, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        out.append({"N": N, "q": q, "us_per_call": us, "examples_per_s": N / (us * 1e-6),
                    "last_batch": int(count.item())})
    return out


def rmsnorm_timing(dp, wl, dev, reps=20):
    """Time the RMSNorm-gain norm pass (per-sample v_i and ||v_i||^2) at the
    workload's B and T, d = the first layer's input width, bf16.  Outside the
    timed steps; reported against HBM (it reads xhat and delta once)."""
    import torch
    from sample_gradient_clipping_amd.inputs import linear_inputs_device
    d = wl.layers[0].d
    copies = [linear_inputs_device(wl.B, wl.T, d, d, "bf16", "llama_logu", 4242 + c, 0, dev)
              for c in range(3)]  # rotated, so the 256 MB MALL cannot hold the inputs
    n = torch.zeros(wl.B, dtype=torch.float32, device=dev)
    v = torch.zeros(wl.B, d, dtype=torch.float32, device=dev)
    for X, D in copies:
        dp.dp_rmsnorm_norm(X, D, n, v=v)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        X, D = copies[r % 3]
        dp.dp_rmsnorm_norm(X, D, n, v=v)
    e1.record()
    torch.cuda.synchronize()
    del copies
    us = e0.elapsed_time(e1) / reps * 1e3
    nbytes = 2 * wl.B * wl.T * d * 2
    return {"B": wl.B, "T": wl.T, "d": d, "us_per_call": us, "GBps": nbytes / (us * 1e-6) / 1e9,
            "frac_hbm": nbytes / (us * 1e-6) / 8e12, "inputs": "3 rotated copies"}


def embedding_timing(dp, wl, dev, V=128256, reps=10):
    """Time the embedding-table norm pass and the table update (every row
    noised) at the workload's B and T, d = the first layer's input width, bf16,
    with a Llama-3.2-sized vocabulary and Zipf-like token ids.  Outside the
    timed steps."""
    import numpy as np
    import torch
    from sample_gradient_clipping_amd.inputs import linear_inputs_device
    B, T, d = wl.B, wl.T, wl.layers[0].d
    r = np.random.default_rng(77)
    ids = torch.from_numpy(np.minimum(r.zipf(1.3, size=(B, T)) - 1, V - 1).astype(np.int32)).to(dev)
    _, D = linear_inputs_device(B, T, 8, d, "bf16", "llama_logu", 4343, 0, dev)
    E = torch.zeros(V, d, dtype=torch.float32, device=dev)
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    dp.dp_embedding_norm(ids, D, n)
    dp.dp_embedding_clip_aggregate_update(ids, D, n, 1.0, 1.0, 1e-4, 7, 5000, E)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(reps):
        dp.dp_embedding_norm(ids, D, n)
    ev[1].record()
    for _ in range(reps):
        dp.dp_embedding_clip_aggregate_update(ids, D, n, 1.0, 1.0, 1e-4, 7, 5000, E)
    ev[2].record()
    torch.cuda.synchronize()
    us_n = ev[0].elapsed_time(ev[1]) / reps * 1e3
    us_u = ev[1].elapsed_time(ev[2]) / reps * 1e3
    bytes_n = B * T * d * 2
    bytes_u = 8 * V * d + B * T * d * 2  # E read and written, delta rows read once
    return {"B": B, "T": T, "d": d, "V": V, "distinct_ids_sample0": int(ids[0].unique().numel()),
            "norm_us": us_n, "norm_GBps": bytes_n / (us_n * 1e-6) / 1e9,
            "update_us": us_u, "update_GBps": bytes_u / (us_u * 1e-6) / 1e9}


def mlp_block_timing(dp, wl, dev, d=2048, f=8192, k=32, reps=5):
    """One DP-SGD-RC step of a Llama-3.2-1B-shaped MLP block (RMSNorm, SwiGLU
    gate/up/down, residual) at the workload's B and T: forward pass, backward
    pass 1, then norms (Hutch for the three linears, the gain exactly), clip,
    clipped sums, noise and updates of all four parameters.  Outside the timed
    steps; the NT GEMM of the forward pass is also timed alone."""
    import torch
    from sample_gradient_clipping_amd.inputs import mlp_block_inputs_device
    B, T = wl.B, wl.T
    M = B * T
    x, gamma, thetas, R = mlp_block_inputs_device(B, T, d, f, 5151, dev)
    Wb = {name: dp.dp_weights_bf16(t) for name, t in thetas.items()}
    acts, grads = {}, {}
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    v = torch.empty(B, d, dtype=torch.float32, device=dev)
    ids = {"W_gate": 0, "W_up": 1, "W_down": 2, "gamma": 3}

    def forward():
        dp.dp_mlp_forward(x, gamma, Wb["W_gate"][0], Wb["W_up"][0], Wb["W_down"][0], acts=acts)

    def backward():
        dp.dp_mlp_backward(x, acts["rstd"], gamma, acts["g"], acts["u"], Wb["W_gate"][1],
                           Wb["W_up"][1], Wb["W_down"][1], R, grads=grads)

    def dp_part(it):
        lin = {"W_gate": (acts["y"], grads["G_gate"]), "W_up": (acts["y"], grads["G_up"]),
               "W_down": (acts["h"], R)}
        dp.dp_rmsnorm_norm(acts["xhat"], grads["dy"], n, v=v)
        for name, (A, G) in lin.items():
            dp.dp_norm_est("hutch", A, G, k, 900 + it, ids[name], n, flags=dp.DP_ACCUMULATE)
        for name, (A, G) in lin.items():
            dp.dp_clip_aggregate_update(A, G, n, 1.0, 1.0, 1e-4, 1900 + it, ids[name],
                                        thetas[name])
        dp.dp_rmsnorm_clip_aggregate_update(v, n, 1.0, 1.0, 1e-4, 1900 + it, ids["gamma"], gamma)

    def gemm():
        dp.dp_linear_forward(acts["y"], Wb["W_gate"][0], C=acts["g"])

    forward(); backward(); dp_part(0); gemm()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    ev[0].record()
    for _ in range(reps):
        gemm()
    ev[1].record()
    for _ in range(reps):
        forward()
    ev[2].record()
    torch.cuda.synchronize()
    t_gemm = ev[0].elapsed_time(ev[1]) / reps
    t_fwd = ev[1].elapsed_time(ev[2]) / reps
    ev[0].record()
    for _ in range(reps):
        backward()
    ev[1].record()
    for it in range(reps):
        dp_part(it + 1)
    ev[2].record()
    for it in range(reps):
        forward(); backward(); dp_part(it + 1)
    ev[3].record()
    torch.cuda.synchronize()
    t_bwd = ev[0].elapsed_time(ev[1]) / reps
    t_dp = ev[1].elapsed_time(ev[2]) / reps
    t_step = ev[2].elapsed_time(ev[3]) / reps
    gemm_flops = 2.0 * M * d * f
    del acts, grads
    return {"B": B, "T": T, "d": d, "f": f, "k": k, "method": "hutch",
            "nt_gemm_us": t_gemm * 1e3, "nt_gemm_TFLOPs": gemm_flops / (t_gemm * 1e-3) / 1e12,
            "nt_gemm_frac_mfma": gemm_flops / (t_gemm * 1e-3) / 2.5e15,
            "forward_ms": t_fwd, "forward_TFLOPs": 3 * gemm_flops / (t_fwd * 1e-3) / 1e12,
            "backward1_ms": t_bwd, "backward1_TFLOPs": 3 * gemm_flops / (t_bwd * 1e-3) / 1e12,
            "dp_step_ms": t_dp, "block_step_ms": t_step,
            "block_step_tokens_per_s": M / (t_step * 1e-3)}


def attn_block_timing(dp, wl, dev, d=2048, H=32, KV=8, k=32, reps=5):
    """One DP-SGD-RC step of a Llama-3.2-1B-shaped attention block (RMSNorm, q/k/v
    projections, RoPE, causal grouped-query attention, o projection, residual) at
    the workload's B and T: forward pass, backward pass 1, then Hutch norms of the
    four linears, the gain's exact norm, clip, clipped sums, noise and updates.
    Outside the timed steps; the attention kernels are also timed alone."""
    import torch
    B, T = wl.B, wl.T
    M = B * T
    gen = torch.Generator(device=dev)
    gen.manual_seed(6161)

    def randn(*shape):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)

    x = randn(B, T, d).to(torch.bfloat16)
    gamma = 1.0 + 0.1 * randn(d)
    thetas = {"W_q": 0.02 * randn(64 * H, d), "W_k": 0.02 * randn(64 * KV, d),
              "W_v": 0.02 * randn(64 * KV, d), "W_o": 0.02 * randn(d, 64 * H)}
    R = (0.01 * randn(B, T, d)).to(torch.bfloat16)
    Wb = {name: dp.dp_weights_bf16(t) for name, t in thetas.items()}
    acts, grads = {}, {}
    ws = torch.empty(dp.load_library().dp_attn_backward_workspace(B, T, H), dtype=torch.uint8,
                     device=dev)
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    v = torch.empty(B, d, dtype=torch.float32, device=dev)
    ids = {"W_q": 0, "W_k": 1, "W_v": 2, "W_o": 3, "gamma": 4}

    def forward():
        dp.dp_attn_forward(x, gamma, Wb["W_q"][0], Wb["W_k"][0], Wb["W_v"][0], Wb["W_o"][0], H, KV,
                           acts=acts)

    def backward():
        dp.dp_attn_backward(x, acts, gamma, Wb["W_q"][1], Wb["W_k"][1], Wb["W_v"][1], Wb["W_o"][1],
                            R, H, KV, grads=grads, ws=ws)

    def dp_part(it):
        lin = {"W_q": (acts["y"], grads["G_q"]), "W_k": (acts["y"], grads["G_k"]),
               "W_v": (acts["y"], grads["G_v"]), "W_o": (acts["o"], R)}
        dp.dp_rmsnorm_norm(acts["xhat"], grads["dy"], n, v=v)
        for name, (A, G) in lin.items():
            dp.dp_norm_est("hutch", A, G, k, 700 + it, ids[name], n, flags=dp.DP_ACCUMULATE)
        for name, (A, G) in lin.items():
            dp.dp_clip_aggregate_update(A, G, n, 1.0, 1.0, 1e-4, 1700 + it, ids[name],
                                        thetas[name])
        dp.dp_rmsnorm_clip_aggregate_update(v, n, 1.0, 1.0, 1e-4, 1700 + it, ids["gamma"], gamma)

    dO = (0.01 * randn(B, T, 64 * H)).to(torch.bfloat16)

    def attn_only_fwd():
        dp.dp_attention_forward(acts["q"], acts["k"], acts["v"], H, KV, o=acts["o"], lse=acts["lse"])

    def attn_only_bwd():
        dp.dp_attention_backward(acts["q"], acts["k"], acts["v"], acts["o"], acts["lse"], dO, H, KV)

    forward(); backward(); dp_part(0); attn_only_fwd(); attn_only_bwd()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    ev[0].record()
    for _ in range(reps):
        attn_only_fwd()
    ev[1].record()
    for _ in range(reps):
        attn_only_bwd()
    ev[2].record()
    for _ in range(reps):
        forward()
    ev[3].record()
    for _ in range(reps):
        backward()
    ev[4].record()
    for it in range(reps):
        dp_part(it + 1)
    ev[5].record()
    for it in range(reps):
        forward(); backward(); dp_part(it + 1)
    ev[6].record()
    torch.cuda.synchronize()
    t = [ev[i].elapsed_time(ev[i + 1]) / reps for i in range(6)]
    attn_flops = 128.0 * B * H * T * T  # two products of 2 * 64 flops per (query, key), causal half
    del acts, grads
    return {"B": B, "T": T, "d": d, "H": H, "KV": KV, "k": k, "method": "hutch",
            "attention_fwd_ms": t[0], "attention_fwd_TFLOPs": attn_flops / (t[0] * 1e-3) / 1e12,
            "attention_bwd_ms": t[1],
            "attention_bwd_TFLOPs": 3.5 * attn_flops / (t[1] * 1e-3) / 1e12,
            "forward_ms": t[2], "backward1_ms": t[3], "dp_step_ms": t[4], "block_step_ms": t[5],
            "block_step_tokens_per_s": M / (t[5] * 1e-3)}


def layer_timing(dp, wl, dev, d=2048, f=8192, H=32, KV=8, k=32, reps=3):
    """One DP-SGD-RC step of a whole Llama-3.2-1B-shaped decoder layer at the
    workload's B and T: the attention block's forward pass feeding the MLP
    block's, backward pass 1 through both (the MLP block's dL/d(input) is the
    attention block's output gradient), then Hutch norms of the seven linears and
    the two gains' exact norms summed per sample, one clip factor per sample,
    and the clipped sums, noise and updates of all eleven parameters."""
    import torch
    from sample_gradient_clipping_amd.inputs import mlp_block_inputs_device
    B, T = wl.B, wl.T
    M = B * T
    x, g_mlp, th_mlp, R = mlp_block_inputs_device(B, T, d, f, 7171, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7272)

    def randn(*shape):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)

    g_attn = 1.0 + 0.1 * randn(d)
    thetas = {"W_q": 0.02 * randn(64 * H, d), "W_k": 0.02 * randn(64 * KV, d),
              "W_v": 0.02 * randn(64 * KV, d), "W_o": 0.02 * randn(d, 64 * H), **th_mlp}
    Wb = {name: dp.dp_weights_bf16(t) for name, t in thetas.items()}
    a_acts, a_grads, m_acts, m_grads = {}, {}, {}, {}
    ws = torch.empty(dp.load_library().dp_attn_backward_workspace(B, T, H), dtype=torch.uint8,
                     device=dev)
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    va = torch.empty(B, d, dtype=torch.float32, device=dev)
    vm = torch.empty(B, d, dtype=torch.float32, device=dev)
    ids = {"W_q": 0, "W_k": 1, "W_v": 2, "W_o": 3, "gamma": 4, "W_gate": 5, "W_up": 6,
           "W_down": 7, "mlp_gamma": 8}

    def step(it):
        dp.dp_attn_forward(x, g_attn, Wb["W_q"][0], Wb["W_k"][0], Wb["W_v"][0], Wb["W_o"][0], H,
                           KV, acts=a_acts)
        h1 = a_acts["out"]
        dp.dp_mlp_forward(h1, g_mlp, Wb["W_gate"][0], Wb["W_up"][0], Wb["W_down"][0], acts=m_acts)
        dp.dp_mlp_backward(h1, m_acts["rstd"], g_mlp, m_acts["g"], m_acts["u"], Wb["W_gate"][1],
                           Wb["W_up"][1], Wb["W_down"][1], R, grads=m_grads)
        dp.dp_attn_backward(x, a_acts, g_attn, Wb["W_q"][1], Wb["W_k"][1], Wb["W_v"][1],
                            Wb["W_o"][1], m_grads["dx"], H, KV, grads=a_grads, ws=ws)
        lin = {"W_q": (a_acts["y"], a_grads["G_q"]), "W_k": (a_acts["y"], a_grads["G_k"]),
               "W_v": (a_acts["y"], a_grads["G_v"]), "W_o": (a_acts["o"], m_grads["dx"]),
               "W_gate": (m_acts["y"], m_grads["G_gate"]), "W_up": (m_acts["y"], m_grads["G_up"]),
               "W_down": (m_acts["h"], R)}
        dp.dp_rmsnorm_norm(a_acts["xhat"], a_grads["dy"], n, v=va)
        dp.dp_rmsnorm_norm(m_acts["xhat"], m_grads["dy"], n, v=vm, flags=dp.DP_ACCUMULATE)
        for name, (A, G) in lin.items():
            dp.dp_norm_est("hutch", A, G, k, 1100 + it, ids[name], n, flags=dp.DP_ACCUMULATE)
        for name, (A, G) in lin.items():
            dp.dp_clip_aggregate_update(A, G, n, 1.0, 1.0, 1e-4, 2100 + it, ids[name],
                                        thetas[name])
        dp.dp_rmsnorm_clip_aggregate_update(va, n, 1.0, 1.0, 1e-4, 2100 + it, ids["gamma"], g_attn)
        dp.dp_rmsnorm_clip_aggregate_update(vm, n, 1.0, 1.0, 1e-4, 2100 + it, ids["mlp_gamma"],
                                            g_mlp)

    step(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for it in range(reps):
        step(it + 1)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps
    del a_acts, a_grads, m_acts, m_grads
    return {"B": B, "T": T, "d": d, "f": f, "H": H, "KV": KV, "k": k, "method": "hutch",
            "parameters": 11, "layer_step_ms": t, "layer_step_tokens_per_s": M / (t * 1e-3)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the hot path is "
              "built and measured on one MI355X; multi-GPU sharding is a design note, not built.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from sample_gradient_clipping_amd import binding as dp
    from sample_gradient_clipping_amd import roofline as rf
    from sample_gradient_clipping_amd.configs import workloads

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 1 GiB device copies")
        return

    wl = workloads()[args.workload]
    method = args.method or wl.method
    dev = torch.device("cuda:0")
    dp.load_library()
    E = rf.elem_size(wl.dtype)
    per_copy = sum(wl.tokens * (l.d + l.p) * E for l in wl.layers)
    copies = args.copies or max(1, min(4, math.ceil((768 << 20) / per_copy)))
    log(f"[bench] workload {wl.name}: B={wl.B} T={wl.T} layers={len(wl.layers)} method={method} "
        f"k={wl.k} inputs {per_copy / 2**30:.2f} GiB x {copies} copies")
    inputs = make_inputs(wl, copies, dev)

    L = len(wl.layers)
    n = torch.zeros(wl.B, dtype=torch.float32, device=dev)
    S = ([torch.empty(l.p, l.d, dtype=torch.float32, device=dev) for l in wl.layers]
         if args.unfused else None)
    theta = [torch.zeros(l.p, l.d, dtype=torch.float32, device=dev) for l in wl.layers]
    # the batched calls over the step's layers (one descriptor list per input copy)
    lay_n = [[(A, G, l.layer_id) for (A, G), l in zip(cp, wl.layers)] for cp in inputs]
    lay_u = [[(A, G, l.layer_id, th) for (A, G), l, th in zip(cp, wl.layers, theta)]
             for cp in inputs]
    ws_n = max(dp.dp_norm_est_workspace(method, wl.dtype, wl.B, wl.T, l.d, l.p, wl.k)
               for l in wl.layers)
    ws_n = max(ws_n, dp.dp_norm_est_layers_workspace(method, wl.dtype, wl.B, wl.T, wl.k, lay_n[0]))
    ws_a = max(dp.dp_clip_aggregate_update_workspace(wl.dtype, wl.B, wl.T, l.d, l.p)
               for l in wl.layers)
    ws_a = max(ws_a, dp.dp_clip_aggregate_update_layers_workspace(wl.dtype, wl.B, wl.T, lay_u[0]))
    ws_norm = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    ws_agg = dp.clip_workspace(ws_a, dev)

    K, W = args.steps, args.warmup
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(L)]
          for _ in range(K)]
    for s in ev:
        for l in s:
            for e in l:
                e.record()
    torch.cuda.synchronize()

    def step(it, evs, only=None):
        """One step.  evs: per layer the six events (norm_est, aggregate, noise_update
        pairs), or None; with ``only`` set, just that kernel's pair is recorded.  The
        batched norm call records its pair once, in layer 0's slot, around all layers'
        streaming passes."""
        def pair(li, name):
            if evs is None or (only is not None and only != name):
                return None
            j = {"norm_est": 0, "aggregate": 2, "noise_update": 4}[name]
            return (evs[li][j], evs[li][j + 1])
        ci = it % copies
        cp = inputs[ci]
        probe = dp.DP_PROBE_RADEMACHER if args.rademacher else 0
        if args.per_layer:  # one call per layer
            for li, l in enumerate(wl.layers):
                A, G = cp[li]
                dp.dp_norm_est(method, A, G, wl.k, wl.method_seed + it, l.layer_id, n,
                               flags=(dp.DP_ACCUMULATE if li else 0) | probe, ws=ws_norm,
                               events=pair(li, "norm_est"))
        else:  # all layers in one call
            dp.dp_norm_est_layers(method, lay_n[ci], wl.k, wl.method_seed + it, n, flags=probe,
                                  ws=ws_norm, events=pair(0, "norm_est"))
        if args.unfused:  # clipped sum to S, then noise + update: two calls per layer
            for li, l in enumerate(wl.layers):
                A, G = cp[li]
                dp.dp_clip_aggregate(A, G, n, wl.C, S[li], ws=ws_agg, events=pair(li, "aggregate"))
                dp.dp_noise_update(theta[li], S[li], wl.sigma, wl.C, wl.eta, wl.B,
                                   wl.noise_seed + it, l.layer_id, events=pair(li, "noise_update"))
        elif args.per_layer:  # one fused call per layer: clip, clipped sum, noise, update
            for li, l in enumerate(wl.layers):
                A, G = cp[li]
                ea, eu = pair(li, "aggregate"), pair(li, "noise_update")
                dp.dp_clip_aggregate_update(
                    A, G, n, wl.C, wl.sigma, wl.eta, wl.noise_seed + it, l.layer_id, theta[li],
                    ws=ws_agg, events=None if ea is None and eu is None else (ea, eu))
        else:  # all layers in one call: the clip factors once, then per layer the rest
            ea = [pair(li, "aggregate") for li in range(L)]
            eu = [pair(li, "noise_update") for li in range(L)]
            dp.dp_clip_aggregate_update_layers(
                lay_u[ci], n, wl.C, wl.sigma, wl.eta, wl.noise_seed + it, ws=ws_agg,
                agg_events=None if all(e is None for e in ea) else ea,
                upd_events=None if all(e is None for e in eu) else eu)

    for it in range(W):
        step(it, None)
    torch.cuda.synchronize()

    # An instrumented pass outside the timed region: every kernel group's duration,
    # which picks the dominant kernel.  Inside the timed steps only the dominant
    # kernel's launches are bracketed by events (each event record costs GPU time).
    KI = min(K, 10)
    ev_i = [[[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(L)]
            for _ in range(KI)]
    for it in range(KI):
        step(W + it, ev_i[it])
    torch.cuda.synchronize()
    t_inst = {"norm_est": 0.0, "aggregate": 0.0, "noise_update": 0.0}
    for it in range(KI):
        for li in range(L):
            e = ev_i[it][li]
            if args.per_layer or li == 0:
                t_inst["norm_est"] += e[0].elapsed_time(e[1]) / KI
            t_inst["aggregate"] += e[2].elapsed_time(e[3]) / KI
            t_inst["noise_update"] += e[4].elapsed_time(e[5]) / KI
    dom_name = max(t_inst, key=t_inst.get)

    # Every EV_STRIDE-th timed step brackets each launch of the dominant kernel with
    # two events; an event record costs the GPU a few microseconds, about 1.5% of a
    # step when every launch of every step is bracketed.
    timed_ev = [it for it in range(K) if it % EV_STRIDE == 0]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for it in range(K):
        step(W + KI + it, ev[it] if it % EV_STRIDE == 0 else None, only=dom_name)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / K
    tokens_per_s = wl.tokens * K / (ms_total / 1e3)
    log(f"[bench] {K} steps in {ms_total:.3f} ms (wall {wall * 1e3:.1f} ms): {ms_step:.4f} ms/step, "
        f"{tokens_per_s / 1e6:.2f} M tokens/s")

    # Per-step durations: the dominant kernel from its events in the timed steps, the
    # others from the instrumented pass.
    t_step = dict(t_inst)
    j = {"norm_est": 0, "aggregate": 2, "noise_update": 4}[dom_name]
    t_step[dom_name] = sum(ev[it][li][j].elapsed_time(ev[it][li][j + 1])
                           for it in timed_ev for li in range(L)
                           if dom_name != "norm_est" or args.per_layer or li == 0) / len(timed_ev)
    t_norm, t_agg, t_noise = (t_step["norm_est"] * K, t_step["aggregate"] * K,
                              t_step["noise_update"] * K)
    launches = K * L
    # the batched update shares contraction launches between layers whose output
    # tiles are too few to fill the chip alone: per-launch figures use real launches
    agg_per_step = (L if args.per_layer or args.unfused else
                    dp.dp_clip_aggregate_update_layers_launches(wl.dtype, wl.B, wl.T, lay_u[0]))
    if method in ("hutch",):
        b_norm = sum(rf.hutch_bytes(wl.B, wl.T, l.d, l.p, wl.dtype) for l in wl.layers)
        f_norm = sum(rf.hutch_flops(wl.B, wl.T, l.d, l.p, wl.k) for l in wl.layers)
    elif method == "hutchpp":
        b_norm = sum(rf.hutchpp_bytes(wl.B, wl.T, l.d, l.p, wl.dtype) for l in wl.layers)
        f_norm = sum(rf.hutchpp_flops(wl.B, wl.T, l.d, l.p, wl.k) for l in wl.layers)
    elif method == "ghost":
        b_norm = sum(rf.hutch_bytes(wl.B, wl.T, l.d, l.p, wl.dtype) for l in wl.layers)
        f_norm = sum(rf.ghost_flops(wl.B, wl.T, l.d, l.p) for l in wl.layers)
    else:
        b_norm = sum(rf.fgc_bytes(wl.B, wl.T, l.d, l.p, wl.dtype) for l in wl.layers)
        f_norm = sum(rf.gemm_flops(wl.B, wl.T, l.d, l.p) for l in wl.layers)
    f_agg = sum(rf.gemm_flops(wl.B, wl.T, l.d, l.p) for l in wl.layers)
    b_agg = sum(rf.aggregate_bytes(wl.B, wl.T, l.d, l.p, wl.dtype) for l in wl.layers)
    b_noise = sum(rf.noise_bytes(l.d, l.p) for l in wl.layers)
    # per step: algorithmic work of all layers / summed kernel time of one step
    s_norm, s_agg, s_noise = t_norm / K / 1e3, t_agg / K / 1e3, t_noise / K / 1e3
    kernels = {
        "norm_est": {"name": f"{method} passes (per layer: sketch+projection"
                     + ("" if args.per_layer else "; all layers timed in one call, per-layer mean")
                     + ")" if method == "hutch"
                     else f"{method} main kernels", "ms_per_launch": t_norm / launches,
                     "bound": "hbm" if method in ("hutch", "hutchpp") else "mfma",
                     "GBps": b_norm / s_norm / 1e9, "TFLOPs": f_norm / s_norm / 1e12},
        "aggregate": {"name": "clipped-sum contraction", "ms_per_launch": t_agg / (K * agg_per_step),
                      "launches_per_step": agg_per_step,
                      "bound": "mfma", "GBps": b_agg / s_agg / 1e9, "TFLOPs": f_agg / s_agg / 1e12},
        "noise_update": {"name": "Philox noise + SGD update" + (
                             "" if args.unfused else " (summing the contraction's token splits)"),
                         "ms_per_launch": t_noise / launches,
                         "bound": "hbm", "GBps": b_noise / s_noise / 1e9},
    }
    for kname, kv in kernels.items():
        kv["frac"] = (kv["GBps"] / rf.PEAK_HBM_GBPS if kv["bound"] == "hbm"
                      else kv["TFLOPs"] / rf.PEAK_BF16_TFLOPS)
        kv["share_of_step"] = (kv["ms_per_launch"] * kv.get("launches_per_step", L)) / ms_step
    for kname, kv in kernels.items():
        kv["timing"] = (f"HIP events in every {EV_STRIDE}th timed step ({len(timed_ev)} of {K})"
                        if kname == dom_name else
                        f"HIP events in an instrumented pass of {KI} steps before the timed ones")
    dom = kernels[dom_name]
    traffic = measured_traffic(dom_name, wl.name)
    if dom["bound"] == "hbm":
        roof = {"bound": "hbm", "achieved": dom["GBps"], "peak": rf.PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": dom["GBps"] / rf.PEAK_HBM_GBPS, "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": dom["TFLOPs"], "peak": rf.PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": dom["TFLOPs"] / rf.PEAK_BF16_TFLOPS, "traffic": traffic}
    roof["kernel"] = dom["name"]
    roof["algorithmic_per_launch"] = (
        {"bytes": b_norm / L} if dom["bound"] == "hbm" and dom_name == "norm_est" else
        {"bytes": b_noise / L} if dom_name == "noise_update" else
        {"flops": f_agg / agg_per_step, "bytes": b_agg / agg_per_step} if dom_name == "aggregate" else
        {"flops": f_norm / L, "bytes": b_norm / L})
    ceiling = None
    if not args.only_step:
        # the practical HBM read ceiling, measured in the same run, beside the spec fraction
        ceiling = read_ceiling(dp, dev)
        log(f"[bench] HBM read ceiling {ceiling['GBps']:.1f} GB/s ({ceiling['frac_of_spec']:.3f} of spec)")
        for kv in kernels.values():
            if kv["bound"] == "hbm":
                kv["frac_of_read_ceiling"] = kv["GBps"] / ceiling["GBps"]
    for kname, kv in kernels.items():
        log(f"[bench] {kname:13s} {kv['ms_per_launch'] * 1e3:9.2f} us/launch  "
            f"{kv['GBps']:8.1f} GB/s  {kv.get('TFLOPs', 0):8.1f} TF/s  frac {kv['frac']:.3f}  "
            f"share {kv['share_of_step']:.2f}"
            + (f"  of read ceiling {kv['frac_of_read_ceiling']:.3f}" if "frac_of_read_ceiling" in kv
               else ""))

    accuracy = sampler = rms = emb = mlp = attn = layer = costs = None
    if not args.only_step:
        accuracy = estimator_accuracy(dp, wl, inputs[0][0], dev, rademacher=args.rademacher)
        log(f"[bench] estimator accuracy {accuracy}")
        sampler = poisson_timing(dp, dev)
        log(f"[bench] poisson sampler {sampler}")
        rms = rmsnorm_timing(dp, wl, dev) if wl.dtype == "bf16" else None
        log(f"[bench] rmsnorm gain norms {rms}")
        emb = embedding_timing(dp, wl, dev) if wl.dtype == "bf16" else None
        log(f"[bench] embedding {emb}")
        del inputs
        torch.cuda.empty_cache()
        costs = estimator_costs(dp, dev)
        log(f"[bench] estimator costs {costs}")
        torch.cuda.empty_cache()
        mlp = mlp_block_timing(dp, wl, dev) if wl.dtype == "bf16" else None
        log(f"[bench] mlp block {mlp}")
        torch.cuda.empty_cache()
        attn = attn_block_timing(dp, wl, dev) if wl.dtype == "bf16" and wl.T % 128 == 0 else None
        log(f"[bench] attention block {attn}")
        torch.cuda.empty_cache()
        layer = layer_timing(dp, wl, dev) if wl.dtype == "bf16" and wl.T % 128 == 0 else None
        log(f"[bench] decoder layer {layer}")

    cpu = None
    if not args.no_cpu_baseline and not args.only_step:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(wl, method, rademacher=args.rademacher)
        log(f"[bench] cpu_baseline {cpu}")

    line = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "layers": len(wl.layers),
                   "shapes_dp": sorted({(l.d, l.p) for l in wl.layers}), "method": method,
                   "k": wl.k, "probes": "rademacher" if args.rademacher else "gaussian",
                   "C": wl.C, "sigma": wl.sigma, "eta": wl.eta,
                   "input_copies": copies, "global_batch": wl.B, "seq_len": wl.T,
                   "calls": ("one per layer" if args.per_layer or args.unfused
                             else "batched over the layers")},
        "roofline": roof,
        "kernels": kernels,
        "hbm_read_ceiling": ceiling,
        "estimator_accuracy": accuracy,
        "estimator_costs": costs,
        "poisson_sampler": sampler,
        "rmsnorm_gain_norms": rms,
        "embedding": emb,
        "mlp_block": mlp,
        "attn_block": attn,
        "decoder_layer": layer,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
