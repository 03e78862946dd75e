#!/usr/bin/env python3
"""Benchmark of the W4A16 fused dequantize-GEMM on one MI355X.

One step = every linear of a decode step of the chosen workload, each a W4A16 GEMM through
the library's C ABI. The default is the Llama-3-70B-shaped decode step at M = 1: 80 layers x
{qkv 8192x10240, o 8192x8192, gate+up 8192x57344, down 28672x8192}, symmetric INT4 g128,
fp16, the whole 35.3 GB INT4 weight set resident on the one GPU. Each linear has its own
weight buffers, so the set streams from HBM every step (it is 140 times the 256 MB Infinity
Cache). The step is captured once as a HIP graph and replayed: W untimed replays, then K
timed replays between HIP events on the replay stream. Weights are seeded random codes and
scales drawn on the device, activations seeded N(0, 1) from the host; all are resident in HBM
before the timed region starts.

Prints one JSON line: metric/value (whole-step effective GB/s over algorithmic bytes), the
roofline object of the step's dominant kernel, a second roofline object for the same-metric
M = 256 point (the 4096x14336 g128 crossover shape, TFLOP/s against the dense fp16 MFMA
peak), the measured streaming ceiling of the box, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMM effective HBM GB/s at M=1 (% of peak) and TFLOPS at M=256"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
MFMA_I8_PEAK_TOPS = 5033.2     # dense int8 MFMA: twice the fp16 rate (published 5.0 POP/s)

WORKLOADS = {
    # name: shapes (K, N), layers, group size, symmetric, activation dtype, seed config
    "llama3-8b-decode": dict(shapes=[(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096)],
                             names=["qkv", "o", "gate_up", "down"], layers=32, g=128,
                             sym=False, act="f16", config=2, m=1),
    "llama3-70b-decode": dict(shapes=[(8192, 10240), (8192, 8192), (8192, 57344), (28672, 8192)],
                              names=["qkv", "o", "gate_up", "down"], layers=80, g=128,
                              sym=True, act="f16", config=3, m=1),
    "gemv-4096x4096": dict(shapes=[(4096, 4096)], names=["w"], layers=120, g=128, sym=False,
                           act="f16", config=1, m=1),
    "crossover-4096x14336-g128": dict(shapes=[(4096, 14336)], names=["w"], layers=32, g=128,
                                      sym=False, act="f16", config=4, m=256),
    "crossover-4096x14336-g32": dict(shapes=[(4096, 14336)], names=["w"], layers=32, g=32,
                                     sym=False, act="f16", config=4, m=256),
    "crossover-4096x14336-nf4": dict(shapes=[(4096, 14336)], names=["w"], layers=32, g=64,
                                     sym=True, act="f16", config=4, m=256, nf4=True),
    "prefill-2048x8192x28672-bf16": dict(shapes=[(8192, 28672)], names=["w"], layers=4, g=128,
                                         sym=False, act="bf16", config=5, m=2048),
}


def algo_bytes(M, K, N, g, zeros, nf4=False, act_bytes=2, out_bytes=2):
    """Bytes the GEMM must move: codes, scales (or NF4 absmax), zeros, x and y."""
    G = K // g
    b = K * N // 2 + G * N * 2 + act_bytes * M * K + out_bytes * M * N
    if zeros and not nf4:
        b += G * N // 2
    return b


KERNEL_SOURCES = {
    # kernel family -> the sources that define its code and launch geometry
    "decode": lambda f: f.startswith("w4a16_decode"),
    "tiled": lambda f: f.startswith("w4a16_tiled"),
    "skinny": lambda f: f == "w4a16_skinny.hip",
}


def kernel_family(kernel: str) -> str:
    for family in ("decode", "skinny"):
        if kernel.startswith("w4a16_" + family):
            return family
    return "tiled"


def source_hash(family: str = "decode") -> str:
    """Hash of the sources that define a kernel family's code and launch geometry (the
    kernel the committed HBM-traffic counters were taken on), with the shared device and
    launch headers; the dispatch that picks it is checked separately, by kernel name."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_only_int4_w4a16_amd", "csrc")
    pick = KERNEL_SOURCES[family]
    for f in sorted(os.listdir(csrc)):
        if not (pick(f) or f in ("w4a16_device.hpp", "w4a16_launch.hpp")):
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, m: int):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they were taken on
    the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    key = f"{workload}:M={m}"
    rec = data.get(key)
    if not rec or rec.get("source_hash") != source_hash(kernel_family(kernel)) \
            or rec.get("kernel") != kernel:
        return None
    return rec.get("bytes_per_launch")


def device_weights(K, N, g, seed, torch, w4, symmetric=False, scale_dtype=None, nf4=False):
    """Seeded timing weights drawn on the device (kernel time does not depend on the values):
    uniform random code words, packed by the library; scales U[0.004, 0.009] (NF4 absmax
    U[0.02, 0.09], fp16); uniform zero words unless symmetric."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    qw = torch.randint(-2**31, 2**31 - 1, (K // 8, N), dtype=torch.int32, device=dev, generator=gen)
    packed = w4.pack(qw)
    del qw
    lo, hi = (0.02, 0.09) if nf4 else (0.004, 0.009)
    sdt = torch.float16 if (nf4 or scale_dtype is None) else scale_dtype
    sc = (torch.rand((K // g, N), device=dev, generator=gen) * (hi - lo) + lo).to(sdt)
    qz = None
    if not symmetric and not nf4:
        qz = torch.randint(-2**31, 2**31 - 1, (K // g, N // 8), dtype=torch.int32, device=dev,
                           generator=gen)
    return packed, sc, qz


def build_workload(spec, M, torch, w4, synth):
    """Device buffers for every (layer, linear): packed codes, scales, zeros drawn on the
    device per (config, shape, layer) seed; x from the host generator; y."""
    act = spec["act"]
    tdt = torch.float16 if act == "f16" else torch.bfloat16
    nf4 = spec.get("nf4", False)
    dev = torch.device("cuda:0")
    layers = []
    for layer in range(spec["layers"]):
        lin = []
        for si, (K, N) in enumerate(spec["shapes"]):
            seed = synth.seed_for(spec["config"], si, 0, layer)
            packed, sct, qzt = device_weights(K, N, spec["g"], seed, torch, w4, symmetric=spec["sym"],
                                              scale_dtype=tdt, nf4=nf4)
            lin.append(dict(K=K, N=N, packed=packed, scales=sct, qzeros=qzt))
        layers.append(lin)
    xs, ys = [], []
    for si, (K, N) in enumerate(spec["shapes"]):
        x = synth.activations(M, K, synth.seed_for(spec["config"], si, synth.ROLE_X), act)
        xt = torch.from_numpy(x.view("int16") if act == "bf16" else x).to(dev)
        if act == "bf16":
            xt = xt.view(torch.bfloat16)
        xs.append(xt)
        ys.append(torch.empty((M, N), dtype=tdt, device=dev))
    codebook = None
    if nf4:
        import numpy as np
        vals = np.loadtxt(os.path.join(ROOT, "tests", "golden", "nf4_codebook.txt"))
        codebook = torch.from_numpy(vals.astype(np.float16)).to(dev)
    torch.cuda.synchronize()
    return layers, xs, ys, codebook


def make_step(spec, layers, xs, ys, codebook, w4, only=None):
    """One pass over every (layer, linear); with ``only`` = a linear index, that linear of
    every layer."""
    g = spec["g"]
    nf4 = spec.get("nf4", False)

    def step():
        for lin in layers:
            for si, L in enumerate(lin):
                if only is not None and si != only:
                    continue
                if nf4:
                    w4.gemm_nf4(xs[si], L["packed"], L["scales"], codebook, g, out=ys[si])
                else:
                    w4.gemm(xs[si], L["packed"], L["scales"], L["qzeros"], g, out=ys[si])
    return step


def cpu_baseline(spec, M, cols=2048, reps=5):
    """The CPU oracle as written, timed per linear of one layer: the NumPy dequantization and
    the fp64 matmul separately, median of ``reps`` runs each, on a ``cols``-column slice of
    each linear (both scale linearly in N). The step projection scales each linear by
    N / cols and the layer by the layer count; GB/s uses the same algorithmic bytes as the
    GPU. NumPy's elementwise work runs on one thread, the matmul on the BLAS threads."""
    import platform

    import numpy as np

    import oracle
    from weight_only_int4_w4a16_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    act = spec["act"]
    nf4 = spec.get("nf4", False)
    zeros = not spec["sym"] and not nf4
    per, step_s, step_bytes, wall0 = [], 0.0, 0, time.perf_counter()
    for si, (K, N) in enumerate(spec["shapes"]):
        n = min(cols, N)
        seed = synth.seed_for(spec["config"], si, 0, 0)
        qw, sc, qz = synth.timing_weights(K, n, spec["g"], seed, symmetric=not zeros,
                                          scale_dtype=act if not nf4 else "f16")
        x = synth.activations(M, K, synth.seed_for(spec["config"], si, synth.ROLE_X), act)
        td, tm = [], []
        for _ in range(reps):
            t0 = time.perf_counter()
            if nf4:
                w_hat = oracle.dequant_nf4(qw, sc, oracle.nf4_codebook(), spec["g"], act)
            else:
                w_hat = oracle.dequant_affine(qw, sc, qz, spec["g"], act)
            t1 = time.perf_counter()
            oracle.gemm_ref(x, w_hat, act)
            t2 = time.perf_counter()
            td.append(t1 - t0)
            tm.append(t2 - t1)
            del w_hat
        d, m = float(np.median(td)), float(np.median(tm))
        scale = N / n
        step_s += (d + m) * scale * spec["layers"]
        step_bytes += algo_bytes(M, K, N, spec["g"], zeros, nf4) * spec["layers"]
        per.append({"linear": spec["names"][si], "K": K, "N": N, "sample_cols": n,
                    "dequant_s_median": round(d, 4), "matmul_s_median": round(m, 4),
                    "GB/s": round(algo_bytes(M, K, n, spec["g"], zeros, nf4) / (d + m) / 1e9, 4)})
    return {"value": round(step_bytes / step_s / 1e9, 4), "unit": "GB/s",
            "cores": int(blas_threads), "kind": "oracle",
            "host_cpus": os.cpu_count(), "host_cpu": platform.processor() or platform.machine(),
            "step_s_projected": round(step_s, 2),
            "sample": (f"one layer of {spec['name']} at M={M}: each linear on its first {cols} "
                       f"columns, NumPy dequant (1 thread) and fp64 matmul ({blas_threads} BLAS "
                       f"threads) timed separately, median of {reps}; projected to the full "
                       f"step by N/{cols} per linear and x{spec['layers']} layers; "
                       f"{time.perf_counter() - wall0:.1f} s of CPU time"),
            "per_linear": per}


SWEEP = [
    # (config name, format, group, act, [(K, N)], [M])
    ("c1 gemv", "asym", 128, "f16", [(4096, 4096)], [1]),
    ("c2 llama3-8b", "asym", 128, "f16", [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096)],
     [1, 4, 16]),
    ("c3 llama3-70b", "sym", 128, "f16", [(8192, 10240), (8192, 8192), (8192, 57344), (28672, 8192)],
     [1, 8, 32]),
    ("c4 crossover g128", "asym", 128, "f16", [(4096, 14336)], [1, 2, 4, 8, 16, 32, 64, 128, 256]),
    ("c4 crossover g32", "asym", 32, "f16", [(4096, 14336)], [1, 2, 4, 8, 16, 32, 64, 128, 256]),
    ("c4 crossover nf4", "nf4", 64, "f16", [(4096, 14336)], [1, 2, 4, 8, 16, 32, 64, 128, 256]),
    ("c5 prefill bf16", "asym", 128, "bf16", [(8192, 28672)], [2048]),
]


def sweep(args, torch, w4) -> int:
    """Per (config, shape, M): one GEMM per weight copy, enough copies (>= 600 MB) that the
    weights stream from HBM, replayed from a HIP graph and timed with HIP events. Weights are
    seeded random codes / scales drawn on the device (timing does not depend on values).
    Prints one JSON line per row; at the prefill shape also a dense 16-bit torch.matmul
    (hipBLASLt) and the naive path (dequantize to HBM with the test hook, then matmul)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261203)
    codebook = None
    picks = [c for c in (args.sweep_configs or "").split(",") if c]
    for name, fmt, g, act, shapes, Ms in SWEEP:
        if picks and not any(c in name for c in picks):
            continue
        tdt = torch.float16 if act == "f16" else torch.bfloat16
        nf4 = fmt == "nf4"
        for K, N in shapes:
            wbytes = algo_bytes(0, K, N, g, fmt == "asym", nf4)
            copies = max(2, -(-600_000_000 // wbytes))
            bufs = []
            for _ in range(copies):
                qw = torch.randint(-2**31, 2**31 - 1, (K // 8, N), dtype=torch.int32, device=dev,
                                   generator=gen)
                packed = w4.pack(qw)
                del qw
                sdt = torch.float16 if nf4 else tdt
                sc = (torch.rand((K // g, N), device=dev, generator=gen) * 0.005 + 0.004).to(sdt)
                qz = (torch.randint(-2**31, 2**31 - 1, (K // g, N // 8), dtype=torch.int32,
                                    device=dev, generator=gen) if fmt == "asym" else None)
                bufs.append((packed, sc, qz))
            if nf4 and codebook is None:
                import numpy as np
                vals = np.loadtxt(os.path.join(ROOT, "tests", "golden", "nf4_codebook.txt"))
                codebook = torch.from_numpy(vals.astype(np.float16)).to(dev)
            for M in Ms:
                x = torch.randn((M, K), device=dev, generator=gen).to(tdt)
                y = torch.empty((M, N), device=dev, dtype=tdt)

                def step():
                    for packed, sc, qz in bufs:
                        if nf4:
                            w4.gemm_nf4(x, packed, sc, codebook, g, out=y)
                        else:
                            w4.gemm(x, packed, sc, qz, g, out=y)
                step()
                torch.cuda.synchronize()
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s):
                    step()
                torch.cuda.current_stream().wait_stream(s)
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    step()
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                reps = max(2, min(args.steps, int(2e5 / (copies * max(1.0, M * K * N / 1e9)))))
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    graph.replay()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
                b = algo_bytes(M, K, N, g, fmt == "asym", nf4)
                fl = 2.0 * M * N * K
                t_roof = max(b / (HBM_PEAK_GBS * 1e3), fl / (MFMA_F16_PEAK_TFLOPS * 1e6))
                row = {"config": name, "format": fmt, "group": g, "act": act, "M": M, "K": K, "N": N,
                       "kernel": w4.kernel_name(M, K, N, g), "us": round(us, 2),
                       "GB/s": round(b / us / 1e3, 1), "TFLOP/s": round(fl / us / 1e6, 1),
                       "roof_frac": round(t_roof / us, 3)}
                if name.startswith("c5"):
                    wd = torch.randn((K, N), device=dev, generator=gen).to(tdt)
                    for _ in range(3):
                        torch.matmul(x, wd)
                    torch.cuda.synchronize()
                    e0.record()
                    for _ in range(reps):
                        torch.matmul(x, wd)
                    e1.record()
                    torch.cuda.synchronize()
                    row["dense_matmul_us"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
                    del wd
                    packed, sc, qz = bufs[0]
                    w4.dequant(packed, sc, qz, K, g)  # warm
                    torch.cuda.synchronize()
                    e0.record()
                    for _ in range(reps):
                        torch.matmul(x, w4.dequant(packed, sc, qz, K, g))
                    e1.record()
                    torch.cuda.synchronize()
                    row["naive_dequant_then_matmul_us"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
                print(json.dumps(row), flush=True)
                del graph
            del bufs
            torch.cuda.empty_cache()
    return 0


def _graph_us(torch, fn, steps: int, graph: bool = True) -> float:
    """us per replay of a HIP graph capturing fn (3 warm-up replays, then steps timed); with
    graph=False, fn's launches run eagerly (for counter collection)."""
    fn()
    torch.cuda.synchronize()
    run = fn
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        run = g.replay
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def awq(args, torch, w4) -> int:
    """AWQ-scaled GEMM (w4a16_gemm_awq) against the plain GEMM on the same weights: the 8B
    decode linears at M=1 and 16 (32 distinct weights per shape, so they stream from HBM),
    the crossover shape at M=256 and the prefill shape. One JSON line per shape and M."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261205)
    g = 128
    cases = [(M, K, N, torch.float16, 32) for M in (1, 16)
             for (K, N) in ((4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096))]
    cases += [(256, 4096, 14336, torch.float16, 32), (2048, 8192, 28672, torch.bfloat16, 4)]
    for (M, K, N, dt, copies) in cases:
        ws_ = []
        for _ in range(copies):
            qw = torch.randint(-2**31, 2**31 - 1, (K // 8, N), dtype=torch.int32, device=dev,
                               generator=gen)
            sc = (torch.rand((K // g, N), device=dev, generator=gen) * 0.005 + 0.004).to(dt)
            qz = torch.randint(-2**31, 2**31 - 1, (K // g, N // 8), dtype=torch.int32, device=dev,
                               generator=gen)
            ws_.append((w4.pack(qw), sc, qz))
        x = torch.randn((M, K), device=dev, generator=gen).to(dt)
        s_inv = torch.exp2(torch.rand(K, device=dev, generator=gen) * 4 - 2).to(dt)
        y = torch.empty((M, N), device=dev, dtype=dt)
        ws = torch.empty(max(w4.awq_workspace_bytes(M, K, N, g), 256), dtype=torch.uint8, device=dev)

        def plain():
            for w in ws_:
                w4.gemm(x, *w, g, out=y, workspace=ws)

        def scaled():
            for w in ws_:
                w4.gemm_awq(x, s_inv, *w, g, out=y, workspace=ws)

        res = {k: round(_graph_us(torch, fn, args.steps) / copies, 2)
               for k, fn in (("plain_us", plain), ("awq_us", scaled))}
        res["awq_over_plain"] = round(res["awq_us"] / res["plain_us"], 3)
        print(json.dumps({"config": "awq", "M": M, "K": K, "N": N, "dtype": str(dt).split(".")[-1],
                          "kernel": w4.kernel_name(M, K, N, g),
                          "awq_workspace": w4.awq_workspace_bytes(M, K, N, g), **res}), flush=True)
        del ws_
        torch.cuda.empty_cache()
    return 0


def w4a8(args, torch, w4) -> int:
    """W4A8 (per-token INT8 activations, INT8 MFMA) against W4A16 on the same symmetric codes
    (the W4A16 call gets the per-channel scale repeated in every group of 128): the crossover
    shape over M and the prefill shape. Times include W4A8's activation quantization kernel.
    One JSON line per shape and M."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261206)
    g = 128
    cases = [(M, 4096, 14336, torch.float16, 8) for M in (16, 64, 256, 1024, 4096)]
    cases += [(2048, 8192, 28672, torch.bfloat16, 4)]
    if args.m is not None:
        cases = [c for c in cases if c[0] == args.m]
    for (M, K, N, dt, copies) in cases:
        wts = []
        for _ in range(copies):
            qw = torch.randint(-2**31, 2**31 - 1, (K // 8, N), dtype=torch.int32, device=dev,
                               generator=gen)
            sw = (torch.rand(N, device=dev, generator=gen) * 0.005 + 0.004).to(dt)
            wts.append((w4.pack(qw), sw, sw.repeat(K // g, 1).contiguous()))
        x = torch.randn((M, K), device=dev, generator=gen).to(dt)
        y = torch.empty((M, N), device=dev, dtype=dt)
        ws = torch.empty(max(w4.w4a8_workspace_bytes(M, K, N), w4.workspace_bytes(M, K, N, g), 256),
                         dtype=torch.uint8, device=dev)

        def run16():
            for (pk, _, sg) in wts:
                w4.gemm(x, pk, sg, None, g, out=y, workspace=ws)

        def run8():
            for (pk, sw, _) in wts:
                w4.gemm_w4a8(x, pk, sw, out=y, workspace=ws)

        res = {k: round(_graph_us(torch, fn, args.steps, not args.no_graph) / copies, 2)
               for k, fn in (("w4a16_us", run16), ("w4a8_us", run8))}
        # comparator: a dense INT8 x INT8 -> INT32 GEMM of the same shape (torch._int_mm,
        # hipBLASLt), activations already quantized and the weight 8-bit (twice the bytes)
        try:
            a8 = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=gen)
            b8 = torch.randint(-8, 8, (N, K), dtype=torch.int8, device=dev, generator=gen).t()
            res["dense_int8_us"] = round(_graph_us(torch, lambda: torch._int_mm(a8, b8), args.steps,
                                                   not args.no_graph), 2)
            del a8, b8
        except Exception as e:  # noqa: BLE001 - a comparator only
            res["dense_int8_us"] = None
            res["dense_int8_error"] = str(e)[:120]
        flops = 2.0 * M * K * N
        res["w4a16_tflops"] = round(flops / res["w4a16_us"] / 1e6, 1)
        res["w4a8_tops"] = round(flops / res["w4a8_us"] / 1e6, 1)
        res["w4a8_frac_of_int8_peak"] = round(res["w4a8_tops"] / MFMA_I8_PEAK_TOPS, 3)
        res["speedup"] = round(res["w4a16_us"] / res["w4a8_us"], 3)
        print(json.dumps({"config": "w4a8", "M": M, "K": K, "N": N, "dtype": str(dt).split(".")[-1],
                          "w4a16_kernel": w4.kernel_name(M, K, N, g), **res}), flush=True)
        del wts
        torch.cuda.empty_cache()
    return 0


def mlp(args, torch, w4) -> int:
    """The Llama-3-8B-shaped decode MLP per layer (32 layers of distinct weights, asymmetric
    g128, fp16), replayed from a HIP graph: the fused path is w4a16_gemm_swiglu on the
    (4096, 28672) gate+up weight then the (14336, 4096) down GEMM; the unfused path runs the
    plain gate+up GEMM, SiLU(gate) * up as torch elementwise kernels, then the same down GEMM.
    One JSON line per M with both times per layer."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261204)
    K, N2, Nd = 4096, 28672, 4096
    g = 128
    layers = []
    for _ in range(32):
        def weight(k, n):
            qw = torch.randint(-2**31, 2**31 - 1, (k // 8, n), dtype=torch.int32, device=dev,
                               generator=gen)
            packed = w4.pack(qw)
            sc = (torch.rand((k // g, n), device=dev, generator=gen) * 0.005 + 0.004).half()
            qz = torch.randint(-2**31, 2**31 - 1, (k // g, n // 8), dtype=torch.int32, device=dev,
                               generator=gen)
            return packed, sc, qz
        layers.append((weight(K, N2), weight(N2 // 2, Nd)))
    for M in (1, 4, 16, 64, 256):
        x = torch.randn((M, K), device=dev, generator=gen).half()
        h = torch.empty((M, N2 // 2), device=dev, dtype=torch.float16)
        y2 = torch.empty((M, N2), device=dev, dtype=torch.float16)
        y = torch.empty((M, Nd), device=dev, dtype=torch.float16)
        ws = torch.empty(max(w4.workspace_bytes(M, K, N2, g), w4.workspace_bytes(M, N2 // 2, Nd, g), 256),
                         dtype=torch.uint8, device=dev)

        def fused():
            for (gu, dn) in layers:
                w4.gemm_swiglu(x, *gu, g, out=h, workspace=ws)
                w4.gemm(h, *dn, g, out=y, workspace=ws)

        def unfused():
            for (gu, dn) in layers:
                w4.gemm(x, *gu, g, out=y2, workspace=ws)
                hh = torch.nn.functional.silu(y2[:, :N2 // 2]) * y2[:, N2 // 2:]
                w4.gemm(hh, *dn, g, out=y, workspace=ws)

        res = {}
        for name, fn in (("fused_us", fused), ("unfused_us", unfused)):
            res[name] = round(_graph_us(torch, fn, args.steps) / len(layers), 2)
        res["speedup"] = round(res["unfused_us"] / res["fused_us"], 3)
        print(json.dumps({"config": "mlp llama3-8b (gate+up 4096x28672 with SwiGLU, down 14336x4096)",
                          "M": M, "swiglu_kernel": w4.kernel_name(M, K, N2, g), **res}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3-70b-decode", choices=sorted(WORKLOADS))
    ap.add_argument("--no-m256", action="store_true",
                    help="skip the M=256 crossover point (the metric's TFLOPS half)")
    ap.add_argument("--m256-only", action="store_true",
                    help="only the M=256 crossover point (for counter collection)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-ceiling copy")
    ap.add_argument("--m", type=int, default=None, help="rows of x (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="eager launches instead of a HIP graph")
    ap.add_argument("--mlp", action="store_true",
                    help="time the fused SwiGLU decode MLP against the unfused path, per layer")
    ap.add_argument("--awq", action="store_true",
                    help="time the AWQ-scaled GEMM against the plain GEMM on the same weights")
    ap.add_argument("--w4a8", action="store_true",
                    help="time W4A8 (per-token INT8 activations) against W4A16 on the same codes")
    ap.add_argument("--sweep", action="store_true",
                    help="per-(config, shape, M) timing table of every benchmark config, one JSON "
                         "line per row, instead of the step benchmark")
    ap.add_argument("--sweep-configs", default=None,
                    help="--sweep: only the configs whose name contains one of these "
                         "comma-separated strings (e.g. 'g32,nf4')")
    ap.add_argument("--cpu-baselines", action="store_true",
                    help="only the CPU oracle, timed per benchmark workload and batch size (host "
                         "cores only; one JSON line per (workload, M)), instead of the GPU bench")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (x4), the known-size reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library runs on one GPU "
              "(each GPU of a column or row split would run these kernels on its own shard; "
              "the cross-GPU exchange is not part of it)", file=sys.stderr)
        return 2

    if args.cpu_baselines:
        # every benchmark workload at M=1 and at its own batch size: the oracle's dequant and
        # fp64 matmul timed separately per linear (see cpu_baseline); no GPU is used
        for name, base in WORKLOADS.items():
            for M in sorted({1, base["m"]}):
                spec = dict(base)
                spec["name"] = name
                cb = cpu_baseline(spec, M)
                flops = sum(2.0 * M * K * N for K, N in spec["shapes"]) * spec["layers"]
                print(json.dumps({"workload": name, "M": M, "cpu_baseline": cb,
                                  "GFLOP/s": round(flops / cb["step_s_projected"] / 1e9, 3)}),
                      flush=True)
        return 0

    import torch

    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 4}))
        return 0

    import weight_only_int4_w4a16_amd as w4
    from weight_only_int4_w4a16_amd import synth

    if args.mlp:
        return mlp(args, torch, w4)
    if args.awq:
        return awq(args, torch, w4)
    if args.w4a8:
        return w4a8(args, torch, w4)
    if args.sweep:
        return sweep(args, torch, w4)

    if args.m256_only:
        spec = dict(WORKLOADS[M256_WORKLOAD])
        spec["name"] = M256_WORKLOAD
        r = measure(spec, 256, args, torch, w4, synth)
        print(json.dumps({"workload": M256_WORKLOAD, "M": 256, "roofline": r["roofline"],
                          "ms_per_step": r["ms_per_step"]}), flush=True)
        return 0

    spec = dict(WORKLOADS[args.workload])
    spec["name"] = args.workload
    M = spec["m"] if args.m is None else args.m
    nf4 = spec.get("nf4", False)
    r = measure(spec, M, args, torch, w4, synth)
    mem_bound = r["mem_bound"]
    value, unit = (r["gbs"], "GB/s") if mem_bound else (r["tflops"], "TFLOP/s")
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec["act"], "data": "synthetic (seeded random INT4 codes and scales drawn on "
                                      "the device; activations ~N(0,1))",
        "config": {"workload": args.workload, "M": M, "shapes_KxN": spec["shapes"],
                   "layers": spec["layers"], "group_size": spec["g"],
                   "format": "nf4" if nf4 else ("sym" if spec["sym"] else "asym"),
                   "launches_per_step": r["launches"], "graph": not args.no_graph,
                   "weight_set_GB": round(r["step_bytes"] / 1e9, 3)},
        "pct_of_hbm_peak": round(100 * r["gbs"] / HBM_PEAK_GBS, 2),
        "tflops": round(r["tflops"], 2),
        "wall_s": round(r["wall_s"], 4),
        "roofline": r["roofline"],
        "per_linear": r["per_linear"],
    }
    # the metric's second half: TFLOP/s at M = 256 on the crossover shape, its own roofline
    if not args.no_m256 and args.workload != M256_WORKLOAD:
        del r
        torch.cuda.empty_cache()
        s256 = dict(WORKLOADS[M256_WORKLOAD])
        s256["name"] = M256_WORKLOAD
        r256 = measure(s256, 256, args, torch, w4, synth)
        result["roofline_m256"] = dict(r256["roofline"], workload=M256_WORKLOAD, M=256,
                                       tflops=round(r256["tflops"], 2))
        del r256
        torch.cuda.empty_cache()
    if not args.no_ceiling:
        result["streaming_ceiling"] = streaming_ceiling(torch, w4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, M)
    print(json.dumps(result), flush=True)
    return 0


M256_WORKLOAD = "crossover-4096x14336-g128"


def measure(spec, M, args, torch, w4, synth):
    """Build a workload's buffers, capture one step as a HIP graph, time K replays after W
    warm-up replays, then time each linear alone the same way; the dominant linear (most time
    per launch) gets the roofline object."""
    nf4 = spec.get("nf4", False)
    layers, xs, ys, codebook = build_workload(spec, M, torch, w4, synth)
    step = make_step(spec, layers, xs, ys, codebook, w4)
    launches = [(K, N) for _ in range(spec["layers"]) for (K, N) in spec["shapes"]]
    zeros = not spec["sym"]
    step_bytes = sum(algo_bytes(M, K, N, spec["g"], zeros, nf4) for K, N in launches)
    step_flops = sum(2 * M * N * K for K, N in launches)

    def capture(fn):
        """Warm up eagerly on a side stream, then capture ``fn`` as a HIP graph."""
        fn()
        torch.cuda.synchronize()
        if args.no_graph:
            return fn
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        torch.cuda.synchronize()
        return graph.replay

    def timed(run, reps):
        """HIP events on the stream the replays run on, around ``reps`` back-to-back runs."""
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(reps):
            run()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1)

    run = capture(step)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gpu_ms = timed(run, args.steps)
    wall_s = time.perf_counter() - t0
    ms_per_step = gpu_ms / args.steps
    del run

    # Per linear: the same launches with only that linear of every layer, timed the same way.
    mem_bound = M <= 64
    per_shape = []
    for si, (K, N) in enumerate(spec["shapes"]):
        rr = capture(make_step(spec, layers, xs, ys, codebook, w4, only=si))
        for _ in range(max(1, args.warmup)):
            rr()
        us = timed(rr, args.steps) * 1e3 / (args.steps * spec["layers"])
        del rr
        b = algo_bytes(M, K, N, spec["g"], zeros, nf4)
        per_shape.append({"linear": spec["names"][si], "K": K, "N": N,
                          "kernel": w4.kernel_name(M, K, N, spec["g"]), "us": round(us, 3),
                          "GB/s": round(b / us / 1e3, 1),
                          "TFLOP/s": round(2 * M * N * K / us / 1e6, 2)})
    dom = max(range(len(per_shape)), key=lambda i: per_shape[i]["us"])
    K, N = spec["shapes"][dom]
    kernel = per_shape[dom]["kernel"]
    avg_launch_us = per_shape[dom]["us"]
    bytes_per_launch = algo_bytes(M, K, N, spec["g"], zeros, nf4)
    flops_per_launch = 2 * M * N * K
    if mem_bound:
        achieved = bytes_per_launch / (avg_launch_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = flops_per_launch / (avg_launch_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4)}
    roof["traffic"] = load_traffic(kernel, spec["name"], M)
    roof["kernel"] = kernel
    roof["linear"] = f"{spec['names'][dom]} {K}x{N}"
    roof["avg_launch_us"] = avg_launch_us
    roof["algo_bytes_per_launch"] = int(bytes_per_launch)
    roof["algo_flops_per_launch"] = int(flops_per_launch)
    del layers, xs, ys
    return {"ms_per_step": ms_per_step, "wall_s": wall_s, "mem_bound": mem_bound,
            "gbs": step_bytes / (ms_per_step * 1e-3) / 1e9,
            "tflops": step_flops / (ms_per_step * 1e-3) / 1e12,
            "step_bytes": step_bytes, "launches": len(launches),
            "roofline": roof, "per_linear": per_shape}


def streaming_ceiling(torch, w4, nbytes=4 << 30, reps=10):
    """The device's practical HBM ceiling beside the 8 TB/s spec: the library's streaming-read
    probe (each wave streams a contiguous run with the 16-byte non-temporal loads the packed
    codes use) over 4 GiB, well past the 256 MB last-level cache, and a 4 GiB device-to-device
    copy (bytes read + written); HIP events around ``reps`` launches each."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    out = {}
    for name, fn, moved in (("read_GBps", lambda: w4.read_probe(src, sink), nbytes),
                            ("copy_GBps", lambda: dst.copy_(src), 2 * nbytes)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(moved * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    out["read_frac_of_peak"] = round(out["read_GBps"] / HBM_PEAK_GBS, 4)
    out["bytes"] = nbytes
    del src, dst
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    sys.exit(main())
