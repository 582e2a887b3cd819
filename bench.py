"""Benchmark of the NF4 hot path on one MI355X.

The workload is every linear weight of an L-layer Llama-7B-shaped stack
(L = 32 by default: per layer q, k, v, o 4096x4096, gate and up 11008x4096,
down 4096x11008; bf16 weights N(0, 0.02), distinct per layer; 6.5e9
parameters, 13 GB in bf16, 3.3 GB in NF4).  One step is one pass of every
step of the path over it: quantize-on-load with double quantization of the
whole stack (layer by layer, one grouped call for the seven linears of a
layer; one call per tensor is timed beside it), dequantize of the whole
stack to bf16, the M=1 decode GEMV
(dequant fused) on every weight, and one prefill GEMM, M=2048, N=K=8192, on a
weight quantized once before timing.  Inputs are resident in HBM before
timing; no GEMV weight is re-read before the other weights of its shape have
streamed through, so the 256 MB last-level cache holds none of them.

`value` is the decode GEMV throughput in GB/s of algorithmic bytes (packed
codes + int8 scales + group scales + mean + X + Y) for the three decode shapes
4096x4096, 11008x4096 and 4096x11008 weighted equally: the sum of their
bytes per launch over the sum of their average launch times (each averaged
over all of that shape's weights in the stack).  The stack-weighted decode
rate (7 linears per layer), the GEMM's TFLOP/s, per-kernel timings,
rooflines, and the CPU oracle timed on a bounded sample are reported beside
it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L]
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published (fp16: the same)
METRIC = "NF4 dequant-GEMV HBM GB/s (M=1) + GEMM TFLOP/s (M=2048), % of peak"
DECODE_SHAPES = ((4096, 4096), (11008, 4096), (4096, 11008))
# the linears of one Llama-7B-shaped layer: (name, shape index)
LAYER = (("q", 0), ("k", 0), ("v", 0), ("o", 0), ("gate", 1), ("up", 1), ("down", 2))
PREFILL = (2048, 8192, 8192)
BATCHED = (16, 14336, 4096)     # batched decode: M, N, K
BATCHED_COPIES = 20             # 20 x 29.4 MB of distinct weights (> 512 MB)


def gemv_bytes(M, N, K):
    n = N * K
    nb = n // 64
    ng = -(-nb // 256)
    return n // 2 + nb + 4 * ng + 4 + 2 * M * K + 2 * M * N


def quant_bytes(N, K):
    n = N * K
    nb = n // 64
    ng = -(-nb // 256)
    return 2 * n + n // 2 + nb + 4 * ng + 4


def dequant_bytes(N, K):
    n = N * K
    nb = n // 64
    ng = -(-nb // 256)
    return n // 2 + nb + 4 * ng + 4 + 2 * n


GEMV_SOURCES = ("bnbx_gemv_common.hpp", "bnbx_gemv.hip")   # the M=1 kernel and its launcher


def gemv_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        h.update(open(os.path.join(ROOT, "dequant_gemm_nf4_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def recorded_gemv_traffic():
    """Per-launch HBM bytes of the GEMV from the committed counter runs
    (profiles/gemv_traffic.txt), or None if the kernel source changed since."""
    try:
        rec = dict(line.split(None, 1) for line in open(os.path.join(ROOT, "profiles", "gemv_traffic.txt"))
                   if line.strip() and not line.startswith("#"))
        if gemv_source_hash() != rec["source_sha256"].strip():
            return None
        return int(rec["bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_threads():
    """(CPUs this process may run on, BLAS threads of the all-core mode): the
    affinity set, capped by OMP_NUM_THREADS where the host sets a CPU share."""
    avail = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS")
    return avail, min(avail, int(share)) if share and share.isdigit() else avail


def cpu_baseline(gemv_reps: int = 3):
    """The oracle as it stands, timed on the host in two modes: 1 BLAS thread
    and all cores (NumPy's elementwise work, most of the oracle's time, runs
    on one thread in both).  Each configuration of the GPU workload is timed
    on a bounded sample, in its own unit:

    * decode GEMV M=1 on the three decode shapes (double quant; GB/s of the
      GEMV's algorithmic bytes): fp64 reference GEMV = dequantize + binary64
      matmul, ``gemv_reps`` times per shape; the headline ``value`` is its
      all-core rate over the three shapes, the same weighting as the GPU
      ``value``;
    * batched decode M=16 on 14336x4096 (GB/s), ``gemv_reps`` times;
    * prefill M=2048, N=K=8192 (TFLOP/s), the whole product;
    * quantize with double quant (GB/s of bf16 input read): layers 0 and 31
      of the stack (7 linears each), whose rate stands for the 32-layer stack
      (x16 for its time).

    Inputs come from ``synth`` (host draws of the same shapes and
    distributions as the GPU workload)."""
    import numpy as np
    import oracle
    import synth
    from threadpoolctl import threadpool_limits

    avail, allc = cpu_threads()
    gemv_in = []
    for s in range(len(DECODE_SHAPES)):
        w, x = synth.decode(s)
        gemv_in.append((x, oracle.quantize(w, True), DECODE_SHAPES[s]))
    wb, xb = synth.batched()
    N16, K16 = wb.shape
    st16 = oracle.quantize(wb, True)
    del wb
    wp, xp = synth.prefill()
    Np, Kp = wp.shape
    stp = oracle.quantize(wp, True)
    del wp
    Mp = xp.shape[0]
    qweights = [w for l in (0, 31) for w in synth.bulk_layer(l)]

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    configs = []
    t_total = time.perf_counter()
    for mode, threads in (("1-thread", 1), ("all-core", allc)):
        with threadpool_limits(threads):
            secs = [sum(timed(lambda: oracle.dequant_matmul_ref(x, st["packed"], st, N, K))
                        for _ in range(gemv_reps))
                    for x, st, (N, K) in gemv_in]
            byts = [gemv_reps * gemv_bytes(1, N, K) for _, _, (N, K) in gemv_in]
            configs.append({"config": "decode GEMV M=1, 4096x4096 + 11008x4096 + 4096x11008",
                            "mode": mode, "threads": threads,
                            "value": sum(byts) / sum(secs) / 1e9, "unit": "GB/s",
                            "seconds": sum(secs),
                            "by_shape_s": {f"{N}x{K}": round(t, 3)
                                           for t, (_, _, (N, K)) in zip(secs, gemv_in)},
                            "sample": f"{gemv_reps} reference GEMVs per shape"})
            t = sum(timed(lambda: oracle.dequant_matmul_ref(xb, st16["packed"], st16, N16, K16))
                    for _ in range(gemv_reps))
            configs.append({"config": f"batched decode M=16, {N16}x{K16}", "mode": mode,
                            "threads": threads,
                            "value": gemv_reps * gemv_bytes(16, N16, K16) / t / 1e9,
                            "unit": "GB/s", "seconds": t,
                            "sample": f"{gemv_reps} reference GEMVs"})
            t = timed(lambda: oracle.dequant_matmul_ref(xp, stp["packed"], stp, Np, Kp))
            configs.append({"config": f"prefill GEMM M=2048, N=K={Kp}", "mode": mode,
                            "threads": threads, "value": 2.0 * Mp * Np * Kp / t / 1e12,
                            "unit": "TFLOP/s", "seconds": t,
                            "sample": "the whole product, all 2048 rows"})
            t = sum(timed(lambda w=w: oracle.quantize(w, True)) for w in qweights)
            nin = sum(2 * w.size for w in qweights)
            configs.append({"config": "quantize with double quant", "mode": mode,
                            "threads": threads, "value": nin / t / 1e9,
                            "unit": "GB/s (bf16 input read)", "seconds": t,
                            "sample": ("layers 0 and 31 of the 32-layer stack (14 linears); "
                                       f"the stack would take x16 = {16 * t:.0f} s")})
    for c in configs:
        c["value"] = round(c["value"], 6)
        c["seconds"] = round(c["seconds"], 3)
    head = configs[len(configs) // 2]   # decode GEMV, all-core
    return {
        "value": head["value"],
        "unit": "GB/s",
        "cores": allc,
        "affinity_cpus": avail,
        "kind": "oracle",
        "sample": (f"fp64 reference GEMV (oracle dequantize + binary64 matmul) {gemv_reps} times "
                   f"per decode shape, double quant, M=1, {allc} BLAS threads; every "
                   f"configuration in "
                   f"both modes in 'configs' ({time.perf_counter() - t_total:.0f} s of CPU work "
                   f"in all)"),
        "configs": configs,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-only", action="store_true",
                    help="only the CPU baseline (no GPU work); prints its JSON object")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the FP4 / FP16 measurements (profiling runs)")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="run a 256 MiB plain copy first (counter scaling reference)")
    args = ap.parse_args()
    if args.cpu_only:
        print(json.dumps(cpu_baseline()))
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    from dequant_gemm_nf4_amd import tensors as T

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    L = args.layers

    # ---- inputs resident in HBM (device-side seeded draws) ----
    gen = torch.Generator(device=dev)
    weights, wshape = [], []          # stack order: layer by layer, LAYER order
    for l in range(L):
        for li, (name, si) in enumerate(LAYER):
            N, K = DECODE_SHAPES[si]
            gen.manual_seed(5000 + 10 * l + li)
            w = (torch.randn(N, K, generator=gen, device=dev, dtype=torch.float32) * 0.02)
            weights.append(w.to(torch.bfloat16))
            wshape.append(si)
            del w
    xs = []
    for s, (N, K) in enumerate(DECODE_SHAPES):
        gen.manual_seed(6000 + s)
        xs.append(torch.randn(1, K, generator=gen, device=dev).to(torch.bfloat16))
    qs = [T.empty_quantized(w.shape, True, dev) for w in weights]
    maxn = max(N * K for N, K in DECODE_SHAPES)
    ws = T.workspace_for(maxn, True, dev)
    per_layer = len(LAYER)
    # quantize-on-load layer by layer: one grouped call per layer
    wsg = T.grouped_workspace_for([w.numel() for w in weights[:per_layer]], True, dev)
    deq = torch.empty(maxn, dtype=torch.bfloat16, device=dev)
    ys = [torch.empty(1, N, dtype=torch.bfloat16, device=dev) for N, K in DECODE_SHAPES]
    by_shape = [[i for i, si in enumerate(wshape) if si == s] for s in range(len(DECODE_SHAPES))]

    Mp, Np, Kp = PREFILL
    gen.manual_seed(7000)
    wp = (torch.randn(Np, Kp, generator=gen, device=dev) * 0.015).to(torch.bfloat16)
    gen.manual_seed(7001)
    xp = torch.randn(Mp, Kp, generator=gen, device=dev)
    gen.manual_seed(7002)
    cols = torch.randperm(Kp, generator=gen, device=dev)[:4]
    xp[:, cols] *= 50.0
    xp = xp.to(torch.bfloat16)
    qp = T.quantize(wp, True)
    del wp
    yp = torch.empty(Mp, Np, dtype=torch.bfloat16, device=dev)

    # batched decode, M=16 on 14336x4096 (weights N(0,0.02) with 0.1% of
    # entries x20): distinct weights over more than 512 MB, so each launch
    # streams its weight from HBM
    Mb, Nb, Kb = BATCHED
    qb = []
    for i in range(BATCHED_COPIES):
        gen.manual_seed(8000 + i)
        w = torch.randn(Nb * Kb, generator=gen, device=dev, dtype=torch.float32) * 0.02
        gen.manual_seed(8200 + i)
        idx = torch.randperm(Nb * Kb, generator=gen, device=dev)[: Nb * Kb // 1000]
        w[idx] *= 20.0
        qb.append(T.quantize(w.view(Nb, Kb).to(torch.bfloat16), True))
        del w, idx
    gen.manual_seed(8100)
    xb = torch.randn(Mb, Kb, generator=gen, device=dev).to(torch.bfloat16)
    yb = torch.empty(Mb, Nb, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # Every stage is captured once into a HIP graph and replayed each step, so
    # host launch overhead stays out of the timings; the decode GEMVs get one
    # graph per shape (every weight of that shape in the stack, in stack
    # order) bracketed by events, so the average launch time of each shape is
    # the graph time over its launches (kernel time plus the GPU's
    # back-to-back dispatch gap).
    def stage_quantize():
        for l in range(L):
            sl = slice(l * per_layer, (l + 1) * per_layer)
            T.quantize_grouped(weights[sl], True, outs=qs[sl], workspace=wsg)

    def stage_dequantize():
        for q in qs:
            T.dequantize(q, out=deq[: q.n].view(q.shape))

    def stage_gemv(s):
        def run():
            for i in by_shape[s]:
                T.gemv(xs[s], qs[i], out=ys[s])
        return run

    def stage_gemm():
        T.gemm(xp, qp, out=yp)

    def stage_batched():
        for q in qb:
            T.gemv(xb, q, out=yb)

    stages = [stage_quantize, stage_dequantize] + \
        [stage_gemv(s) for s in range(len(DECODE_SHAPES))] + [stage_gemm, stage_batched]
    for fn in stages:        # eager warm-up (also loads every kernel)
        fn()
    torch.cuda.synchronize()
    graphs = []
    cap = torch.cuda.Stream()
    for fn in stages:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            fn()
        graphs.append(g)
    torch.cuda.synchronize()

    def step():
        marks = [ev() for _ in range(2 * len(graphs))]
        for k, g in enumerate(graphs):
            marks[2 * k].record(stream)
            g.replay()
            marks[2 * k + 1].record(stream)
        return marks

    if args.pmc_calibration:
        # a plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE
        # counters of the kernels (256 MiB read + 256 MiB written per copy)
        src = torch.empty(128 * 1024 * 1024, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    all_marks = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        all_marks.append(step())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def stage_ms(k):
        return sum(m[2 * k].elapsed_time(m[2 * k + 1]) for m in all_marks)

    # Achievable ceiling, outside the timed steps: a plain streaming read of
    # each weight's packed bytes and block codes (what the GEMV streams),
    # launched back to back over the same weights as the GEMV stage.
    import dequant_gemm_nf4_amd as bnbx
    sink = torch.zeros(bnbx.BNBX_PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    read_bytes = [N * K // 2 + N * K // 64 for N, K in DECODE_SHAPES]

    def stage_read(s):
        def run():
            for i in by_shape[s]:
                bnbx.bnbx_probe_stream_read(qs[i].packed, qs[i].packed.numel(), qs[i].absmax,
                                            qs[i].absmax.numel(), sink)
        return run
    read_us = []
    for s in range(len(DECODE_SHAPES)):
        stage_read(s)()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            stage_read(s)()
        g.replay()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(args.steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        read_us.append(e0.elapsed_time(e1) * 1e3 / (args.steps * len(by_shape[s])))
        del g
    read_gbs = (sum(read_bytes) / len(read_bytes)) / (sum(read_us) / len(read_us) * 1e-6) / 1e9

    # The other 4-bit quant type and compute dtype (FP4 levels; FP16 compute),
    # timed after the steps like the read ceiling: the stack quantized again
    # as FP4, then per (quant type, dtype) the dequantize of the stack, the
    # decode GEMVs per shape and the prefill GEMM, each replayed in a graph.
    def timed_ms(fn, reps):
        fn()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            fn()
        g.replay()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) / reps

    def measure_variants():
        reps = max(2, args.steps)
        xs16 = []
        for s, (N, K) in enumerate(DECODE_SHAPES):
            gen.manual_seed(6000 + s)
            xs16.append(torch.randn(1, K, generator=gen, device=dev).to(torch.float16))
        gen.manual_seed(7000)
        wp = (torch.randn(Np, Kp, generator=gen, device=dev) * 0.015).to(torch.bfloat16)
        gen.manual_seed(7001)
        xp16 = torch.randn(Mp, Kp, generator=gen, device=dev)
        gen.manual_seed(7002)
        xp16[:, torch.randperm(Kp, generator=gen, device=dev)[:4]] *= 50.0
        xp16 = xp16.to(torch.float16)
        qp_by = {"nf4": qp, "fp4": T.quantize(wp, True, quant_type="fp4")}
        del wp
        qs_fp4 = [T.empty_quantized(w.shape, True, dev, "fp4") for w in weights]
        q_fp4_ms = timed_ms(lambda: [
            T.quantize_grouped(weights[l * per_layer:(l + 1) * per_layer], True,
                               outs=qs_fp4[l * per_layer:(l + 1) * per_layer], workspace=wsg)
            for l in range(L)], reps)
        stack_by = {"nf4": qs, "fp4": qs_fp4}
        deq16 = torch.empty(maxn, dtype=torch.float16, device=dev)
        ys16 = [torch.empty(1, N, dtype=torch.float16, device=dev) for N, K in DECODE_SHAPES]
        yp16 = torch.empty(Mp, Np, dtype=torch.float16, device=dev)
        variants = {}
        for qt, dt in (("fp4", "bf16"), ("nf4", "f16"), ("fp4", "f16")):
            tdt = torch.float16 if dt == "f16" else torch.bfloat16
            sv = [dataclasses.replace(q, dtype=tdt) for q in stack_by[qt]]
            qpv = dataclasses.replace(qp_by[qt], dtype=tdt)
            dbuf = deq16 if dt == "f16" else deq
            xv, yv = (xs16, ys16) if dt == "f16" else (xs, ys)
            xpv, ypv = (xp16, yp16) if dt == "f16" else (xp, yp)
            d_ms = timed_ms(lambda: [T.dequantize(q, out=dbuf[: q.n].view(q.shape)) for q in sv],
                            reps)
            v_us = []
            for s in range(len(DECODE_SHAPES)):
                ms = timed_ms(lambda: [T.gemv(xv[s], sv[i], out=yv[s]) for i in by_shape[s]],
                              reps)
                v_us.append(ms * 1e3 / len(by_shape[s]))
            m_ms = timed_ms(lambda: T.gemm(xpv, qpv, out=ypv), reps)
            gbs = (sum(gemv_bytes(1, N, K) for N, K in DECODE_SHAPES) / len(DECODE_SHAPES)) / \
                (sum(v_us) / len(v_us) * 1e-6) / 1e9
            tf = 2.0 * Mp * Np * Kp / (m_ms * 1e-3) / 1e12
            entry = {
                "dequantize_gbs": round(sum(dequant_bytes(*DECODE_SHAPES[si]) for si in wshape)
                                        / (d_ms * 1e-3) / 1e9, 1),
                "gemv_gbs": round(gbs, 1),
                "gemv_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "gemv_launch_us_by_shape": {f"{N}x{K}": round(u, 3)
                                            for (N, K), u in zip(DECODE_SHAPES, v_us)},
                "gemm_tflops": round(tf, 1),
                "gemm_frac": round(tf / BF16_PEAK_TFLOPS, 4),
            }
            if qt == "fp4" and dt == "bf16":
                entry["quantize_input_read_gbs"] = round(
                    sum(2 * DECODE_SHAPES[si][0] * DECODE_SHAPES[si][1] for si in wshape)
                    / (q_fp4_ms * 1e-3) / 1e9, 1)
            variants[f"{qt}_{dt}"] = entry
        return variants

    variants = None if args.no_variants else measure_variants()

    # Quantize with one bnbx_quantize_nf4 call per tensor (two launches each)
    # instead of one grouped call per layer, over the same stack, timed after
    # the steps like the above.
    q1_ms = timed_ms(lambda: [T.quantize(w, True, out=qs[i], workspace=ws)
                              for i, w in enumerate(weights)], max(2, args.steps))

    # Grouped decode GEMV (bnbx_gemv_nf4_grouped), M=1: per layer of the
    # stack, q, k, v in one call and gate, up in another (they share X), in
    # one graph over all layers, beside the same weights launched one by one.
    xg = xs[0]                                          # [1, 4096]
    yq = [torch.empty(1, 4096, dtype=torch.bfloat16, device=dev) for _ in range(3)]
    yg = [torch.empty(1, 11008, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    qkv = [[qs[l * per_layer + i] for i in range(3)] for l in range(L)]
    gu = [[qs[l * per_layer + i] for i in (4, 5)] for l in range(L)]
    reps_g = max(2, args.steps)
    grouped = {}
    for name, groups, outs, shape in (("qkv", qkv, yq, (4096, 4096)),
                                      ("gate_up", gu, yg, (11008, 4096))):
        nbytes = sum(gemv_bytes(1, *shape) for _ in groups[0])
        g_ms = timed_ms(lambda: [T.gemv_grouped(xg, grp, outs=outs) for grp in groups],
                        reps_g) / len(groups)
        s_ms = timed_ms(lambda: [T.gemv(xg, q, out=o) for grp in groups
                                 for q, o in zip(grp, outs)], reps_g) / len(groups)
        grouped[name] = {"weights": f"{len(groups[0])} x {shape[0]}x{shape[1]}",
                         "call_us": round(g_ms * 1e3, 3),
                         "gbs": round(nbytes / (g_ms * 1e-3) / 1e9, 1),
                         "hbm_frac": round(nbytes / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "separate_launches_us": round(s_ms * 1e3, 3),
                         "separate_gbs": round(nbytes / (s_ms * 1e-3) / 1e9, 1)}
    del yq, yg

    # Batched decode on the down projection, M=16 on 4096x11008 (K = 11008:
    # three 4096-k chunks per wave), one launch per weight, over 24 distinct
    # weights (540 MB), timed after the steps like the above.
    Nd, Kd = 4096, 11008
    qdown = []
    for i in range(24):
        gen.manual_seed(8300 + i)
        w = (torch.randn(Nd, Kd, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        qdown.append(T.quantize(w, True))
        del w
    gen.manual_seed(8400)
    xdown = torch.randn(Mb, Kd, generator=gen, device=dev).to(torch.bfloat16)
    ydown = torch.empty(Mb, Nd, dtype=torch.bfloat16, device=dev)
    down_us = timed_ms(lambda: [T.gemv(xdown, q, out=ydown) for q in qdown],
                       max(2, args.steps)) * 1e3 / len(qdown)
    del qdown, xdown, ydown

    # Input gradient of the prefill layer, dX = dY . W_hat (M=2048, N=K=8192,
    # the same NF4 double-quant weight), timed after the steps like the above.
    gen.manual_seed(7003)
    dyp = torch.randn(Mp, Np, generator=gen, device=dev).to(torch.bfloat16)
    dxp = torch.empty(Mp, Kp, dtype=torch.bfloat16, device=dev)
    dx_ms = timed_ms(lambda: T.gemm_dx(dyp, qp, out=dxp), max(2, args.steps))
    dx_tflops = 2.0 * Mp * Np * Kp / (dx_ms * 1e-3) / 1e12
    del dyp, dxp

    # Prefill GEMMs of one Llama-7B layer at M=2048 (q, k, v, o 4096x4096;
    # gate, up 11008x4096; down 4096x11008), timed after the steps like the
    # above: each shape with the workspace bnbx_gemm_nf4_workspace_bytes asks
    # for (split K where the 256x256 tiles fill at most half of the CUs) and
    # without one (whole tiles).
    import dequant_gemm_nf4_amd as bnbx_lib
    llama_prefill = {}
    layer_us = {"planned": 0.0, "whole_tiles": 0.0}
    for name, (Nl, Kl), count in (("qkvo", (4096, 4096), 4), ("gate_up", (11008, 4096), 2),
                                  ("down", (4096, 11008), 1)):
        gen.manual_seed(7200 + Nl + Kl)
        wl = (torch.randn(Nl, Kl, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        ql = T.quantize(wl, True)
        del wl
        xl = torch.randn(Mp, Kl, generator=gen, device=dev).to(torch.bfloat16)
        yl = torch.empty(Mp, Nl, dtype=torch.bfloat16, device=dev)
        need = bnbx_lib.bnbx_gemm_nf4_workspace_bytes(Mp, Nl, Kl)
        wsl = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        reps_l = max(2, args.steps)
        ms_plan = timed_ms(lambda: bnbx_lib.bnbx_gemm_nf4(
            xl, Kl, ql.packed, ql.state, Mp, Nl, Kl, yl, Nl, wsl if need else None, need), reps_l)
        ms_whole = timed_ms(lambda: bnbx_lib.bnbx_gemm_nf4(
            xl, Kl, ql.packed, ql.state, Mp, Nl, Kl, yl, Nl, None, 0), reps_l)
        fl = 2.0 * Mp * Nl * Kl
        llama_prefill[name] = {"shape": f"{Mp}x{Nl}x{Kl}", "per_layer": count,
                               "split_workspace_bytes": need,
                               "us": round(ms_plan * 1e3, 1),
                               "tflops": round(fl / (ms_plan * 1e-3) / 1e12, 1),
                               "whole_tiles_us": round(ms_whole * 1e3, 1),
                               "whole_tiles_tflops": round(fl / (ms_whole * 1e-3) / 1e12, 1)}
        layer_us["planned"] += count * ms_plan * 1e3
        layer_us["whole_tiles"] += count * ms_whole * 1e3
        del ql, xl, yl, wsl
    layer_flops = sum(2.0 * Mp * n * k * c for (n, k), c in
                      (((4096, 4096), 4), ((11008, 4096), 2), ((4096, 11008), 1)))
    llama_prefill["layer"] = {
        "us": round(layer_us["planned"], 1),
        "tflops": round(layer_flops / (layer_us["planned"] * 1e-6) / 1e12, 1),
        "whole_tiles_us": round(layer_us["whole_tiles"], 1)}

    # The GEMM with a LoRA term fused in (ranks 16 and 64), same
    # weight and X, and the plain GEMM beside it: one graph each, timed in
    # interleaved rounds (the clock under load drifts between consecutive
    # measurements by more than the difference being measured), the median
    # round of each reported.
    lora_in = {}
    for r in (16, 64):
        gen.manual_seed(7100 + r)
        lora_in[r] = ((torch.randn(Mp, r, generator=gen, device=dev) * 0.5).to(torch.bfloat16),
                      (torch.randn(Np, r, generator=gen, device=dev) * 0.05).to(torch.bfloat16),
                      (torch.randn(r, Kp, generator=gen, device=dev) * 0.02).to(torch.bfloat16))
    fns = {"plain": lambda: T.gemm(xp, qp, out=yp)}
    for r, (xa, lb, la) in lora_in.items():
        fns[f"r{r}"] = (lambda xa=xa, lb=lb: T.gemm_lora(xp, qp, xa, lb, out=yp))
        # the adapter's down-projection in the library too: XA = s X A^T, then
        # the GEMM with the low-rank term
        fns[f"r{r}_down"] = (lambda xa=xa, la=la: T.lora_down(xp, la, 2.0, out=xa))
        fns[f"r{r}_full"] = (lambda xa=xa, lb=lb, la=la: (T.lora_down(xp, la, 2.0, out=xa),
                                                          T.gemm_lora(xp, qp, xa, lb, out=yp)))
    def interleaved_ms(fns):
        # one graph per function, replayed in 5 interleaved rounds; the
        # median round of each, in ms per replay
        graphs = {}
        for name, fn in fns.items():
            fn()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                fn()
            graphs[name] = g
        rounds = {name: [] for name in graphs}
        reps = max(2, args.steps)
        for _ in range(5):
            for name, g in graphs.items():
                g.replay()
                e0, e1 = ev(), ev()
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                rounds[name].append(e0.elapsed_time(e1) / reps)
        del graphs
        return {name: sorted(v)[len(v) // 2] for name, v in rounds.items()}

    med = interleaved_ms(fns)
    plain_ms = med["plain"]
    lora = {"plain_ms": round(plain_ms, 4), "timing": "median of 5 interleaved rounds"}
    for r in (16, 64):
        ms = med[f"r{r}"]
        lora[f"r{r}"] = {"ms": round(ms, 4),
                         "tflops": round(2.0 * Mp * Np * (Kp + r) / (ms * 1e-3) / 1e12, 1),
                         "over_plain": round(ms / plain_ms, 4),
                         "down_ms": round(med[f"r{r}_down"], 4),
                         "down_gbs": round(2.0 * (Mp * Kp + r * Kp + Mp * r) /
                                           (med[f"r{r}_down"] * 1e-3) / 1e9, 1),
                         "with_down_ms": round(med[f"r{r}_full"], 4),
                         "with_down_over_plain": round(med[f"r{r}_full"] / plain_ms, 4)}
    del lora_in

    # The LoRA term at decode sizes (its GEMV forms): M=1 over the stack's
    # 4096x4096 weights and M=16 over the batched decode's 14336x4096
    # weights, so each launch streams its weight from HBM; XA given, one
    # adapter B per run; the plain GEMV over the same weights beside it.
    dec_fns, dec_runs = {}, {}
    for tag, (xd, qd, yd) in {"m1": (xs[0], [qs[i] for i in by_shape[0]], ys[0]),
                              "m16": (xb, qb, yb)}.items():
        Md, Nw, Kw = xd.shape[0], qd[0].shape[0], qd[0].shape[1]
        dec_runs[tag] = (f"{Md}x{Nw}x{Kw}", len(qd))
        dec_fns[f"{tag}_plain"] = (lambda xd=xd, qd=qd, yd=yd:
                                   [T.gemv(xd, q, out=yd) for q in qd])
        for r in (16, 64):
            gen.manual_seed(7300 + r + Md)
            xa = (torch.randn(Md, r, generator=gen, device=dev) * 0.5).to(torch.bfloat16)
            lb = (torch.randn(Nw, r, generator=gen, device=dev) * 0.05).to(torch.bfloat16)
            dec_fns[f"{tag}_r{r}"] = (lambda xd=xd, qd=qd, yd=yd, xa=xa, lb=lb:
                                      [T.gemm_lora(xd, q, xa, lb, out=yd) for q in qd])
    dmed = interleaved_ms(dec_fns)
    gemv_lora = {"timing": "median of 5 interleaved rounds, per launch"}
    for tag, (shape, n) in dec_runs.items():
        e = {"shape": shape, "weights": n,
             "plain_us": round(dmed[f"{tag}_plain"] * 1e3 / n, 3)}
        for r in (16, 64):
            e[f"r{r}_us"] = round(dmed[f"{tag}_r{r}"] * 1e3 / n, 3)
            e[f"r{r}_over_plain"] = round(dmed[f"{tag}_r{r}"] / dmed[f"{tag}_plain"], 4)
        gemv_lora[tag] = e
    del dec_fns

    t_q = stage_ms(0) / 1e3
    t_d = stage_ms(1) / 1e3
    t_shape = [stage_ms(2 + s) / 1e3 for s in range(len(DECODE_SHAPES))]
    t_v = sum(t_shape)
    t_m = stage_ms(2 + len(DECODE_SHAPES)) / 1e3
    K_ = args.steps
    # average launch time and bytes per launch of each decode shape
    us_shape = [t / (K_ * len(by_shape[s])) * 1e6 for s, t in enumerate(t_shape)]
    b_shape = [gemv_bytes(1, N, K) for N, K in DECODE_SHAPES]
    shape_us = {f"{N}x{K}": round(u, 3) for (N, K), u in zip(DECODE_SHAPES, us_shape)}
    # headline: the three decode shapes weighted equally
    avg_gemv_bytes = sum(b_shape) / len(b_shape)
    avg_gemv_us = sum(us_shape) / len(us_shape)
    gemv_gbs = avg_gemv_bytes / (avg_gemv_us * 1e-6) / 1e9
    # the whole stack (7 linears per layer)
    gb_stack = K_ * sum(b_shape[si] for si in wshape)
    stack_gbs = gb_stack / t_v / 1e9
    gb_q = K_ * sum(quant_bytes(*DECODE_SHAPES[si]) for si in wshape)
    gb_d = K_ * sum(dequant_bytes(*DECODE_SHAPES[si]) for si in wshape)
    gb_in = K_ * sum(2 * DECODE_SHAPES[si][0] * DECODE_SHAPES[si][1] for si in wshape)
    gemm_tflops = K_ * 2.0 * Mp * Np * Kp / t_m / 1e12
    t_b = stage_ms(3 + len(DECODE_SHAPES)) / 1e3
    us_b = t_b / (K_ * BATCHED_COPIES) * 1e6
    b_b = gemv_bytes(Mb, Nb, Kb)

    out = {
        "metric": METRIC,
        "value": round(gemv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (NF4 storage, fp32 accumulate)",
        "data": "synthetic (seeded device draws, N(0,0.02) weights, N(0,1) activations)",
        "config": {
            "workload": "decode GEMV M=1 on Llama-7B-shaped linears 4096x4096, 11008x4096, "
                        "4096x11008 (NF4 blocksize 64, double quant), every weight of a "
                        f"{L}-layer stack (q,k,v,o,gate,up,down per layer, distinct weights, "
                        "streamed from HBM); plus quantize (one grouped call per layer) and "
                        "dequantize of the stack and a "
                        "prefill GEMM M=2048 N=K=8192; batched decode M=16 on 14336x4096 "
                        "(0.1% of weights x20) in kernels.gemv_m16",
            "layers": L,
            "gemm": {"M": Mp, "N": Np, "K": Kp},
        },
        "roofline": {
            "kernel": "gemv_kernel",
            "bound": "hbm",
            "achieved": round(avg_gemv_bytes / (avg_gemv_us * 1e-6) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(avg_gemv_bytes / (avg_gemv_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": recorded_gemv_traffic(),
        },
        "gemm": {
            "tflops": round(gemm_tflops, 1),
            "peak": BF16_PEAK_TFLOPS,
            "frac": round(gemm_tflops / BF16_PEAK_TFLOPS, 4),
            "ms": round(t_m / K_ * 1e3, 4),
        },
        "kernels": {
            "quantize_gbs": round(gb_q / t_q / 1e9, 1),
            "quantize_input_read_gbs": round(gb_in / t_q / 1e9, 1),
            "quantize_per_tensor": {
                "what": "one bnbx_quantize_nf4 call per tensor instead of one grouped call "
                        "per layer",
                "gbs": round(gb_q / K_ / (q1_ms * 1e-3) / 1e9, 1),
                "input_read_gbs": round(gb_in / K_ / (q1_ms * 1e-3) / 1e9, 1),
                "ms": round(q1_ms, 3)},
            "dequantize_gbs": round(gb_d / t_d / 1e9, 1),
            "gemv_gbs": round(gemv_gbs, 1),
            "gemv_stack_gbs": round(stack_gbs, 1),
            "gemv_avg_launch_us": round(avg_gemv_us, 3),
            "gemv_launch_us_by_shape": shape_us,
            "gemv_m16": {"shape": f"{Mb}x{Nb}x{Kb}", "launch_us": round(us_b, 3),
                         "gbs": round(b_b / (us_b * 1e-6) / 1e9, 1),
                         "hbm_frac": round(b_b / (us_b * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "tflops": round(2.0 * Mb * Nb * Kb / (us_b * 1e-6) / 1e12, 2)},
            "gemv_grouped": grouped,
            "gemv_m16_down": {"shape": f"{Mb}x{Nd}x{Kd}", "launches_per_call": 1,
                              "launch_us": round(down_us, 3),
                              "gbs": round(gemv_bytes(Mb, Nd, Kd) / (down_us * 1e-6) / 1e9, 1),
                              "hbm_frac": round(gemv_bytes(Mb, Nd, Kd) / (down_us * 1e-6) / 1e9
                                                / HBM_PEAK_GBS, 4)},
            "read_ceiling": {
                "what": "plain streaming read of each weight's packed bytes and block codes, "
                        "back to back over the same weights (bnbx_probe_stream_read)",
                "bytes_by_shape": {f"{N}x{K}": b for (N, K), b in zip(DECODE_SHAPES, read_bytes)},
                "launch_us_by_shape": {f"{N}x{K}": round(u, 3)
                                       for (N, K), u in zip(DECODE_SHAPES, read_us)},
                "gbs": round(read_gbs, 1),
                "hbm_frac": round(read_gbs / HBM_PEAK_GBS, 4),
                "gemv_over_ceiling": round(gemv_gbs / read_gbs, 4),
            },
            "variants": variants,
            "gemm_lora": lora,
            "gemv_lora": gemv_lora,
            "gemm_llama7b_prefill": llama_prefill,
            "gemm_dx": {"what": "dX = dY . W_hat, M=2048 N=K=8192, NF4 double quant, bf16",
                        "ms": round(dx_ms, 4), "tflops": round(dx_tflops, 1),
                        "frac": round(dx_tflops / BF16_PEAK_TFLOPS, 4)},
            "stage_ms_per_step": {"quantize": round(t_q / K_ * 1e3, 3),
                                  "dequantize": round(t_d / K_ * 1e3, 3),
                                  "gemv": round(t_v / K_ * 1e3, 3),
                                  "gemm": round(t_m / K_ * 1e3, 3),
                                  "gemv_m16": round(t_b / K_ * 1e3, 3)},
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
