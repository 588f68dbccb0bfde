#!/usr/bin/env python3
"""Benchmark of the MatMulNBits hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  * decode: Y[1, 8192] = X[1, 2048] . deq(W)^T + (X.A).B, INT4 block-32 weights with the
    default zero point and a rank-32 F16 LoRA fused in the same launch (in-pass T);
  * prefill: Y[1024, 4096] = X[1024, 4096] . deq(W)^T + (X.A).B, INT4 block-32 with explicit
    zero points, rank-32 F16 LoRA (T projection launch + MFMA GEMM with the T.B epilogue).
Inputs are resident in HBM before timing.  Decode rotates over enough copies of its
weights and adapter (default >= 1 GiB, four times the 256 MB Infinity Cache) that every
call streams from HBM; the prefill GEMM is MFMA-bound and uses one copy.

The timed region replays two captured HIP graphs on one stream: K decode calls, then K
prefill calls; HIP events bracket each graph.  `value` is the decode GEMV's effective HBM
bandwidth (algorithmic bytes / mean decode call time, GB/s); the prefill TFLOP/s rides
along in `prefill`.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
FP16_PEAK_TFLOPS = 2516.6       # MI355X dense FP16 MFMA (256 CUs x 2.4 GHz x 4096 flop/clk)
METRIC = "decode GEMV effective HBM GB/s (M=1) + prefill TFLOP/s (M=1024), % roofline"


def algorithmic_bytes(M, N, K, bits, has_zp, rank):
    """Bytes the method must move once: codes + scales + zero points + X + Y + adapter."""
    b = N * K * bits // 8 + (N * K // 32) * 2 + (N * K // 32 * bits // 8 if has_zp else 0)
    b += M * K * 2 + M * N * 2
    if rank:
        b += K * rank * 2 + rank * N * 2
    return b


def algorithmic_flops(M, N, K, rank):
    return 2 * M * N * K + (2 * M * K * rank + 2 * M * rank * N if rank else 0)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cold-mib", type=int, default=1024, help="bytes of rotated decode copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle baseline")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the warm / two-launch / empty-adapter context runs (counter collection)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 10 device-to-device copies of MIB MiB (calibrates FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="only print per-kernel means of the rocprofv3 csv files under DIR (no GPU use)")
    return ap.parse_args()


def summarize(root):
    """Per-kernel means of rocprofv3 csv output under `root`: counter values per dispatch
    (*_counter_collection.csv) or durations (*_kernel_trace.csv)."""
    import csv
    import glob
    import re
    rows = {}
    for path in sorted(glob.glob(os.path.join(root, "**", "*.csv"), recursive=True)):
        kind = "counter" if path.endswith("_counter_collection.csv") else (
            "trace" if path.endswith("_kernel_trace.csv") else None)
        if kind is None:
            continue
        for r in csv.DictReader(open(path)):
            name = re.sub(r"\(anonymous namespace\)::|mnb::", "", r["Kernel_Name"])
            name = re.sub(r"\(.*", "", name)
            if kind == "counter":
                key, val = (name, r["Grid_Size"], r["Counter_Name"]), float(r["Counter_Value"])
            else:
                key = (name, "%sx%s" % (r.get("Grid_Size_X", r.get("Grid_Size", "")), r.get("Grid_Size_Y", "")),
                       "duration_us")
                val = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-3
            rows.setdefault(key, []).append(val)
    for (name, grid, what), v in sorted(rows.items()):
        print("%-60s grid=%-12s %-14s n=%-5d mean=%.6g" % (name[:60], grid, what, len(v), sum(v) / len(v)))


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(how the path would shard is described in the design notes); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    lib_path = os.path.join(ROOT, "blockwise_bit_quantized_amd", "libmnb.so")
    if not os.path.exists(lib_path):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_mnb_build", os.path.join(ROOT, "blockwise_bit_quantized_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    import blockwise_bit_quantized_amd as mnb
    import seeded_inputs as si

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe:
        # a plain copy of known size: the counters' reading for it calibrates their units
        n = args.copy_probe * 2**20
        a = torch.ones(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 10}), flush=True)
        return

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(dev)

    def weight(case):
        zp = torch.from_numpy(case["zp"]).to(dev) if case["zp"] is not None else None
        return mnb.pack(torch.from_numpy(case["codes"]).to(dev), t16(case["scales"]), zp, case["bits"])

    # ---- decode workload, rotated copies ----
    dec = si.make_config(2)
    dM, dN, dK = dec["M"], dec["N"], dec["K"]
    dbytes = algorithmic_bytes(dM, dN, dK, 4, False, 32)
    copies = max(1, math.ceil(args.cold_mib * 2**20 / dbytes))
    pw0 = weight(dec)
    X0, A0, B0 = t16(dec["X"]), t16(dec["adapter"]["A"]), t16(dec["adapter"]["B"])
    dcopies = []
    for _ in range(copies):
        pw = mnb.PackedWeight(pw0.wq.clone(), pw0.sc.clone(), None, dN, dK, 4)
        dcopies.append((X0.clone(), pw, mnb.Adapter(mnb.MNB_ADAPTER_F16, A0.clone(), B0.clone())))
    Yd = torch.empty((dM, dN), dtype=torch.float16, device=dev)

    # ---- prefill workload ----
    pre = si.make_config(3)
    pM, pN, pK = pre["M"], pre["N"], pre["K"]
    pflops = algorithmic_flops(pM, pN, pK, 32)
    pbytes = algorithmic_bytes(pM, pN, pK, 4, True, 32)
    ppw = weight(pre)
    pX = t16(pre["X"])
    pad = mnb.Adapter(mnb.MNB_ADAPTER_F16, t16(pre["adapter"]["A"]), t16(pre["adapter"]["B"]))
    Yp = torch.empty((pM, pN), dtype=torch.float16, device=dev)

    ws = mnb.workspace(dev, max(mnb.mnb_workspace_bytes(dM, dN, dK, 4, 32),
                                mnb.mnb_workspace_bytes(pM, pN, pK, 4, 32)))
    torch.cuda.synchronize()

    def decode(i):
        X, pw, ad = dcopies[i % copies]
        mnb.matmul(X, pw, ad, out=Yd, ws=ws)

    def prefill():
        mnb.matmul(pX, ppw, pad, out=Yp, ws=ws)

    for i in range(args.warmup):
        decode(i)
        prefill()
    torch.cuda.synchronize()

    # The timed region replays two captured graphs: K decode calls (rotating over the cold
    # copies) and then K prefill calls.  Graph replay keeps Python launch overhead out of
    # the measurement; events bracket each graph on the stream the kernels run on.
    K = args.steps
    cap = torch.cuda.Stream()
    g_dec, g_pre = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_dec, stream=cap):
        for i in range(K):
            decode(i)
    with torch.cuda.graph(g_pre, stream=cap):
        for i in range(K):
            prefill()
    torch.cuda.synchronize()
    g_dec.replay()                          # first replay (untimed): graph upload
    g_pre.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    wall0 = time.perf_counter()
    with torch.cuda.stream(cap):
        ev[0].record()
        g_dec.replay()
        ev[1].record()
        g_pre.replay()
        ev[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    dec_s = ev[0].elapsed_time(ev[1]) * 1e-3 / K
    pre_s = ev[1].elapsed_time(ev[2]) * 1e-3 / K
    total_ms = ev[0].elapsed_time(ev[2])
    dec_gbps = dbytes / dec_s / 1e9
    pre_tflops = pflops / pre_s / 1e12

    # context: warm (Infinity-Cache resident) decode, the two-launch decode variant and the
    # empty-adapter decode, each as a replayed graph of K calls
    def graph_time(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for j in range(n):
                fn(j)
        # untimed replays first: the first few replays of a new graph run up to 20% slower
        # (measured on the batched prefill: 110, 101, 100, 97, 94 us, then ~88.5 us); the
        # figure is the median of five timed replays
        for _ in range(4):
            g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(cap):
                a.record()
                g.replay()
                b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3 / n)
        return sorted(times)[2]

    dbytes_base = algorithmic_bytes(dM, dN, dK, 4, False, 0)
    context = None
    if not args.no_context:
        n_ctx = min(K, 100)
        warm_s = graph_time(lambda j: mnb.matmul(*dcopies[0], out=Yd, ws=ws), n_ctx)
        tsep_s = graph_time(lambda j: mnb.matmul(*dcopies[j % copies], flags=mnb.MNB_FLAG_T_SEPARATE, out=Yd,
                                                 ws=ws), n_ctx)
        base_s = graph_time(lambda j: mnb.matmul(dcopies[j % copies][0], dcopies[j % copies][1], None, out=Yd,
                                                 ws=ws), n_ctx)
        context = {"warm_us": round(warm_s * 1e6, 3), "warm_GBps": round(dbytes / warm_s / 1e9, 1),
                   "t_separate_us": round(tsep_s * 1e6, 3),
                   "empty_adapter_us": round(base_s * 1e6, 3),
                   "empty_adapter_GBps": round(dbytes_base / base_s / 1e9, 1)}
        # the same decode shape with 2-bit codes (default zero point 2) and the F16 adapter,
        # cold copies of the weights
        dec2 = si.make_random(2002, dM, dN, dK, 2, False, None)
        pw2 = weight(dec2)
        dbytes2 = algorithmic_bytes(dM, dN, dK, 2, False, 32)
        copies2 = max(1, math.ceil(args.cold_mib * 2**20 / dbytes2))
        w2 = [mnb.PackedWeight(pw2.wq.clone(), pw2.sc.clone(), None, dN, dK, 2) for _ in range(copies2)]
        two_s = graph_time(lambda j: mnb.matmul(X0, w2[j % copies2], dcopies[0][2], out=Yd, ws=ws), n_ctx)
        context["decode_2bit_us"] = round(two_s * 1e6, 3)
        context["decode_2bit_GBps"] = round(dbytes2 / two_s / 1e9, 1)
        del w2
    # context: the other prefill workloads (warm weights), each a replayed graph of calls
    pre_context = None
    if not args.no_context:
        pre_context = {}
        c256 = si.make_config(3, M=256)
        X256, Y256 = t16(c256["X"]), torch.empty((256, pN), dtype=torch.float16, device=dev)
        ws256 = torch.zeros(mnb.mnb_workspace_bytes(256, pN, pK, 4, 32), dtype=torch.uint8, device=dev)
        s256 = graph_time(lambda j: mnb.matmul(X256, ppw, pad, out=Y256, ws=ws256), 20)
        f256 = algorithmic_flops(256, pN, pK, 32)
        pre_context["m256_us"] = round(s256 * 1e6, 3)
        pre_context["m256_TFLOPs"] = round(f256 / s256 / 1e12, 2)
        pre_context["m256_route"] = mnb.mnb_describe_route(256, pN, pK, 4, True, mnb.MNB_ADAPTER_F16)[1]
        c5 = si.make_config(5)
        M5, N5, K5 = c5["M"], c5["N"], c5["K"]
        pw5 = weight(c5)
        a5 = c5["adapter"]
        ad5 = mnb.Adapter(mnb.MNB_ADAPTER_Q8, torch.from_numpy(a5["A"]).to(dev), torch.from_numpy(a5["B"]).to(dev),
                          t16(a5["A_scales"]), t16(a5["B_scales"]))
        X5, Y5 = t16(c5["X"]), torch.empty((M5, N5), dtype=torch.float16, device=dev)
        ws5 = torch.zeros(mnb.mnb_workspace_bytes(M5, N5, K5, 4, 32), dtype=torch.uint8, device=dev)
        s5 = graph_time(lambda j: mnb.matmul(X5, pw5, ad5, out=Y5, ws=ws5), 20)
        pre_context["batched_q8_us"] = round(s5 * 1e6, 3)
        pre_context["batched_q8_TFLOPs"] = round(algorithmic_flops(M5, N5, K5, 32) / s5 / 1e12, 2)
        pre_context["batched_q8_route"] = mnb.mnb_describe_route(M5, N5, K5, 4, False, mnb.MNB_ADAPTER_Q8)[1]
    dec_route = mnb.mnb_describe_route(dM, dN, dK, 4, False, mnb.MNB_ADAPTER_F16)[1]
    pre_route = mnb.mnb_describe_route(pM, pN, pK, 4, True, mnb.MNB_ADAPTER_F16)[1]
    traffic = recorded_traffic("gemv")

    out = {
        "metric": METRIC,
        "value": round(dec_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; shapes of the pages' decode and prefill projections)",
        "config": {
            "workload": "decode GEMV M=1 N=8192 K=2048 int4 block-32 default-zp + rank-32 F16 LoRA "
                        "(cold HBM, %d rotated copies) + prefill M=1024 N=4096 K=4096 int4 block-32 "
                        "explicit-zp + rank-32 F16 LoRA" % copies,
            "decode_bytes": dbytes, "prefill_flops": pflops,
        },
        "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": dec_route, "mean_us": round(dec_s * 1e6, 3)},
        "prefill": {"value": round(pre_tflops, 2), "unit": "TFLOP/s", "mean_us": round(pre_s * 1e6, 3),
                    "route": pre_route,
                    "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2), "peak": FP16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(pre_tflops / FP16_PEAK_TFLOPS, 4),
                                 "traffic": recorded_traffic("gemm")},
                    "bytes": pbytes},
        "decode_context": context,
        "prefill_context": pre_context,
        "wall_s": round(wall, 3),
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(si, dec, pre, dbytes, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>_*_traffic.md, if the kernel sources still hash to the recorded value
    (else None: the counters describe a kernel that no longer exists)."""
    import glob
    import hashlib
    import re
    for path in glob.glob(os.path.join(ROOT, "profiles", kernel + "_*_traffic.md")):
        text = open(path).read()
        h = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
        b = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
        if not (h and b):
            continue
        if h.group(1) == kernel_source_hash(kernel):
            return int(b.group(1))
    return None


def kernel_source_hash(kernel):
    import hashlib
    csrc = os.path.join(ROOT, "blockwise_bit_quantized_amd", "csrc")
    d = hashlib.sha256()
    for f in (kernel + ".hip", "common.h"):
        d.update(open(os.path.join(csrc, f), "rb").read())
    return d.hexdigest()


def cpu_baseline(si, dec, pre, dbytes, budget_s):
    """The FP64 oracle as it stands, on this host's cores, on a bounded sample."""
    import numpy as np
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(threads)
    oracle.matmul(dict(dec, X=dec["X"][:1], M=1, N=64, codes=dec["codes"][:64], scales=dec["scales"][:64],
                       adapter=None))                       # load + warm
    t = []
    t_end = time.perf_counter() + budget_s * 0.6
    while time.perf_counter() < t_end or len(t) < 2:
        a = time.perf_counter()
        oracle.matmul(dec)
        t.append(time.perf_counter() - a)
    dec_s = float(np.median(t))
    rows = 8
    a = time.perf_counter()
    oracle.matmul(dict(pre, X=pre["X"][:rows], M=rows))
    pre_s = time.perf_counter() - a
    pre_flops = algorithmic_flops(rows, pre["N"], pre["K"], 32)
    return {"value": round(dbytes / dec_s / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "decode 8192x2048 int4 + F16 LoRA, full call, median of %d runs (%.3f s each); "
                      "prefill sample %d of 1024 rows of 1024x4096x4096: %.4f TFLOP/s"
                      % (len(t), dec_s, rows, pre_flops / pre_s / 1e12),
            "decode_s": round(dec_s, 4), "prefill_rows_s": round(pre_s, 3),
            "prefill_TFLOPs": round(pre_flops / pre_s / 1e12, 6)}


if __name__ == "__main__":
    main()
