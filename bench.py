#!/usr/bin/env python3
"""Benchmark of the MatMulNBits hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  * decode: Y[1, 8192] = X[1, 2048] . deq(W)^T + (X.A).B, INT4 block-32 weights with the
    default zero point and a rank-32 F16 LoRA fused in the same launch (in-pass T);
  * prefill: Y[1024, 4096] = X[1024, 4096] . deq(W)^T + (X.A).B, INT4 block-32 with explicit
    zero points, rank-32 F16 LoRA (T projection launch + MFMA GEMM with the T.B epilogue).
Inputs are resident in HBM before timing.  Decode-shaped (HBM-bound) runs rotate over
enough copies of their weights, activations and adapter (default >= 1 GiB, four times the
256 MB Infinity Cache) that every call streams from HBM; prefill-shaped (MFMA-bound) runs
use one copy.

Timing: every figure comes from replays of captured HIP graphs of calls, events bracketing
each replay on the stream the kernels run on.  Each graph (or, for cold runs, each of the
graphs that together cover every copy once) is replayed four times untimed -- the first
replays of a new graph run up to 20% slower -- and then five times timed; the figure is the
median of the five.  The headline graphs hold exactly --steps calls each.

`value` is the decode GEMV's effective HBM bandwidth (algorithmic bytes / decode call time,
GB/s); the prefill TFLOP/s rides along in `prefill`; `runs` holds every decode and prefill
workload (µs, rate, fraction of the roofline, route) and `ceilings` what the same GPU does
on plain work of the same size: a streaming read of the decode byte counts (cold) and the
dense FP16 GEMM of the prefill shape.
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
    ap.add_argument("--cold-mib", type=int, default=1024, help="bytes of rotated copies for HBM-bound runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle decode baseline")
    ap.add_argument("--no-context", action="store_true",
                    help="only the two headline graphs (counter collection and kernel traces)")
    ap.add_argument("--only", choices=["decode", "prefill"],
                    help="with --no-context: only that headline graph (a cold-only decode trace)")
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
        v = sorted(v)
        print("%-60s grid=%-12s %-26s n=%-5d mean=%.6g median=%.6g" % (name[:60], grid, what, len(v),
                                                                      sum(v) / len(v), v[len(v) // 2]))


class Timer:
    """Median-of-five timing of captured graphs on one stream (four untimed replays first)."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream

    def capture(self, fn, calls):
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g, stream=self.stream):
            for j in calls:
                fn(j)
        return g

    def time_graphs(self, graphs, n_calls):
        """Seconds per call: graphs are replayed round-robin (4 untimed, 5 timed); each timed
        replay holds n_calls calls; returns the median replay / n_calls."""
        torch = self.torch
        torch.cuda.synchronize()
        i = 0
        for _ in range(4):
            graphs[i % len(graphs)].replay()
            i += 1
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(self.stream):
                a.record()
                graphs[i % len(graphs)].replay()
                b.record()
            i += 1
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3 / n_calls)
        return sorted(times)[2]

    def paired(self, fn_a, fn_b, n_calls):
        """Seconds per call of fn_a and of fn_b (warm, no rotation): one graph of n_calls calls
        each, replayed alternately (4 untimed pairs, then 5 timed), so that both see the same
        clocks and cache state; returns the two medians."""
        torch = self.torch
        fn_a(0)
        fn_b(0)
        torch.cuda.synchronize()
        ga, gb = self.capture(fn_a, range(n_calls)), self.capture(fn_b, range(n_calls))
        for _ in range(4):
            ga.replay()
            gb.replay()
        torch.cuda.synchronize()
        ta, tb = [], []
        for _ in range(5):
            for g, out in ((ga, ta), (gb, tb)):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(self.stream):
                    a.record()
                    g.replay()
                    b.record()
                torch.cuda.synchronize()
                out.append(a.elapsed_time(b) * 1e-3 / n_calls)
        del ga, gb
        return sorted(ta)[2], sorted(tb)[2]

    def per_call(self, fn, n_items, n_calls):
        """Seconds per call of fn(j), n_calls calls per graph.  fn rotates over n_items items
        (cold copies) by j; with more items than calls per graph, consecutive graphs take
        consecutive items, so that a replay finds its items cold."""
        fn(0)                              # eager first: libraries initialise outside capture
        self.torch.cuda.synchronize()
        if n_items <= n_calls:
            graphs = [self.capture(fn, range(n_calls))]
        else:
            graphs = [self.capture(fn, range(s, s + n_calls)) for s in range(0, n_items - n_calls + 1, n_calls)]
        t = self.time_graphs(graphs, n_calls)
        del graphs
        return t


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

    def adapter(case):
        a = case.get("adapter")
        if a is None:
            return None
        if a["kind"] == "f16":
            return mnb.Adapter(mnb.MNB_ADAPTER_F16, t16(a["A"]), t16(a["B"]))
        return mnb.Adapter(mnb.MNB_ADAPTER_Q8, torch.from_numpy(a["A"]).to(dev), torch.from_numpy(a["B"]).to(dev),
                           t16(a["A_scales"]), t16(a["B_scales"]))

    def clone_weight(pw):
        return mnb.PackedWeight(pw.wq.clone(), pw.sc.clone(), None if pw.zp is None else pw.zp.clone(),
                                pw.N, pw.K, pw.bits)

    def clone_adapter(a):
        if a is None:
            return None
        c = lambda t: None if t is None else t.clone()
        return mnb.Adapter(a.kind, c(a.A), c(a.B), c(a.A_scales), c(a.B_scales))

    def route(case, ad_kind, flags=0):
        opt = mnb.mnb_options(0, flags) if flags else None
        return mnb.mnb_describe_route(case["M"], case["N"], case["K"], case["bits"], case["zp"] is not None,
                                      ad_kind, opt)[1]

    def cold_copies(case, nbytes):
        """(X, weight, adapter) copies whose total bytes reach --cold-mib, so that a call
        finds none of its inputs in the 256 MB Infinity Cache."""
        r = max(1, math.ceil(args.cold_mib * 2**20 / nbytes))
        pw, ad, X = weight(case), adapter(case), t16(case["X"])
        return [(X.clone(), clone_weight(pw), clone_adapter(ad)) for _ in range(r)]

    timer = Timer(torch, torch.cuda.Stream())
    K = args.steps

    # ---- headline: cold decode (cfg2 + F16 LoRA) and prefill (cfg3, M = 1024) ----
    dec = si.make_config(2)
    dM, dN, dK = dec["M"], dec["N"], dec["K"]
    dbytes = algorithmic_bytes(dM, dN, dK, 4, False, 32)
    dcopies = cold_copies(dec, dbytes)
    Yd = torch.empty((dM, dN), dtype=torch.float16, device=dev)

    pre = si.make_config(3)
    pM, pN, pK = pre["M"], pre["N"], pre["K"]
    pflops = algorithmic_flops(pM, pN, pK, 32)
    pbytes = algorithmic_bytes(pM, pN, pK, 4, True, 32)
    ppw, pX, pad = weight(pre), t16(pre["X"]), adapter(pre)
    Yp = torch.empty((pM, pN), dtype=torch.float16, device=dev)

    ws = torch.zeros(max(mnb.mnb_workspace_bytes(dM, dN, dK, 4, 32), mnb.mnb_workspace_bytes(pM, pN, pK, 4, 32),
                         mnb.mnb_workspace_bytes(256, pN, pK, 4, 32), 1 << 20), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def decode(j):
        X, pw, ad = dcopies[j % len(dcopies)]
        mnb.matmul(X, pw, ad, out=Yd, ws=ws)

    def prefill(j):
        mnb.matmul(pX, ppw, pad, out=Yp, ws=ws)

    for i in range(args.warmup):
        decode(i)
        prefill(i)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    dec_s = pre_s = 0.0
    if args.only != "prefill":
        dec_s = timer.per_call(decode, len(dcopies), K)
    if args.only != "decode":
        pre_s = timer.per_call(prefill, 1, K)
    wall = time.perf_counter() - wall0
    dec_gbps = dbytes / dec_s / 1e9 if dec_s else 0.0
    pre_tflops = pflops / pre_s / 1e12 if pre_s else 0.0
    dec_route = route(dec, mnb.MNB_ADAPTER_F16)
    pre_route = route(pre, mnb.MNB_ADAPTER_F16)

    runs = ceilings = context = None
    if not args.no_context:
        runs, ceilings, context = {}, {}, {}

        def hbm_run(name, case, ad_kind, nbytes, flags=0, with_adapter=True):
            copies = cold_copies(case, nbytes)
            Y = torch.empty((case["M"], case["N"]), dtype=torch.float16, device=dev)
            w = torch.zeros(max(mnb.mnb_workspace_bytes(case["M"], case["N"], case["K"], case["bits"], 32), 1),
                            dtype=torch.uint8, device=dev)

            def call(j):
                X, pw, ad = copies[j % len(copies)]
                mnb.matmul(X, pw, ad if with_adapter else None, flags=flags, out=Y, ws=w)
            s = timer.per_call(call, len(copies), min(K, 100))
            runs[name] = {"us": round(s * 1e6, 3), "GBps": round(nbytes / s / 1e9, 1),
                          "frac": round(nbytes / s / 1e9 / HBM_PEAK_GBPS, 4), "bytes": nbytes, "cold": True,
                          "copies": len(copies), "route": route(case, ad_kind if with_adapter else 0, flags)}
            del copies
            return s

        def mfma_run(name, case, ad_kind, n_calls=20, flags=0):
            pw, ad, X = weight(case), adapter(case), t16(case["X"])
            M, N, Kc = case["M"], case["N"], case["K"]
            Y = torch.empty((M, N), dtype=torch.float16, device=dev)
            w = torch.zeros(max(mnb.mnb_workspace_bytes(M, N, Kc, case["bits"], 32), 1), dtype=torch.uint8,
                            device=dev)
            s = timer.per_call(lambda j: mnb.matmul(X, pw, ad, flags=flags, out=Y, ws=w), 1, n_calls)
            fl = algorithmic_flops(M, N, Kc, 32 if ad is not None else 0)
            runs[name] = {"us": round(s * 1e6, 3), "TFLOPs": round(fl / s / 1e12, 2),
                          "frac": round(fl / s / 1e12 / FP16_PEAK_TFLOPS, 4), "flops": fl, "cold": False,
                          "route": route(case, ad_kind, flags)}
            return s

        def mfma_pair(name, name_empty, case, case_empty, ad_kind, n_calls=50):
            """The prefill with its adapter and without, timed interleaved (same clocks and
            cache state), and the adapter's cost as their difference.  Graphs of 50 calls,
            like the headline's: with the adapter (two launches per call) the time per call
            still falls with the graph's length (1024x4096x4096: 53 us at 20 calls, 50 at 50,
            48.7 at 100), without it it is flat from 5 calls on."""
            pw, ad, X = weight(case), adapter(case), t16(case["X"])
            M, N, Kc = case["M"], case["N"], case["K"]
            Y = torch.empty((M, N), dtype=torch.float16, device=dev)
            w = torch.zeros(max(mnb.mnb_workspace_bytes(M, N, Kc, case["bits"], 32), 1), dtype=torch.uint8,
                            device=dev)
            sa, sb = timer.paired(lambda j: mnb.matmul(X, pw, ad, out=Y, ws=w),
                                  lambda j: mnb.matmul(X, pw, None, out=Y, ws=w), n_calls)
            for nm, sec, kind, r in ((name, sa, ad_kind, 32), (name_empty, sb, 0, 0)):
                fl = algorithmic_flops(M, N, Kc, r)
                runs[nm] = {"us": round(sec * 1e6, 3), "TFLOPs": round(fl / sec / 1e12, 2),
                            "frac": round(fl / sec / 1e12 / FP16_PEAK_TFLOPS, 4), "flops": fl, "cold": False,
                            "route": route(case if kind else case_empty, kind, 0)}
            runs[name]["lora_cost_us"] = round((sa - sb) * 1e6, 3)
            runs[name]["timing"] = "replayed alternately with %s" % name_empty

        # every decode and prefill run of the workloads
        c1 = si.make_config(1)
        hbm_run("cfg1_m1", c1, mnb.MNB_ADAPTER_F16, algorithmic_bytes(1, 896, 896, 4, True, 32))
        runs["cfg2_m1_lora"] = {"us": round(dec_s * 1e6, 3), "GBps": round(dec_gbps, 1),
                                "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "bytes": dbytes, "cold": True,
                                "copies": len(dcopies), "route": dec_route, "note": "headline"}
        hbm_run("cfg2_m1_empty", dec, 0, algorithmic_bytes(1, dN, dK, 4, False, 0), with_adapter=False)
        runs["cfg3_m1024"] = {"us": round(pre_s * 1e6, 3), "TFLOPs": round(pre_tflops, 2),
                              "frac": round(pre_tflops / FP16_PEAK_TFLOPS, 4), "flops": pflops, "cold": False,
                              "route": pre_route, "note": "headline"}
        mfma_run("cfg3_m256", si.make_config(3, M=256), mnb.MNB_ADAPTER_F16)
        mfma_pair("cfg3_m1024_paired", "cfg3_m1024_empty", pre, si.make_config(3, adapter=False),
                  mnb.MNB_ADAPTER_F16)
        hbm_run("cfg3_m1", si.make_config(3, M=1), mnb.MNB_ADAPTER_F16, algorithmic_bytes(1, pN, pK, 4, True, 32))
        hbm_run("cfg4_m1", si.make_config(4, M=1), 0, algorithmic_bytes(1, 49152, 576, 8, True, 0))
        hbm_run("cfg4_m8", si.make_config(4, M=8), 0, algorithmic_bytes(8, 49152, 576, 8, True, 0))
        mfma_pair("cfg5_m1024", "cfg5_m1024_empty", si.make_config(5), si.make_config(5, adapter=False),
                  mnb.MNB_ADAPTER_Q8)
        # accuracy level 4 (block-quantized activations) at the prefill shape
        mfma_run("cfg3_m1024_acc4", pre, mnb.MNB_ADAPTER_F16, flags=mnb.MNB_FLAG_ACC4)

        # ceilings: a plain streaming read of the decode byte counts (cold), and the dense
        # FP16 GEMM at the prefill shape (hipBLASLt through torch)
        ceilings.update(stream_read_ceilings(torch, dev, timer, args.cold_mib, min(K, 100),
                                             {"cfg2_m1_lora": dbytes,
                                              "cfg4_m1": algorithmic_bytes(1, 49152, 576, 8, True, 0)}))
        Wd = torch.randn((pN, pK), dtype=torch.float16, device=dev) * 0.02
        Xd = torch.randn((pM, pK), dtype=torch.float16, device=dev)
        Yg = torch.empty((pM, pN), dtype=torch.float16, device=dev)
        sg = timer.per_call(lambda j: torch.matmul(Xd, Wd.t(), out=Yg), 1, 20)
        ceilings["dense_fp16_gemm_1024x4096x4096"] = {
            "us": round(sg * 1e6, 3), "TFLOPs": round(2 * pM * pN * pK / sg / 1e12, 2),
            "frac": round(2 * pM * pN * pK / sg / 1e12 / FP16_PEAK_TFLOPS, 4),
            "what": "torch.matmul of fp16 X[1024,4096] by W^T (dense fp16 weights, rocBLAS/hipBLASLt), no LoRA"}
        del Wd, Xd, Yg

        # context: warm decode, the two-launch decode, and 2-bit codes
        warm = dcopies[0]
        s = timer.per_call(lambda j: mnb.matmul(*warm, out=Yd, ws=ws), 1, min(K, 100))
        context["cfg2_warm_us"] = round(s * 1e6, 3)
        context["cfg2_warm_GBps"] = round(dbytes / s / 1e9, 1)
        s = timer.per_call(lambda j: mnb.matmul(*dcopies[j % len(dcopies)], flags=mnb.MNB_FLAG_T_SEPARATE, out=Yd,
                                                ws=ws), len(dcopies), min(K, 100))
        context["cfg2_t_separate_us"] = round(s * 1e6, 3)
        dec2 = si.make_random(2002, dM, dN, dK, 2, False, None)
        pw2 = weight(dec2)
        dbytes2 = algorithmic_bytes(dM, dN, dK, 2, False, 32)
        r2 = max(1, math.ceil(args.cold_mib * 2**20 / dbytes2))
        w2 = [clone_weight(pw2) for _ in range(r2)]
        s = timer.per_call(lambda j: mnb.matmul(dcopies[0][0], w2[j % r2], dcopies[0][2], out=Yd, ws=ws), r2,
                           min(K, 100))
        context["cfg2_2bit_us"] = round(s * 1e6, 3)
        context["cfg2_2bit_GBps"] = round(dbytes2 / s / 1e9, 1)
        del w2

    traffic = recorded_traffic("gemv")
    out = {
        "metric": METRIC,
        "value": round(dec_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round((dec_s + pre_s) * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; shapes of the pages' decode and prefill projections)",
        "config": {
            "workload": "decode GEMV M=1 N=8192 K=2048 int4 block-32 default-zp + rank-32 F16 LoRA "
                        "(cold HBM, %d rotated copies) + prefill M=1024 N=4096 K=4096 int4 block-32 "
                        "explicit-zp + rank-32 F16 LoRA" % len(dcopies),
            "decode_bytes": dbytes, "prefill_flops": pflops,
            "timing": "median of 5 timed replays of %d-call graphs after 4 untimed replays" % K,
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
        "runs": runs,
        "ceilings": ceilings,
        "decode_context": context,
        "wall_s": round(wall, 3),
    }

    if not args.no_cpu_baseline and not args.no_context:
        out["cpu_baseline"] = cpu_baseline(si, dec, pre, dbytes, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def stream_read_ceilings(torch, dev, timer, cold_mib, n_calls, sizes):
    """A plain streaming read (ceiling.hip) of each byte count, cold: copies totalling
    cold_mib rotate; the best of 1, 2, 4 and 8 16-byte loads per thread is reported."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "blockwise_bit_quantized_amd", "libmnb_ceiling.so"))
    lib.mnb_ceiling_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int, C.c_void_p, C.c_void_p]
    lib.mnb_ceiling_stream_read.restype = C.c_int
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    out = {}
    for name, nbytes in sizes.items():
        nb = (nbytes + 15) // 16 * 16
        r = max(1, math.ceil(cold_mib * 2**20 / nb))
        bufs = [torch.randint(0, 255, (nb,), dtype=torch.uint8, device=dev) for _ in range(r)]
        best = None
        for u in (1, 2, 4, 8):
            def call(j, u=u):
                st = lib.mnb_ceiling_stream_read(bufs[j % r].data_ptr(), nb, u, sink.data_ptr(),
                                                 torch.cuda.current_stream(dev).cuda_stream)
                if st != 0:
                    raise RuntimeError("stream read launch failed: %d" % st)
            s = timer.per_call(call, r, n_calls)
            if best is None or s < best[0]:
                best = (s, u)
        out["stream_read_" + name] = {"us": round(best[0] * 1e6, 3), "bytes": nb,
                                      "GBps": round(nb / best[0] / 1e9, 1),
                                      "frac": round(nb / best[0] / 1e9 / HBM_PEAK_GBPS, 4),
                                      "loads_per_thread": best[1], "copies": r,
                                      "what": "one launch reading the bytes once (16 B loads, 256 threads per "
                                              "workgroup), cold, best of 1/2/4/8 loads per thread"}
        del bufs
    return out


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>_*_traffic.md, if the kernel sources still hash to the recorded value
    (else None: the counters describe a kernel that no longer exists)."""
    import glob
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(si, dec, pre, dbytes, budget_s):
    """The FP64 oracle as it stands, on this host's cores: full decode calls (median over
    about 0.6 x budget_s) and one full prefill call of all 1024 rows."""
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
    a = time.perf_counter()
    oracle.matmul(pre)
    pre_s = time.perf_counter() - a
    pre_flops = algorithmic_flops(pre["M"], pre["N"], pre["K"], 32)
    return {"value": round(dbytes / dec_s / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "decode 8192x2048 int4 + F16 LoRA, full call, median of %d runs (%.4f s each); "
                      "prefill 1024x4096x4096 int4 + F16 LoRA, one full call (all 1024 rows): %.3f s, "
                      "%.4f TFLOP/s" % (len(t), dec_s, pre_s, pre_flops / pre_s / 1e12),
            "decode_s": round(dec_s, 5), "prefill_s": round(pre_s, 3),
            "prefill_TFLOPs": round(pre_flops / pre_s / 1e12, 6)}


if __name__ == "__main__":
    main()
