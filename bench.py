#!/usr/bin/env python3
"""Throughput of the LLM.int8() linear layer on one MI355X.

One step = one int8_linear call (outlier scan, row quantization, int8 GEMM,
outlier fp16 product, dequantize + add) on synthetic seeded inputs already
resident in HBM; the weight is quantized once, untimed, as the layer does when
it is placed on the GPU.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload decode]
    python bench.py --copy-calibration 512   # plain 512 MiB device copy only

--copy-calibration runs nothing but torch's device-to-device copy of a buffer
of known size; under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE it gives the
factor that turns those counters into bytes.

The default workload is the decode shape X 8x4096 . W 4096x16384 with 4
outlier columns.  The K timed steps are captured into one HIP graph and
replayed (--no-graph launches each step from Python instead).  To keep the 256 MB Infinity Cache from serving the weight,
steps rotate over several copies of (X, Wq, sw, W, Y, workspace) totalling
more than 512 MB.
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

# MI355X published peaks.
PEAK_HBM_GBS = 8000.0
PEAK_INT8_TOPS = 5000.0

# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs,
# scaled by the copy-kernel calibration factor; valid only for the kernel
# source it was measured on (sha256 of the listed files).
# (profiles/traffic-decode.md: FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000 KiB, the
# factors a 512 MiB device copy gives).
TRAFFIC = {
    ("decode_kernel", "decode"): {"bytes": 68493926, "src": "8f99556e532f1095"},
    ("decode_stream_kernel", "decode_mlp_down"): {"bytes": 828347298, "src": "8f99556e532f1095"},
    ("gemm_i8_kernel", "qkv_prefill"): {"bytes": 2186834511, "src": "2d0553e1e5f71659"},
    ("gemm_i8_kernel", "mlp_down_prefill"): {"bytes": 5555634139, "src": "2d0553e1e5f71659"},
}


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mixed_precision_quantized_int8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w):
    """Bytes the method must move once: X, Wq, the outlier weight rows, Y, scales."""
    return (2 * w.M * w.K + w.N * w.K + 2 * w.n_out * w.N + 2 * w.M * w.N
            + 4 * w.N + 4 * w.M + 4 * w.n_out)


def dominant_kernel(w):
    """The kernel that carries the call: the fused small-M kernel (M <= 16,
    K <= 4096), the streaming kernel (M <= 64 otherwise) or the GEMM."""
    if w.M <= 64:
        name = "decode_kernel" if w.M <= 16 and w.K <= 4096 else "decode_stream_kernel"
        return name, "hbm", ["decode.hip", "common.h"]
    return "gemm_i8_kernel", "mfma", ["gemm.hip", "common.h"]


def cpu_baseline(w, X, W, budget_s=12.0, sample_rows=64):
    """Time the CPU oracle (as it stands) on the same workload on the host cores.

    Small-M workloads run whole; for larger M the sample is the first
    ``sample_rows`` rows of X against the whole weight (every row of X carries
    the same injected outlier columns, so the sample's outlier set is the
    workload's), and the rate is scaled by the sample's share of the ops."""
    import numpy as np
    from oracle import int8_oracle as O

    threads = None
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((i.get("num_threads") or 0) for i in info) if info else None
    except Exception:
        pass
    Wq, sw = O.quantize_weight(W)            # untimed, as on the GPU side
    rows = w.M if w.M <= 2 * sample_rows else sample_rows
    Xs = X[:rows]
    reps, t_total, out = 0, 0.0, None
    t0 = time.perf_counter()
    while reps < 100 and (time.perf_counter() - t0) < budget_s:
        s = time.perf_counter()
        out = O.int8_linear(Xs, Wq, sw, W, w.threshold)
        t_total += time.perf_counter() - s
        reps += 1
    per_call = t_total / reps
    what = (f"full {w.name} call ({w.M}x{w.K}x{w.N})" if rows == w.M else
            f"first {rows} of {w.M} rows of the {w.name} call ({rows}x{w.K}x{w.N}), "
            f"rate scaled by the row share")
    return {
        "value": round(2.0 * rows * w.N * w.K / per_call / 1e12, 6),
        "unit": "TOPS",
        "cores": threads or os.cpu_count(),
        "kind": "oracle",
        "sample": f"{what}, weight pre-quantized, {reps} calls, {per_call * 1e3:.1f} ms/call; "
                  f"host has {os.cpu_count()} cpus",
    }, out, Wq, sw, rows


def copy_ceiling(torch, dev, mib=1024, reps=10):
    """Device-to-device copy rate (bytes read + written per second) of torch's copy kernel."""
    src = torch.empty((mib << 20,), dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps):
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2 * (mib << 20) / (best * 1e-3) / 1e9


def fp16_context(torch, w, sets, int8_ms, reps):
    """Context only, not part of the library: the plain fp16 product X.W at the
    same shape through torch.matmul (the vendor BLAS), over the same rotated
    buffer sets, timed with events around `reps` back-to-back calls."""
    out = torch.empty((w.M, w.N), dtype=torch.float16, device=sets[0][0].device)
    R = len(sets)
    for i in range(3):
        torch.matmul(sets[i % R][0], sets[i % R][3], out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        torch.matmul(sets[i % R][0], sets[i % R][3], out=out)
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    return {"op": "torch.matmul fp16 X.W (vendor BLAS), eager launches, same buffer sets",
            "ms_per_call": round(ms, 5),
            "tflops": round(2.0 * w.M * w.N * w.K / (ms * 1e-3) / 1e12, 2),
            "int8_layer_speedup": round(ms / int8_ms, 3)}


def copy_calibration(mib):
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    src = torch.empty((mib << 20,), dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": mib << 20,
                      "copy_calibration_bytes_written": mib << 20, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets (0: auto, >512 MB)")
    ap.add_argument("--rebuilt-rows", action="store_true",
                    help="keep no fp16 weight: outlier rows rebuilt from the codes")
    ap.add_argument("--bias", action="store_true", help="add an fp16 bias [N]")
    ap.add_argument("--zero-point", action="store_true",
                    help="zero-point (unsigned) activation codes: int8_linear_zp")
    ap.add_argument("--no-fp16-context", action="store_true",
                    help="skip timing torch.matmul in fp16 at the same shape")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every step from Python instead of replaying a captured graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB buffer three times (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    import mixed_precision_quantized_int8_amd as pkg
    from mixed_precision_quantized_int8_amd import _binding, workloads

    if not os.path.exists(_binding.LIB_PATH):
        from mixed_precision_quantized_int8_amd import build
        build.build_library()

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    X, W, _ = workloads.make_inputs(w)
    Xd = torch.from_numpy(X).to(dev)
    Wd = torch.from_numpy(W).to(dev)
    Wq, sw = pkg.quantize_weight(Wd)
    ws_bytes = pkg.workspace_bytes(w.M, w.K, w.N)
    # bytes a step streams: X, Wq, Y (the fp16 weight is only read at outlier rows)
    set_bytes = Xd.numel() * 2 + Wq.numel() + 2 * w.M * w.N
    R = args.rotate or max(1, min(16, -(-512 * 2**20 // set_bytes)))
    sets = []
    for r in range(R):
        if r == 0:
            s = (Xd, Wq, sw, Wd)
        else:
            s = (Xd.clone(), Wq.clone(), sw.clone(), Wd.clone())
        ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
        Y = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
        S = pkg.weight_code_sums(s[1]) if args.zero_point else None   # once per layer
        sets.append((*s, ws, Y, S))

    bias_t = (torch.randn(w.N, device=dev) * 0.1).half() if args.bias else None

    def step(i):
        x, q, s, wf, ws, y, S = sets[i % R]
        rows = None if args.rebuilt_rows else wf
        if args.zero_point:
            pkg.linear_zp(x, q, s, S, rows, w.threshold, workspace=ws, out=y, bias=bias_t)
        else:
            pkg.linear(x, q, s, rows, w.threshold, workspace=ws, out=y, bias=bias_t)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    eager_ms = None
    if not args.no_graph:
        # The K steps are captured once into a HIP graph and replayed: the
        # kernels then run back to back, as in a serving loop, instead of
        # waiting on the Python launch path.  The graph holds no memset nodes
        # (the library clears its flags with a fill kernel).
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            for i in range(3):
                step(i)
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                step(i)
        graph.replay()   # untimed first replay
        torch.cuda.synchronize()
        t_begin = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_begin.record()
        graph.replay()
        t_end.record()
        torch.cuda.synchronize()
        ms_total = t_begin.elapsed_time(t_end)
        ms_per_step = ms_total / K
        per_launch = np.array([ms_per_step])
        ms_launch = ms_per_step
        # eager launches, for reference (Python launch path included)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / K
    else:
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        t_begin = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_begin.record()
        for i in range(K):
            starts[i].record()
            step(i)
            ends[i].record()
        t_end.record()
        torch.cuda.synchronize()
        ms_total = t_begin.elapsed_time(t_end)
        ms_per_step = ms_total / K
        per_launch = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
        ms_launch = float(per_launch.mean())

    value = w.int_ops / (ms_per_step * 1e-3) / 1e12
    kname, bound, files = dominant_kernel(w)
    src_hash = kernel_source_hash(files)
    if bound == "hbm":
        alg = algorithmic_bytes(w)
        achieved = alg / (ms_launch * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = w.int_ops / (ms_launch * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_INT8_TOPS,
                "unit": "TOPS", "frac": round(achieved / PEAK_INT8_TOPS, 4)}
    # counter figures were taken on the default layer (fp16 outlier rows, absmax codes)
    tr = None if (args.zero_point or args.rebuilt_rows) else TRAFFIC.get((kname, w.name))
    roof["traffic"] = tr["bytes"] if tr and tr["src"] == src_hash else None
    roof["kernel"] = kname
    roof["kernel_ms"] = round(ms_launch, 5)
    if args.no_graph:
        roof["kernel_ms_p10_p50_p90"] = [round(float(np.percentile(per_launch, q)), 5)
                                         for q in (10, 50, 90)]
    roof["kernel_src"] = src_hash
    roof["measured_copy_GBs"] = round(copy_ceiling(torch, dev), 1)

    result = {
        "metric": "int8_linear TOPS and % of int8-MFMA / HBM roofline on one MI355X",
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "K": w.K, "N": w.N,
                   "outlier_columns": w.n_out, "threshold": w.threshold,
                   "buffer_sets": R, "x_dtype": "fp16", "y_dtype": "fp16",
                   "outlier_rows": "rebuilt from codes" if args.rebuilt_rows else "fp16 weight",
                   "bias": bool(args.bias),
                   "activation_codes": "zero-point" if args.zero_point else "absmax",
                   "ops_int8": 2 * w.M * w.N * (w.K - w.n_out), "ops_fp16": 2 * w.M * w.N * w.n_out,
                   "launch": "eager" if args.no_graph else "hip_graph"},
        "roofline": roof,
    }
    if eager_ms is not None:
        result["eager_ms_per_step"] = round(eager_ms, 5)

    if not args.no_fp16_context:
        result["fp16_context"] = fp16_context(torch, w, sets, ms_per_step, min(K, 50))

    if not args.no_cpu_baseline:
        if args.rebuilt_rows or args.bias or args.zero_point:
            raise SystemExit("the CPU baseline and parity check cover the default layer only "
                             "(run with --no-cpu-baseline)")
        cb, ref, Wq_o, sw_o, rows = cpu_baseline(w, X, W)
        result["cpu_baseline"] = cb
        y = sets[0][5][:rows].cpu().numpy().astype(np.float64)
        err = np.abs(y - ref["Y64"])
        tol = np.maximum(2e-3 * np.abs(ref["Y64"]), 1e-2)
        result["parity"] = {
            "Y_within_tol": bool(np.all(err <= tol)),
            "Wq_bitexact": bool(np.array_equal(Wq.cpu().numpy(), Wq_o)),
            "max_abs_err": float(err.max()),
        }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
