"""Benchmark of the MI355X DeepSeekMoE layer forward (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|skew|fp8]
    python bench.py --workload fp8 --save-inputs DIR   # write the inputs, then ...
    python bench.py --workload fp8 --load-inputs DIR   # ... time them without generator kernels
    python bench.py --copy-calibration          # plain copy of known size, for HBM counters
    python bench.py --matmul-calibration        # a large library bf16 GEMM, for MFMA counters
    python bench.py --summarize-profile DIR     # text summary of rocprofv3 CSV output

A step is one moe_forward call (router, node-limited top-8 selection, gates,
permutation, routed + shared SwiGLU experts, gated combine) over one batch of
synthetic V3-shaped input already resident in HBM.  Prints one JSON line.

The default workload is the decode batch (T=256, bf16 weights): the
configuration the headline metric is quoted on, which gives `value`.  The
same line then carries `prefill` (T=8192, MFMA roofline), `skew` (T=4096,
200 loss-free bias steps with the per-step load ratio) and `fp8` (T=4096,
E4M3 weights) objects, each timed the same way on its own inputs
(`--no-extra` skips them).  Kernel durations come from HIP events recorded by
the library around each launch on the same stream, over the timed steps.  The
CPU baseline is the float64 oracle timed on a bounded sample of the decode
workload on this host's cores.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "e4m3": 5000.0, "f32": 157.3}


# HBM traffic of the dominant kernel, from rocprofv3 counter runs of this
# script (FETCH_SIZE and WRITE_SIZE, one run each, KiB per dispatch averaged
# over the profiled steps), each scaled by bytes / counter for a plain copy of
# known size (--copy-calibration).  The figures hold for the kernel sources
# whose digest is recorded; after any change to them traffic reads null.
COPY_CALIBRATION = {"fetch_bytes_per_kib": 1073741824 / 524302.8,   # 1 GiB buffer copy
                    "write_bytes_per_kib": 1073741824 / 1048576.0}
MEASURED_TRAFFIC = {         # workload -> counters per launch of the roofline's kernel
    "decode": {"src_sha256": "8a0b3e815a6bb8eb2a8c619719e7b54853d7f42ca3b936a329d60aa6b17927ca",
            "fetch_kib": 7494875.7, "write_kib": 9216.0},
    "fp8": {"src_sha256": "7274f2c893aa849aefb217607f641dfd9ff36ad1c2c8f306a8a16c7618d02bc9",
         "fetch_kib": 4913586.8, "write_kib": 92250.3},
    "prefill": {"src_sha256": "57672187660a41f15929fa5546331706d1b33d8efbc96d9881425f5038d69f06",
             "fetch_kib": 12248709.7, "write_kib": 294912.1},
    "backward_prefill_bf16": {"src_sha256": "2128ce0fa66e0506a9238675fc3ef127e496b8b08d0243b59df5b3c91fa379b5",
                            "fetch_kib": 6459360.2, "write_kib": 44215141.9},
    "backward_decode_bf16": {"src_sha256": "2128ce0fa66e0506a9238675fc3ef127e496b8b08d0243b59df5b3c91fa379b5",
                            "fetch_kib": 85689.9, "write_kib": 44234533.9},
}
# MFMA counters of gemm_gate_up from one rocprofv3 --pmc run (SQ_VALU_MFMA_BUSY_CYCLES,
# SQ_INSTS_VALU_MFMA_MOPS_BF16 or _F8, GRBM_GUI_ACTIVE; profiles/moe_forward_prefill_bf16.md):
# busy = fraction of SIMD-cycles the matrix cores worked at the clock the chip held
MEASURED_MFMA = {
    "prefill": {"src_sha256": "57672187660a41f15929fa5546331706d1b33d8efbc96d9881425f5038d69f06",
                "busy": 0.598, "clock_ghz": 1.59, "executed_bf16_tflop": 4.56},
    # (SQ_INSTS_VALU_MFMA_MOPS_F8; profiles/moe_forward_fp8_e4m3.md)
    "fp8": {"src_sha256": "7274f2c893aa849aefb217607f641dfd9ff36ad1c2c8f306a8a16c7618d02bc9",
            "busy": 0.319, "clock_ghz": 1.94, "executed_f8_tflop": 2.40},
}
# A plain 8192 x 8192 x 7168 bf16 GEMM through torch.matmul (hipBLASLt), `--matmul-calibration`,
# with its MFMA counters (profiles/moe_forward_prefill_bf16.md): what the vendor library sustains
# on this part on an ideal shape, at the clock the chip held under it.  Independent of this
# library's sources.
MATMUL_REFERENCE = {"kernel": "hipBLASLt bf16 GEMM 8192x8192x7168 (torch.matmul)",
                    "tflops_timed": 1164.0, "mfma_busy": 0.696, "clock_ghz": 1.70}
# sources the gate/up kernel of each workload is built and launched from
_COMMON_SOURCES = ("common.h", "kernels.h", "moe_api.cpp")
KERNEL_SOURCES = {"decode": _COMMON_SOURCES + ("lds_async.h", "stream_gemm.hip"),
                  "prefill": _COMMON_SOURCES + ("tile_gemm.hip",),
                  "skew": _COMMON_SOURCES + ("lds_async.h", "stream_gemm.hip", "tile_gemm.hip"),
                  "fp8": _COMMON_SOURCES + ("fp8_kernels.hip",),
                  # backward: the weight-gradient stage (all its launches in one call)
                  "backward_prefill_bf16": _COMMON_SOURCES + ("lds_async.h", "bwd.h", "bwd_kernels.hip"),
                  "backward_decode_bf16": _COMMON_SOURCES + ("lds_async.h", "bwd.h", "bwd_kernels.hip"),
                  "backward_prefill_e4m3": _COMMON_SOURCES + ("lds_async.h", "bwd.h", "bwd_fp8_kernels.hip")}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sources_sha256(workload):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[workload]:
        with open(os.path.join(ROOT, "sparse_moe_layer_group_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the roofline's kernel (gemm_gate_up; the backward's
    weight-gradient launches of one call together), or None when not measured for the
    current sources."""
    t = MEASURED_TRAFFIC.get(workload)
    if not t or not COPY_CALIBRATION or t["src_sha256"] != kernel_sources_sha256(workload):
        return None
    return int(t["fetch_kib"] * COPY_CALIBRATION["fetch_bytes_per_kib"] +
               t["write_kib"] * COPY_CALIBRATION["write_bytes_per_kib"])


def measured_mfma(workload):
    """MFMA busy-cycle counters of gemm_gate_up, or None when not measured for the current sources."""
    t = MEASURED_MFMA.get(workload)
    if not t or t["src_sha256"] != kernel_sources_sha256(workload):
        return None
    return {k: v for k, v in t.items() if k != "src_sha256"}


def copy_calibration(reps=5, nbytes=1 << 30):
    """Known-size copies whose HBM counters calibrate FETCH_SIZE / WRITE_SIZE.

    Two forms: torch's copy_ and an elementwise negation (one read and one
    write stream of nbytes each); 1 GiB is far beyond the 256 MB last-level
    cache, so every byte moves through HBM."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": nbytes, "bytes_written": nbytes,
                                            "reps": reps, "forms": ["copy_", "neg"]}}), flush=True)


def matmul_calibration(reps=20, m=8192, n=8192, k=7168):
    """A large plain bf16 GEMM through torch (hipBLASLt): what the vendor library
    sustains on this part, and, under rocprofv3 --pmc, the MFMA busy fraction and
    the clock the chip holds under a dense MFMA load."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(m, k, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(k, n, device=dev, dtype=torch.bfloat16, generator=g)  # contiguous, plain 2-D mm
    c = torch.empty(m, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    flops = 2.0 * m * n * k
    print(json.dumps({"matmul_calibration": {"m": m, "n": n, "k": k, "dtype": "bf16", "reps": reps,
                                             "ms": round(ms, 4),
                                             "tflops": round(flops / ms / 1e9, 1)}}), flush=True)


def summarize_profile(path):
    """Text summary of rocprofv3 CSV output under path: kernel time statistics
    (kernel_stats / kernel_trace) and per-dispatch counter averages."""
    files = sorted(glob.glob(os.path.join(path, "**", "*.csv"), recursive=True))
    for f in files:
        rows = list(csv.DictReader(open(f)))
        if f.endswith("kernel_stats.csv"):
            print(f"# {os.path.relpath(f, path)}: kernel durations")
            print(f"{'kernel':70s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s} {'total %':>8s}")
            for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
                print(f"{r['Name'][:70]:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                      f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f} "
                      f"{float(r['Percentage']):8.2f}")
        elif f.endswith("counter_collection.csv"):
            # counter names are truncated; the kernel id tells template instances apart
            d = collections.defaultdict(list)
            first = {}
            for r in rows:
                key = (r["Kernel_Name"], int(r["Kernel_Id"]), r["Counter_Name"])
                d[key].append(float(r["Counter_Value"]))
                first.setdefault(key, int(r["Dispatch_Id"]))
            print(f"# {os.path.relpath(f, path)}: counters per dispatch")
            print(f"{'kernel':40s} {'id':>6s} {'1st disp':>9s} {'counter':12s} {'dispatches':>10s} "
                  f"{'mean':>14s} {'min':>14s} {'max':>14s}")
            for key, v in sorted(d.items(), key=lambda kv: first[kv[0]]):
                k, kid, cn = key
                print(f"{k[:40]:40s} {kid:6d} {first[key]:9d} {cn:12s} {len(v):10d} "
                      f"{sum(v) / len(v):14.1f} {min(v):14.1f} {max(v):14.1f}")
            # MFMA utilisation per kernel when the run collected these counters:
            # busy = MFMA busy SIMD-cycles / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs)
            per = collections.defaultdict(lambda: collections.defaultdict(list))
            dur = collections.defaultdict(list)
            for r in rows:
                kk = (r["Kernel_Name"], int(r["Kernel_Id"]))
                per[kk][r["Counter_Name"]].append(float(r["Counter_Value"]))
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    dur[kk].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
            for fmt in ("BF16", "F8"):  # executed flops = MOPS x 512
                need = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_" + fmt)
                table = [(kk, c) for kk, c in per.items() if all(n in c for n in need) and dur[kk]]
                if not table:
                    continue
                print(f"{'kernel':40s} {'id':>6s} {'us':>9s} {'clock GHz':>10s} {'MFMA busy':>10s} "
                      f"{fmt.lower() + ' TFLOP':>11s} {'TFLOP/s':>9s}")
                for (k, kid), c in table:
                    t = sum(dur[(k, kid)]) / len(dur[(k, kid)])
                    grbm = sum(c[need[0]]) / len(c[need[0]])
                    busy = sum(c[need[1]]) / len(c[need[1]]) / (grbm / 8 * 1024)
                    tf = sum(c[need[2]]) / len(c[need[2]]) * 512 / 1e12
                    print(f"{k[:40]:40s} {kid:6d} {t * 1e6:9.1f} {grbm / 8 / t / 1e9:10.2f} "
                          f"{100 * busy:9.1f}% {tf:11.3f} {tf / t:9.1f}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "skew", "fp8", "backward"])
    ap.add_argument("--no-extra", action="store_true",
                    help="decode workload: skip the prefill, skew and fp8 objects of the line")
    ap.add_argument("--backward-shape", default="prefill", choices=["decode", "prefill"],
                    help="backward workload: batch shape (prefill T=8192 or decode T=256)")
    ap.add_argument("--backward-weights", default="bf16", choices=["bf16", "e4m3"],
                    help="backward workload: expert weights in bf16, or E4M3 with 128x128 block "
                         "scales (every expert GEMM in E4M3; inputs of the fp8 workload)")
    ap.add_argument("--skew-steps", type=int, default=200,
                    help="skew workload: bias-update steps (forward timed at first, middle, last)")
    ap.add_argument("--cpu-tokens", type=int, default=32,
                    help="tokens in the CPU oracle sample (0 disables the CPU baseline)")
    ap.add_argument("--save-inputs", default=None, metavar="DIR",
                    help="generate the workload's inputs on the GPU, write them under DIR and exit")
    ap.add_argument("--load-inputs", default=None, metavar="DIR",
                    help="read the workload's inputs from DIR (written by --save-inputs) instead "
                         "of generating them: the process then dispatches no generator kernels")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run plain copies of known size (for HBM counter calibration) and exit")
    ap.add_argument("--matmul-calibration", action="store_true",
                    help="time a large library bf16 GEMM (for MFMA counter reference) and exit")
    ap.add_argument("--summarize-profile", default=None, metavar="DIR",
                    help="print a text summary of the rocprofv3 CSV files under DIR and exit")
    args = ap.parse_args()

    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is benchmarked on a single MI355X)", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_moe_layer_group_amd as moe
    import synthetic as S

    if args.workload == "backward":
        bench_backward(args, np, torch, moe, S)
        return

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    if args.matmul_calibration:
        matmul_calibration()
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.save_inputs:
        save_inputs(args.save_inputs, S.get_config(args.workload), S, torch, dev)
        return

    res = bench_forward(args.workload, args, np, torch, moe, S, dev, primary=True)
    if args.workload == "decode" and not args.no_extra:
        # the other forward workloads, each timed the same way on its own inputs
        for name in ("prefill", "skew", "fp8"):
            torch.cuda.empty_cache()
            res[name] = bench_forward(name, args, np, torch, moe, S, dev, primary=False)
    print(json.dumps(res), flush=True)


_INPUT_FILES = ("x", "w_router", "bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")


def save_inputs(path, c, S, torch, dev):
    """The workload's inputs, generated on the GPU, as raw .npy files under path."""
    import numpy as np
    os.makedirs(path, exist_ok=True)
    t = {"x": S.gen_x(c, device=dev), "w_router": S.gen_router(c, device=dev),
         "bias": S.gen_bias(c, device=dev), **S.gen_experts(c, device=dev)}
    for k, v in t.items():
        v = v.cpu()
        if v.dtype == torch.bfloat16:
            v = v.view(torch.int16)
        np.save(os.path.join(path, k + ".npy"), v.numpy())
    with open(os.path.join(path, "workload.json"), "w") as f:
        json.dump({"workload": c.name, "T": c.T, "dtypes": {k: str(v.dtype) for k, v in t.items()}},
                  f)
    log(f"inputs of {c.name} written to {path}")


def load_inputs(path, c, torch, dev):
    """Inputs written by save_inputs, uploaded with plain host-to-device copies."""
    import numpy as np
    meta = json.load(open(os.path.join(path, "workload.json")))
    assert meta["workload"] == c.name and meta["T"] == c.T, (meta, c.name, c.T)
    out = {}
    for k, dt in meta["dtypes"].items():
        a = torch.from_numpy(np.load(os.path.join(path, k + ".npy")))
        if dt == "torch.bfloat16":
            a = a.view(torch.bfloat16)
        out[k] = a.to(dev)
    ex = {k: out[k] for k in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down") if k in out}
    return out["x"], out["w_router"], out["bias"], ex


def bench_forward(name, args, np, torch, moe, S, dev, primary):
    """Time moe_forward on one workload; returns the JSON line (primary) or its object."""
    c = S.get_config(name)
    cfg = moe.cfg_from(c)
    T = c.T
    log(f"workload {c.name}: T={T} H={c.hidden} I={c.inter} E={c.n_experts}+{c.n_shared} "
        f"K={c.topk} w={c.w_dtype}; " + ("reading inputs" if args.load_inputs and primary
                                         else "generating inputs on the GPU"))
    t0 = time.time()
    if args.load_inputs and primary:
        x, wr, b, ex = load_inputs(args.load_inputs, c, torch, dev)
    else:
        x = S.gen_x(c, device=dev)
        wr = S.gen_router(c, device=dev)
        b = S.gen_bias(c, device=dev)
        ex = S.gen_experts(c, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")
    y = torch.empty_like(x)
    out = moe.alloc_routing(cfg, T, dev)
    ws = moe.alloc_workspace(cfg, T, dev)

    stream = torch.cuda.current_stream()

    def timed_forward(xb, bb):
        """Warmup, then args.steps forwards timed with HIP events on the stream;
        then the same number again with the library's event pair around every
        launch, for the per-kernel durations (those events cost about 1.5% of
        a step, so the timed pass runs without them)."""
        for _ in range(args.warmup):
            moe.forward(cfg, xb, wr, bb, ex, y, ws, out=out, stream=stream)
        moe.profile_enable(False)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            moe.forward(cfg, xb, wr, bb, ex, y, ws, out=out, stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall1 = time.perf_counter()
        ms = ev0.elapsed_time(ev1) / args.steps
        moe.profile_read()           # clear
        moe.profile_enable(True)
        for _ in range(args.steps):
            moe.forward(cfg, xb, wr, bb, ex, y, ws, out=out, stream=stream)
        torch.cuda.synchronize()
        moe.profile_enable(False)
        kern = moe.profile_read()
        log(f"{name}: timed {args.steps} steps: {ms:.4f} ms/step "
            f"(wall {1e3 * (wall1 - wall0) / args.steps:.4f})")
        for k, (kms, n) in kern.items():
            if n:
                log(f"  {k:14s} {kms / n * 1e3:9.1f} us/launch  ({n} launches)")
        return ms, kern

    skew = None
    if c.name == "skew":
        # the loss-free bias loop: step st routes a fresh batch with the bias of
        # st earlier updates, then updates it from that batch's loads; the
        # forward is timed at checkpoint steps before their update
        checkpoints = sorted(set(min(v, args.skew_steps - 1) for v in (0, args.skew_steps // 2,
                                                                       args.skew_steps - 1)))
        ratios, at = [], {}
        wsr = moe.alloc_workspace(cfg, T, dev)
        outr = moe.alloc_routing(cfg, T, dev)
        for st in range(args.skew_steps):
            xs = S.gen_x(c, step=st, device=dev)
            if st in checkpoints:
                log(f"skew: step {st}")
                ms_c, kern_c = timed_forward(xs, b)
                at[st] = (ms_c, kern_c, out["counts"].clone(), b.clone())
            moe.route(cfg, xs, wr, b, outr, wsr)
            moe.bias_update(cfg, T, outr["counts"], b, c.gamma)
            cn = outr["counts"].cpu().numpy().astype(np.float64)
            ratios.append(float(cn.max() / cn.mean()))
        torch.cuda.synchronize()
        log(f"skew: {args.skew_steps} bias steps; max/mean load at step 0 {ratios[0]:.2f}, "
            f"step {args.skew_steps // 2} {ratios[args.skew_steps // 2]:.2f}, last {ratios[-1]:.2f}")
        # the reported figures are those of the last checkpoint (its batch and bias)
        ms_step, kern, counts_t, b = at[checkpoints[-1]]
        out["counts"].copy_(counts_t)
        x = S.gen_x(c, step=checkpoints[-1], device=dev)
        skew = {"steps": args.skew_steps, "gamma": c.gamma,
                "max_over_mean_load_per_step": [round(v, 3) for v in ratios],
                "checkpoints": {str(k): {"ms_per_step": round(v[0], 4),
                                         "tokens_per_s": round(T / (v[0] / 1e3), 1),
                                         "gemm_gate_up_us": round(
                                             v[1]["gemm_gate_up"][0] / v[1]["gemm_gate_up"][1] * 1e3, 1),
                                         "max_over_mean_load": round(ratios[k], 3)}
                                for k, v in at.items()}}
    else:
        ms_step, kern = timed_forward(x, b)

    counts = out["counts"].cpu().numpy().astype(np.int64)
    active = int((counts > 0).sum())
    H, I, E, K, Sn = c.hidden, c.inter, c.n_experts, c.topk, c.n_shared
    wbytes = {"bf16": 2, "e4m3": 1, "f32": 4}[c.w_dtype]
    abytes = {"bf16": 2, "f32": 4}[c.act_dtype]
    rows = T * K + Sn * T
    n_exp = active + Sn
    scale_bytes = (3 * (I // 128) * (H // 128) * 4) if c.w_dtype == "e4m3" else 0
    # algorithmic work of the layer: weights of every expert with rows, router, x and y
    layer_bytes = n_exp * (3 * H * I * wbytes + scale_bytes) + H * E * 4 + 2 * T * H * abytes
    layer_flops = rows * 2 * 3 * H * I + 2 * T * H * E
    # dominant kernel: gate/up grouped GEMM (two of the three expert matrices)
    gu_ms, gu_n = kern["gemm_gate_up"]
    gu_s = gu_ms / max(gu_n, 1) / 1e3
    if c.w_dtype == "e4m3":   # reads x and writes H as E4M3 codes with 1x128 scales
        gu_bytes = (n_exp * (2 * H * I * wbytes + 2 * scale_bytes // 3) + T * H + T * (H // 128) * 4
                    + rows * I + rows * (I // 128) * 4)
    else:
        gu_bytes = n_exp * (2 * H * I * wbytes + 2 * scale_bytes // 3) + T * H * abytes + rows * I * abytes
    gu_flops = rows * 2 * 2 * H * I
    if c.name == "decode" or c.name == "skew" or c.name == "fp8":
        bound, achieved, peak, unit = "hbm", gu_bytes / gu_s / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", gu_flops / gu_s / 1e12, MFMA_PEAK_TFLOPS[c.w_dtype], "TFLOP/s"
    traffic = measured_traffic(c.name)
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": "gemm_gate_up", "kernel_us": round(gu_s * 1e6, 2),
                "alg_bytes_per_launch": int(gu_bytes), "alg_flops_per_launch": int(gu_flops)}
    if bound == "mfma":
        roofline["mfma_counters"] = measured_mfma(c.name)
        roofline["library_gemm_reference"] = MATMUL_REFERENCE
    if c.w_dtype == "e4m3":   # the same kernel against the fp8 matrix cores
        roofline["mfma_frac_e4m3"] = round(gu_flops / gu_s / 1e12 / MFMA_PEAK_TFLOPS["e4m3"], 4)
        roofline["mfma_counters"] = measured_mfma(c.name)
    layer = {"ms": round(ms_step, 4), "alg_bytes": int(layer_bytes), "alg_flops": int(layer_flops),
             "hbm_frac": round(layer_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
             "mfma_frac": round(layer_flops / (ms_step / 1e3) / 1e12 /
                                MFMA_PEAK_TFLOPS[c.w_dtype], 4),
             "active_experts": active, "max_over_mean_load": round(float(counts.max() / counts.mean()), 3),
             "kernels_us": {k: round(ms / n * 1e3, 1) for k, (ms, n) in kern.items() if n}}

    value = T / (ms_step / 1e3)
    workload = (f"{c.name}: DeepSeek-V3 MoE layer forward, T={T}, hidden {H}, inter {I}, {E} routed "
                f"in {c.n_groups} groups (keep {c.topk_groups}) + {Sn} shared, top-{K}, "
                f"{c.w_dtype} weights")
    if not primary:
        obj = {"workload": workload, "T": T, "w_dtype": c.w_dtype, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
               "tokens_per_s": round(value, 1), "roofline": roofline, "layer": layer}
        if skew is not None:
            obj["skew"] = skew
        del x, y, ex, ws, out
        return obj
    bal = balance_loss_timing(moe, torch, cfg, c, x, wr, ws, dev)
    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline(c, args.cpu_tokens, x, b)
        if skew is not None:
            cpu["route_update_ms"] = cpu_route_update_ms(c, x, b)

    return {
        "metric": "MoE-layer tokens/s on 1 MI355X; MFMA util (prefill) / HBM GB/s (decode)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.w_dtype,
        "data": "synthetic (seeded SplitMix64 inputs, V3 layer shapes)",
        "config": {"workload": workload, "T": T, "hidden": H, "inter": I, "n_experts": E,
                   "n_shared": Sn, "topk": K, "w_dtype": c.w_dtype},
        "roofline": roofline,
        "layer": layer,
        "cpu_baseline": cpu,
        "balance_loss": bal,
        **({"skew": skew} if skew is not None else {}),
    }


def bench_backward(args, np, torch, moe, S):
    """Layer backward for one training step (moe_backward) on a V3-shape batch:
    tokens/s of the backward, and the roofline of its dominant kernel, the
    weight-gradient GEMMs (float32 gradients of all 257 experts' matrices)."""
    dev = torch.device("cuda:0")
    shape = S.get_config(args.backward_shape)
    f8 = args.backward_weights == "e4m3"
    # E4M3: the fp8 workload's inputs (outliers included) at the shape's batch size
    c = S.get_config("fp8", T=shape.T) if f8 else shape
    cfg = moe.cfg_from(c)
    T, H, I, E, K, Sn = c.T, c.hidden, c.inter, c.n_experts, c.topk, c.n_shared
    n = E + Sn
    wb = 1 if f8 else 2   # bytes per weight element
    log(f"backward on the {shape.name} batch, {c.w_dtype} weights: T={T}; generating inputs on "
        f"the GPU")
    x = S.gen_x(c, device=dev)
    wr = S.gen_router(c, device=dev)
    b = S.gen_bias(c, device=dev)
    ex = S.gen_experts(c, device=dev)
    g = torch.Generator().manual_seed(99)
    dy_cpu = torch.randn((T, H), generator=g).to(torch.bfloat16)
    dy = dy_cpu.to(dev)
    dx = torch.empty_like(x)
    dwr = torch.empty((H, E), dtype=torch.float32, device=dev)
    dwg = torch.empty((n, I, H), dtype=torch.float32, device=dev)
    dwu = torch.empty_like(dwg)
    dwd = torch.empty((n, H, I), dtype=torch.float32, device=dev)
    ws = moe.alloc_backward_workspace(cfg, T, dev)
    stream = torch.cuda.current_stream()

    def call():
        moe.backward(cfg, x, wr, b, ex, dy, dx, dwr, dwg, dwu, dwd, ws, stream=stream)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # timed without the library's per-launch events; then the same number of
    # calls with them, for the per-stage durations
    moe.profile_enable(False)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    moe.profile_read()
    moe.profile_enable(True)
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    moe.profile_enable(False)
    kern = moe.profile_read()
    log(f"timed {args.steps} backward steps: {ms:.4f} ms/step")
    for k, (kms, nn) in kern.items():
        if nn:
            log(f"  {k:18s} {kms / nn * 1e3:9.1f} us/call  ({nn} calls)")

    rows = T * K + Sn * T
    mfma_peak = MFMA_PEAK_TFLOPS["e4m3" if f8 else "bf16"]
    # weight-gradient GEMMs (dW_down, dW_gate, dW_up; two or three launches a
    # call): float32 gradients of every expert written once, each staged operand
    # read once (dY, H, dG, dU, X), wb bytes per element (E4M3: their 128x1 codes)
    wg_ms, wg_n = kern["bwd_wgrad"]
    wg_s = wg_ms / max(wg_n, 1) / 1e3
    wg_bytes = n * 3 * H * I * 4 + rows * (2 * H + 3 * I) * wb
    wg_flops = 3 * 2 * rows * H * I
    roofline = {"bound": "hbm", "achieved": round(wg_bytes / wg_s / 1e9, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(wg_bytes / wg_s / 1e9 / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(f"backward_{args.backward_shape}_{c.w_dtype}"),
                "kernel": "bwd_wgrad (dW_down, dW_gate, dW_up)",
                "kernel_us": round(wg_s * 1e6, 2), "alg_bytes_per_launch": int(wg_bytes),
                "alg_flops_per_launch": int(wg_flops),
                "mfma_frac": round(wg_flops / wg_s / 1e12 / mfma_peak, 4)}
    # the whole backward: expert recompute, dgrad and wgrad (3 x the forward's
    # expert flops) plus the router's; weights read twice, gradients written
    bw_flops = 3 * rows * 2 * 3 * H * I + 2 * T * K * H * 2
    bw_bytes = 2 * n * 3 * H * I * wb + n * 3 * H * I * 4 + 3 * T * H * 2 + 2 * H * E * 4
    backward = {"ms": round(ms, 4), "alg_bytes": int(bw_bytes), "alg_flops": int(bw_flops),
                "hbm_frac": round(bw_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                "mfma_frac": round(bw_flops / (ms / 1e3) / 1e12 / mfma_peak, 4),
                "weights": c.w_dtype,
                "kernels_us": {k: round(v / nn * 1e3, 1) for k, (v, nn) in kern.items() if nn}}
    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline_backward(c, min(args.cpu_tokens, 4), x, b, dy_cpu)
    res = {
        "metric": "MoE-layer backward tokens/s on 1 MI355X (one training step's layer gradients)",
        "value": round(T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": c.w_dtype,
        "data": "synthetic (seeded SplitMix64 inputs and upstream gradient, V3 layer shapes)",
        "config": {"workload": f"backward on the {shape.name} batch: DeepSeek-V3 MoE layer "
                               f"gradients (dx, dW_r, dW of 257 experts in float32), T={T}, hidden "
                               f"{H}, inter {I}, {E} routed + {Sn} shared, top-{K}, "
                               + ("E4M3 weights and GEMM operands" if f8 else "bf16"),
                   "T": T, "hidden": H, "inter": I, "n_experts": E, "n_shared": Sn, "topk": K},
        "roofline": roofline, "backward": backward, "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def cpu_baseline_backward(c, n_tok, x_dev, b_dev, dy_cpu):
    """The oracle's backward (float64, as it stands) on the first n_tok tokens
    of the batch as a batch of their own, with the weight gradients of every
    expert they touch and of the shared expert; input generation excluded."""
    import numpy as np
    import oracle as O
    import synthetic as S
    x = O.lift(x_dev[:n_tok].float().cpu())
    wr = O.lift(S.gen_router(c, "cpu"))
    b = b_dev.cpu().numpy()
    dy = O.lift(dy_cpu[:n_tok].float())
    L, s, r, p = O.route(x, wr, b, n_groups=c.n_groups, topk_groups=c.topk_groups, topk=c.topk,
                         group_topn=c.group_topn)
    touched = sorted(set(int(v) for v in r.idx.reshape(-1))) + list(range(c.n_experts, c.n_experts + c.n_shared))
    cache = {e: S.gen_expert(c, e, "cpu") for e in touched}
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    f8 = c.w_dtype == "e4m3"
    O.backward(x, wr, b, lambda e: cache[e], dy, n_groups=c.n_groups, topk_groups=c.topk_groups,
               topk=c.topk, group_topn=c.group_topn, n_shared=c.n_shared, grad_experts=touched,
               fp8_emulation=f8)
    dt = time.perf_counter() - t0
    log(f"cpu baseline: oracle backward of {n_tok} tokens ({len(touched)} experts' gradients) "
        f"in {dt:.1f}s on {cores} cores")
    return {"value": round(n_tok / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 oracle backward{' (E4M3 emulation)' if f8 else ''} of the first "
                      f"{n_tok} tokens as their own batch "
                      f"(dx, dW_r, and dW of the {len(touched)} experts they touch, shared included)",
            **host_info()}


def router_partials(T, H, E):
    """Number of float32 [T][E] router partials the library's bf16 router writes:
    K = 3H split into 128-aligned chunks of about H/8 for small batches; from
    2048 tokens the tiled router (128 x 256 tiles, K steps of 32) uses about
    256 workgroups' worth of chunks."""
    chunk = ((H + 7) // 8 + 127) // 128 * 128
    ks = (H + chunk - 1) // chunk
    if T < 2048:
        return ks
    tiles = ((T + 127) // 128) * ((E + 255) // 256)
    chunks = max(1, min(ks, 256 // tiles))
    nsteps = 3 * H // 32
    spc = (nsteps + chunks - 1) // chunks
    return (nsteps + spc - 1) // spc


def balance_loss_timing(moe, torch, cfg, c, x, wr, ws, dev, calls=5, alpha=1e-4):
    """Sequence-wise balance loss over the batch as one sequence (router + loss
    kernels), timed like the layer: HIP events per launch on the stream."""
    T, E, K = c.T, c.n_experts, c.topk
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    moe.balance_loss(cfg, x, wr, T, alpha, loss, ws)
    torch.cuda.synchronize()
    moe.profile_read()
    moe.profile_enable(True)
    for _ in range(calls):
        moe.balance_loss(cfg, x, wr, T, alpha, loss, ws)
    torch.cuda.synchronize()
    moe.profile_enable(False)
    kern = moe.profile_read()
    r_ms, r_n = kern["router_logits"]
    b_ms, b_n = kern["balance_loss"]
    b_s = b_ms / max(b_n, 1) / 1e3
    # loss kernels: router partials read, s / sum(s) written and read back, top-K ids
    ksplit = router_partials(T, c.hidden, E)
    b_bytes = ksplit * T * E * 4 + 2 * T * E * 4 + 2 * T * K * 4
    log(f"balance loss: router {r_ms / max(r_n, 1) * 1e3:.1f} us, loss kernels "
        f"{b_s * 1e6:.1f} us per call; loss/alpha {float(loss[0]) / alpha:.4f}")
    return {"seq_len": T, "alpha": alpha, "loss": float(loss[0]),
            "router_us": round(r_ms / max(r_n, 1) * 1e3, 1), "loss_kernels_us": round(b_s * 1e6, 1),
            "loss_kernels_gbs": round(b_bytes / b_s / 1e9, 1)}


def host_info():
    """BLAS threads numpy's matmuls use and the host CPU's model string."""
    try:
        from threadpoolctl import threadpool_info
        import numpy as np
        np.ones((2, 2)) @ np.ones((2, 2))  # load the BLAS
        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                   default=None)
    except Exception:
        blas = None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"blas_threads": blas, "cpu_model": model}


def cpu_route_update_ms(c, x_dev, b_dev):
    """The oracle's routing of one whole batch plus its bias update (one step of
    the loss-free balancing loop), in ms; input generation excluded."""
    import oracle as O
    import synthetic as S
    x64 = O.lift(x_dev.float().cpu())
    wr64 = O.lift(S.gen_router(c, "cpu"))
    b = b_dev.cpu().numpy()
    t0 = time.perf_counter()
    L, s, r, p = O.route(x64, wr64, b, n_groups=c.n_groups, topk_groups=c.topk_groups, topk=c.topk,
                         group_topn=c.group_topn)
    O.bias_update(b, p.counts, c.T, c.topk, c.gamma)
    ms = (time.perf_counter() - t0) * 1e3
    log(f"cpu baseline: oracle route + bias update of {c.T} tokens in {ms:.1f} ms")
    return round(ms, 2)


def cpu_baseline(c, n_tok, x_dev, b_dev):
    """The float64 oracle on the first n_tok tokens' outputs (routing covers the whole batch)."""
    import numpy as np
    import torch

    import oracle as O
    import synthetic as S

    x_cpu = x_dev.cpu()
    b = b_dev.cpu().numpy()
    x64 = O.lift(x_cpu)
    wr64 = O.lift(S.gen_router(c, "cpu"))
    tokens = list(range(n_tok))
    # inputs the oracle will need, generated before the clock starts
    L, s, r, p = O.route(x64, wr64, b, n_groups=c.n_groups, topk_groups=c.topk_groups, topk=c.topk,
                         group_topn=c.group_topn)
    need = sorted(set(int(e) for e in r.idx[tokens].reshape(-1))) + list(range(c.n_experts, c.n_experts + c.n_shared))
    log(f"cpu baseline: generating {len(need)} experts for {n_tok} tokens")
    weights = {e: S.gen_expert(c, e, "cpu") for e in need}
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                   default=1)
    except Exception:
        blas = None
    threads = max(blas or 1, torch.get_num_threads())
    log(f"cpu baseline: timing the oracle ({threads} threads)")
    t0 = time.perf_counter()
    O.forward(x64, wr64, b, lambda e: weights[e], n_groups=c.n_groups, topk_groups=c.topk_groups,
              topk=c.topk, group_topn=c.group_topn, n_shared=c.n_shared, tokens=tokens)
    dt = time.perf_counter() - t0
    log(f"cpu baseline: {dt:.1f}s")
    return {"value": round(n_tok / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 oracle forward: routing of all {c.T} tokens, expert outputs of the "
                      f"first {n_tok} tokens ({len(need)} experts' weights lifted to float64); "
                      f"input generation excluded; {dt:.1f}s",
            "host_cpus": len(os.sched_getaffinity(0)), **host_info()}


if __name__ == "__main__":
    main()
