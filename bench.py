"""Benchmark of the MI355X DeepSeekMoE layer forward (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|skew|fp8]

A step is one moe_forward call (router, node-limited top-8 selection, gates,
permutation, routed + shared SwiGLU experts, gated combine) over one batch of
synthetic V3-shaped input already resident in HBM.  Prints one JSON line.

The default workload is the decode batch (T=256, bf16 weights): the
configuration the headline metric is quoted on.  Kernel durations come from
HIP events recorded by the library around each launch on the same stream,
over the timed steps.  The CPU baseline is the float64 oracle timed on a
bounded sample of the same workload on this host's cores.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "e4m3": 5000.0, "f32": 157.3}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "skew", "fp8"])
    ap.add_argument("--skew-step", type=int, default=0,
                    help="skew workload: bias-update steps applied before timing")
    ap.add_argument("--cpu-tokens", type=int, default=12,
                    help="tokens in the CPU oracle sample (0 disables the CPU baseline)")
    ap.add_argument("--traffic", default=None,
                    help="JSON file with measured HBM bytes per launch of the dominant kernel")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is benchmarked on a single MI355X)", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_moe_layer_group_amd as moe
    import synthetic as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = S.get_config(args.workload)
    cfg = moe.cfg_from(c)
    T = c.T
    log(f"workload {c.name}: T={T} H={c.hidden} I={c.inter} E={c.n_experts}+{c.n_shared} "
        f"K={c.topk} w={c.w_dtype}; generating inputs on the GPU")
    t0 = time.time()
    x = S.gen_x(c, device=dev)
    wr = S.gen_router(c, device=dev)
    b = S.gen_bias(c, device=dev)
    ex = S.gen_experts(c, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")
    y = torch.empty_like(x)
    out = moe.alloc_routing(cfg, T, dev)
    ws = moe.alloc_workspace(cfg, T, dev)

    if c.name == "skew" and args.skew_step > 0:
        wsr = moe.alloc_workspace(cfg, T, dev)
        for st in range(args.skew_step):
            xs = S.gen_x(c, step=st, device=dev)
            moe.route(cfg, xs, wr, b, out, wsr)
            moe.bias_update(cfg, T, out["counts"], b, c.gamma)
        torch.cuda.synchronize()
        log(f"skew: applied {args.skew_step} bias steps")

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        moe.forward(cfg, x, wr, b, ex, y, ws, out=out, stream=stream)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    moe.profile_read()           # clear
    moe.profile_enable(True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        moe.forward(cfg, x, wr, b, ex, y, ws, out=out, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    moe.profile_enable(False)
    kern = moe.profile_read()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    log(f"timed {args.steps} steps: {ms_step:.4f} ms/step (wall {1e3 * (wall1 - wall0) / args.steps:.4f})")
    for k, (ms, n) in kern.items():
        if n:
            log(f"  {k:14s} {ms / n * 1e3:9.1f} us/launch  ({n} launches)")

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
    gu_bytes = n_exp * (2 * H * I * wbytes + 2 * scale_bytes // 3) + T * H * abytes + rows * I * abytes
    gu_flops = rows * 2 * 2 * H * I
    if c.name == "decode" or c.name == "skew" or c.name == "fp8":
        bound, achieved, peak, unit = "hbm", gu_bytes / gu_s / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", gu_flops / gu_s / 1e12, MFMA_PEAK_TFLOPS[c.w_dtype], "TFLOP/s"
    traffic = None
    if args.traffic and os.path.exists(args.traffic):
        tr = json.load(open(args.traffic)).get(c.name, {})
        traffic = tr.get("gemm_gate_up_bytes_per_launch")
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": "gemm_gate_up", "kernel_us": round(gu_s * 1e6, 2),
                "alg_bytes_per_launch": int(gu_bytes), "alg_flops_per_launch": int(gu_flops)}
    layer = {"ms": round(ms_step, 4), "alg_bytes": int(layer_bytes), "alg_flops": int(layer_flops),
             "hbm_frac": round(layer_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
             "mfma_frac": round(layer_flops / (ms_step / 1e3) / 1e12 /
                                MFMA_PEAK_TFLOPS[c.w_dtype], 4),
             "active_experts": active, "max_over_mean_load": round(float(counts.max() / counts.mean()), 3),
             "kernels_us": {k: round(ms / n * 1e3, 1) for k, (ms, n) in kern.items() if n}}

    value = T / (ms_step / 1e3)
    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline(c, args.cpu_tokens, x, b)

    res = {
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
        "config": {"workload": f"{c.name}: DeepSeek-V3 MoE layer forward, T={T}, hidden {H}, "
                               f"inter {I}, {E} routed in {c.n_groups} groups (keep "
                               f"{c.topk_groups}) + {Sn} shared, top-{K}, {c.w_dtype} weights",
                   "T": T, "hidden": H, "inter": I, "n_experts": E, "n_shared": Sn, "topk": K,
                   "w_dtype": c.w_dtype},
        "roofline": roofline,
        "layer": layer,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


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
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
