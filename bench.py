"""Benchmark of the fused selected-token log-probability path on one MI355X.

One step = one forward (rlk_linear_logp_fwd: active-row compaction, MFMA
logit tiles with per-chunk statistics, split fold + tree merge) plus one
backward (rlk_linear_logp_bwd: recomputed logits -> dz, grad_W, grad_h) over
one batch of synthetic inputs resident in HBM.  Default workload: the
Qwen3-8B-shaped LM head, T=4096 rows, H=4096, V=151936, 15% of rows
ignored (-100).

Prints ONE JSON line.  `value` is tokens/s (all T rows of the batch per
step).  `roofline` prices the kernel with the largest total time against the
bf16 MFMA peak, from algorithmic FLOPs (active rows) and that kernel's
average duration measured with HIP events around each of its launches in
the timed region.  `cpu_baseline` times the fp64 oracle on a bounded sample
of the same workload on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "linear_logp fwd+bwd tokens/s + MFMA % of bf16 peak at H=4096, V=151936"
PEAK_BF16 = 2.5e15  # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12   # MI355X HBM3E, B/s

WORKLOADS = {
    # name: (T, H, V, masked fraction, backward?, description)
    "qwen3_8b_fwd_bwd": (4096, 4096, 151936, 0.15, True,
                         "linear_logp fwd+bwd, Qwen3-8B-shaped LM head (T=4096, H=4096, V=151936, 15% rows ignored)"),
    "qwen3_8b_fwd": (4096, 4096, 151936, 0.15, False,
                     "linear_logp fwd, Qwen3-8B-shaped LM head (T=4096, H=4096, V=151936, 15% rows ignored)"),
    "qwen3_30b_a3b_fwd_bwd": (16384, 2048, 151936, 0.15, True,
                              "linear_logp fwd+bwd, Qwen3-30B-A3B-shaped LM head (T=16384, H=2048, V=151936, 15% rows ignored)"),
}

# Kernels that carry the operator's MFMA work, with their algorithmic FLOPs
# per step in units of 2*T_act*H*V (one contraction over the active rows):
# forward logits; backward recompute; grad_h and grad_W (one launch), spread
# over the kernel's launches in that step.
GEMM_KERNELS = {"fwd_tiles": 1, "dz_tiles": 1, "grad_tiles": 2}


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selected_token_lm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, digest):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp, rows, backward):
    import numpy as np
    import oracle

    T = inp.T
    sel = np.arange(rows)
    hs, ys, gs = inp.h[sel], inp.y[sel], inp.g[sel]
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle.forward(hs, inp.W, ys)
    if backward:
        oracle.backward(hs, inp.W, ys, gs)
    dt = time.perf_counter() - t0
    return {
        "value": rows / dt,
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"first {rows} of the {T} rows ({int((ys != -100).sum())} active) through the fp64 "
                  f"oracle's forward{' and backward' if backward else ''}, same W; {dt:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_fwd_bwd", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the operator is measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import selected_token_lm_amd as rlk
    import synth

    T, H, V, mask, do_bwd, desc = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(T, H, V, mask)
    h = torch.from_numpy(inp.h.view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(inp.W.view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.from_numpy(inp.y).to(dev)
    g = torch.from_numpy(inp.g).to(dev)
    T_act = inp.n_active
    ws_f = torch.empty(rlk.workspace_bytes(rlk.OP_FWD, T, H, V), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(rlk.workspace_bytes(rlk.OP_BWD, T, H, V), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    reserved0 = torch.cuda.memory_reserved()

    def step():
        logp, lse = rlk.linear_logp_fwd(h, W, y, ws=ws_f)
        if do_bwd:
            rlk.linear_logp_bwd(h, W, y, lse, g, ws=ws_b)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    rlk.profile_begin()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = rlk.profile_end()
    peak_reserved = torch.cuda.max_memory_reserved()

    ms_wall = (t1 - t0) * 1e3 / args.steps
    ms_ev = ev0.elapsed_time(ev1) / args.steps
    ms = max(ms_wall, ms_ev)
    flops_step = 2.0 * T_act * H * V * (4 if do_bwd else 1)

    digest = source_digest()
    kernels = {}
    per_step_flops = 2.0 * T_act * H * V
    for name, (n, tot) in sorted(kern.items(), key=lambda kv: -kv[1][1]):
        avg = tot / n
        d = {"launches_per_step": n / args.steps, "avg_ms": avg, "ms_per_step": tot / args.steps}
        if name in GEMM_KERNELS:
            d["flops_per_launch"] = GEMM_KERNELS[name] * per_step_flops / (n / args.steps)
            d["tflops"] = d["flops_per_launch"] / (avg * 1e-3) / 1e12
        kernels[name] = d
    dom = max((k for k in kernels if k in GEMM_KERNELS), key=lambda k: kernels[k]["ms_per_step"])
    dom_fl = kernels[dom]["flops_per_launch"]
    achieved = dom_fl / (kernels[dom]["avg_ms"] * 1e-3)
    roofline = {
        "bound": "mfma",
        "kernel": dom,
        "achieved": achieved / 1e12,
        "peak": PEAK_BF16 / 1e12,
        "unit": "TFLOP/s",
        "frac": achieved / PEAK_BF16,
        "traffic": traffic_for(dom, digest),
        "flops_per_launch": dom_fl,
        "avg_launch_ms": kernels[dom]["avg_ms"],
    }

    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "T": T, "H": H, "V": V, "active_rows": T_act,
                   "ignore_index": -100, "parallelism": "single GPU"},
        "mfma_frac_step": flops_step / (ms * 1e-3) / PEAK_BF16,
        "algorithmic_tflop_per_step": flops_step / 1e12,
        "roofline": roofline,
        "kernels": kernels,
        "workspace_bytes": int(ws_f.numel() + (ws_b.numel() if do_bwd else 0)),
        "peak_reserved_delta_mb": (peak_reserved - reserved0) / 2**20,
        "source_digest": digest,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline ({args.cpu_rows} rows)", file=sys.stderr, flush=True)
        del h, W, y, g, ws_f, ws_b
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows, do_bwd)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
