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
    "qwen3_8b_fwd_bwd_saved": (4096, 4096, 151936, 0.15, True,
                               "linear_logp fwd+bwd, save-logits variant (fp32 logits kept between the passes, "
                               "no recompute), Qwen3-8B-shaped LM head (T=4096, H=4096, V=151936, 15% rows ignored)"),
    "qwen3_8b_tp2_partials": (4096, 4096, 151936, 0.15, False,
                              "linear_logp forward as two vocabulary shards of 75968 rows on one GPU "
                              "(rlk_lse_partial x 2 + rlk_lse_merge), Qwen3-8B-shaped LM head"),
    "qwen3_30b_a3b_fwd_bwd": (16384, 2048, 151936, 0.15, True,
                              "linear_logp fwd+bwd, Qwen3-30B-A3B-shaped LM head (T=16384, H=2048, V=151936, 15% rows ignored)"),
    "qwen3_30b_a3b_tp2_share_fwd_bwd": (6827, 2048, 75968, 0.15, True,
                                        "linear_logp fwd+bwd at one GPU's share of a tensor-parallel (2-way) "
                                        "Qwen3-30B-A3B step: T=6827, H=2048, V=75968 (half the vocabulary), "
                                        "15% rows ignored"),
}

# Ragged re-batching of the Qwen3-8B-shaped forward: one step = the forward
# of each batch of rows drawn by synth.rebatch_plan, in its shuffled order.
REBATCH_WORKLOAD = "qwen3_8b_rebatch_fwd"
REBATCH_DESC = ("linear_logp fwd over ragged re-batchings of the Qwen3-8B-shaped rows (batches of 1, 7, 128, "
                "1000 and 8192 rows drawn from seeded permutations of the 4096, in shuffled order; H=4096, "
                "V=151936, 15% rows ignored)")

# Dense-product workloads (rlk_gemm_bf16_nt): name -> (M, N, K, description).
GEMM_WORKLOADS = {
    "gemm_lm_head": (3482, 151936, 4096,
                     "deterministic bf16 GEMM x W^T, the Qwen3-8B-shaped LM head at its 3482 active rows "
                     "(M=3482, N=151936, K=4096), fp32 out"),
    "gemm_8192": (8192, 8192, 8192, "deterministic bf16 GEMM, M=N=K=8192, fp32 out"),
    "gemm_lm_head_bf16": (3482, 151936, 4096,
                          "deterministic bf16 GEMM x W^T, the Qwen3-8B-shaped LM head at its 3482 active rows "
                          "(M=3482, N=151936, K=4096), bf16 out"),
    "gemm_8192_bf16": (8192, 8192, 8192, "deterministic bf16 GEMM, M=N=K=8192, bf16 out"),
}

# Kernels that carry the operator's MFMA work, with their algorithmic FLOPs
# per step in units of 2*T_act*H*V (one contraction over the active rows):
# forward logits; backward recompute; grad_h and grad_W (one launch), spread
# over the kernel's launches in that step.
GEMM_KERNELS = {"fwd_tiles": 1, "dz_tiles": 1, "grad_tiles": 2, "gemm_tiles": 1}


def _elf_sections(data):
    """{name: (address, bytes)} of the sections of a 64-bit little-endian ELF image."""
    import struct
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    sec = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize) for i in range(shnum)]
    names = data[sec[shstrndx][4]:sec[shstrndx][4] + sec[shstrndx][5]]
    return {names[s[0]:names.index(b"\0", s[0])].decode(): (s[3], data[s[4]:s[4] + s[5]]) for s in sec}


def _gfx950_code_objects(lib_path):
    """The gfx950 code objects (ELF images) inside the library's offload
    bundles, one per translation unit (the .hip_fatbin section holds the
    bundles one after another)."""
    import struct
    with open(lib_path, "rb") as f:
        section = _elf_sections(f.read())[".hip_fatbin"][1]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    assert section.startswith(magic), "uncompressed offload bundle expected"
    found, start = [], 0
    while start >= 0:
        bundle = section[start:]
        n, = struct.unpack_from("<Q", bundle, len(magic))
        pos = len(magic) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", bundle, pos)
            triple = bundle[pos + 24:pos + 24 + tlen].decode()
            pos += 24 + tlen
            if "gfx950" in triple:
                found.append(bundle[off:off + size])
        start = section.find(magic, start + len(magic))
    if not found:
        raise KeyError("gfx950")
    return found


def kernel_digest(kernel):
    """Digest of the machine code of the library's kernels named `kernel`
    (every template instance): it changes exactly when that kernel's code
    does, whatever else changes in the sources."""
    import struct
    import selected_token_lm_amd as rlk
    h = hashlib.sha256()
    found = []
    for co in _gfx950_code_objects(rlk.library_path):
        secs = _elf_sections(co)
        text_addr, text = secs[".text"]
        strtab = secs[".strtab"][1]
        symtab = secs[".symtab"][1]
        for i in range(0, len(symtab), 24):
            name_off, info, _, _, value, size = struct.unpack_from("<IBBHQQ", symtab, i)
            name = strtab[name_off:strtab.index(b"\0", name_off)].decode()
            if (info & 0xF) == 2 and size and f"{len(kernel)}{kernel}" in name:  # STT_FUNC, mangled name
                found.append((name, text[value - text_addr:value - text_addr + size]))
    for name, code in sorted(found):
        h.update(name.encode() + code)
    return h.hexdigest()[:16] if found else None


def traffic_for(kernel):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the kernel's current machine code; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_digest") != kernel_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


# Calibration of the HBM byte counters: a plain device copy of a known size
# (read COPY_BYTES, write COPY_BYTES per launch) run in the same process.
COPY_BYTES = 1 << 30
COPY_LAUNCHES = 4


def copy_calibration(dev):
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(COPY_LAUNCHES):
        torch.neg(src, out=dst)  # elementwise: reads and writes COPY_BYTES
    torch.cuda.synchronize()


def _short_name(full):
    """Kernel name without namespace, template arguments and signature
    (all template instances of one of the library's kernels share it)."""
    return full.split("(")[0].split("<")[0].split("::")[-1]


def _counter_means(csv_dir, counter, key=_short_name):
    """Mean of `counter` per dispatch for each kernel, grouped by key(full
    kernel name), over the rocprofv3 counter-collection CSVs under csv_dir
    (kernels whose key is None are left out)."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = key(r["Kernel_Name"])
                if name is None:
                    continue
                k = (name, r["Dispatch_Id"])
                per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {k: (sum(v) / len(v), len(v)) for k, v in out.items()}


# The calibration copy: torch.neg over COPY_BYTES (copy_calibration).  Only
# its own dispatches count: torch's other elementwise kernels (the fill that
# creates the source, for one) share its short name and move other byte
# counts.
CALIBRATION_KERNEL = "neg_kernel"


def _calibration_key(full):
    return "copy" if CALIBRATION_KERNEL in full else None


def traffic_from(run_dir, command, out_dir=None):
    """Writes <out_dir>/traffic_<kernel>.json (default: profiles/) for the GEMM kernels from two
    counter runs of `bench.py --steps 2 --warmup 1 --no-cpu-baseline
    --copy-calibration` (run_dir/fetch: --pmc FETCH_SIZE, run_dir/write:
    --pmc WRITE_SIZE; both in KiB per dispatch).  Each counter is scaled by
    what it reads for the calibration copy (COPY_BYTES each way)."""
    fetch = _counter_means(os.path.join(run_dir, "fetch"), "FETCH_SIZE")
    write = _counter_means(os.path.join(run_dir, "write"), "WRITE_SIZE")
    # the machine code the counters were taken on: the JSON line each
    # counter run printed (run_dir/fetch.log, run_dir/write.log)
    measured = []
    for log in ("fetch.log", "write.log"):
        with open(os.path.join(run_dir, log)) as f:
            lines = [ln for ln in f if ln.startswith("{")]
        if not lines:
            raise SystemExit(f"no bench JSON line in {os.path.join(run_dir, log)}")
        measured.append(json.loads(lines[-1]).get("kernel_digests", {}))
    if measured[0] != measured[1]:
        raise SystemExit("the FETCH_SIZE and WRITE_SIZE runs measured different builds")
    f_copy = _counter_means(os.path.join(run_dir, "fetch"), "FETCH_SIZE", _calibration_key)
    w_copy = _counter_means(os.path.join(run_dir, "write"), "WRITE_SIZE", _calibration_key)
    if "copy" not in f_copy or "copy" not in w_copy:
        raise SystemExit(f"no dispatch of the calibration copy ({CALIBRATION_KERNEL}) under {run_dir}")
    ck = f"torch.neg over {COPY_BYTES} bytes ({CALIBRATION_KERNEL}, {f_copy['copy'][1]} dispatches)"
    f_scale = COPY_BYTES / (f_copy["copy"][0] * 1024.0)
    w_scale = COPY_BYTES / (w_copy["copy"][0] * 1024.0)
    rows = []
    for k in GEMM_KERNELS:
        if k not in fetch or k not in write:
            continue
        fb = fetch[k][0] * 1024.0 * f_scale
        wb = write[k][0] * 1024.0 * w_scale
        if k not in measured[0]:
            continue
        if measured[0][k] != kernel_digest(k):
            print(f"{k}: the library has changed since these counters were taken; the record keeps the "
                  f"measured digest and bench.py will report no traffic for it", flush=True)
        rec = {"kernel": k, "kernel_digest": measured[0][k], "bytes_per_launch": fb + wb, "fetch_bytes": fb,
               "write_bytes": wb, "dispatches": fetch[k][1], "calibration_kernel": ck,
               "fetch_scale": f_scale, "write_scale": w_scale, "command": command}
        with open(os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"traffic_{k}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        rows.append(rec)
        print(f"{k}: fetch {fb / 1e9:.3f} GB, write {wb / 1e9:.3f} GB per launch", flush=True)
    print(f"calibration {ck}: fetch scale {f_scale:.4f}, write scale {w_scale:.4f}", flush=True)
    return rows


class ClockPowerSampler:
    """GFX clock and socket power of the benchmarked GPU, read through
    amdsmi on a helper thread every `period` seconds (the firmware refreshes
    them less often; repeats are kept).  Everything degrades to None where
    amdsmi is missing or refuses."""

    def __init__(self, torch, period=0.02):
        import threading
        self.period, self.samples, self.handle, self.smi = period, [], None, None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.smi = amdsmi
            bus = torch.cuda.get_device_properties(0).pci_bus_id
            for h in amdsmi.amdsmi_get_processor_handles():
                if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                    self.handle = h
        except Exception:  # no amdsmi, no permission: report nothing
            self.handle = None

    def _read(self):
        c = self.smi.amdsmi_get_clock_info(self.handle, self.smi.AmdSmiClkType.GFX)
        p = self.smi.amdsmi_get_power_info(self.handle)
        return c["clk"], c["max_clk"], p["current_socket_power"], p["power_limit"]

    def _loop(self):
        while not self._stop.wait(self.period):
            try:
                self.samples.append(self._read())
            except Exception:
                return

    def start(self):
        if self.handle is None:
            return
        import threading
        self._thread = threading.Thread(target=self._loop, daemon=True)
        self._thread.start()

    def stop(self, skip=0):
        if self._thread is None:
            return None
        self._stop.set()
        self._thread.join()
        try:
            self.smi.amdsmi_shut_down()
        except Exception:
            pass
        s = [x for x in self.samples[skip:] if all(isinstance(v, (int, float)) for v in x)]
        if not s:
            return None
        clk = sorted(x[0] for x in s)
        pw = sorted(x[2] for x in s)
        return {"gfx_clock_mhz": {"median": clk[len(clk) // 2], "min": clk[0], "max": clk[-1]},
                "max_gfx_clock_mhz": s[0][1],
                "socket_power_w": {"median": pw[len(pw) // 2], "max": pw[-1]},
                "power_limit_w": s[0][3] / 1e6,
                "samples": len(s)}


def clock_power_window(torch, step, seconds=2.5, settle=0.75):
    """Steady-state GFX clock and socket power under this workload: `step`
    repeated for `seconds` after the timed region (not part of any timing),
    sampled by ClockPowerSampler; samples of the first `settle` seconds
    (clock ramp, firmware refresh) are dropped."""
    sampler = ClockPowerSampler(torch)
    if sampler.handle is None:
        return None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sampler.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    n_settle = int(settle / sampler.period)
    res = sampler.stop(skip=n_settle)
    if res is not None:
        res["source"] = (f"amdsmi every {sampler.period * 1e3:.0f} ms while the step repeats for "
                         f"{seconds:.1f} s after the timed region (first {settle:.2f} s dropped)")
    return res


def rocminfo_agent(arch="gfx950"):
    """The first `arch` agent that rocminfo lists: its name, marketing name
    (empty on some systems), chip id and compute units; None without rocminfo."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception:  # no rocminfo on PATH, or it failed: report nothing
        return None
    for agent in txt.split("Agent ")[1:]:
        fields = {}
        for line in agent.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                fields.setdefault(k.strip(), v.strip())
        if fields.get("Name", "").startswith(arch):
            return {"name": fields.get("Name"), "marketing_name": fields.get("Marketing Name"),
                    "chip_id": fields.get("Chip ID"), "compute_units": fields.get("Compute Unit")}
    return None


def amdsmi_names(torch):
    """(market name, product name) of the benchmarked GPU from amdsmi, or Nones."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        try:
            bus = torch.cuda.get_device_properties(0).pci_bus_id
            for h in amdsmi.amdsmi_get_processor_handles():
                if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                    asic = amdsmi.amdsmi_get_gpu_asic_info(h)
                    board = amdsmi.amdsmi_get_gpu_board_info(h)
                    return asic.get("market_name"), board.get("product_name")
        finally:
            amdsmi.amdsmi_shut_down()
    except Exception:  # no amdsmi, no permission: report nothing
        pass
    return None, None


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    market, product = amdsmi_names(torch)
    # the clock and power under load come from ClockPowerSampler
    return {"name": p.name, "rocminfo": rocminfo_agent(), "amdsmi_market_name": market,
            "amdsmi_product_name": product, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count}


def host_cpu():
    """(CPU model, the cores this process may run on).  The model is cpuinfo's
    name of the first CPU with its family / model / stepping numbers (a
    virtual machine may report a bare vendor name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # end of the first CPU's record
                k, _, v = line.partition(":")
                fields.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    model = fields.get("model name")
    nums = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    if model and nums:
        model = f"{model} ({', '.join(nums)})"
    return model, len(os.sched_getaffinity(0))


def gemm_bench(args):
    """Times rlk_gemm_bf16_nt on resident synthetic operands (A ~ N(0,1),
    B ~ N(0, 1/sqrt(K))), with the vendor library's bf16 GEMM (torch.matmul,
    hipBLASLt) on the same operands timed after it as context."""
    import numpy as np
    import torch

    import selected_token_lm_amd as rlk
    import synth

    M, N, K, desc = GEMM_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    A_bits = synth.normal_bf16(synth.SEED_H, M, K)
    B_bits = synth.normal_bf16(synth.SEED_W, N, K, float(1.0 / np.sqrt(K)))
    A = torch.from_numpy(A_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    B = torch.from_numpy(B_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    flops = 2.0 * M * N * K

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return max(e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3) / steps

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    rlk.profile_begin()
    out_dtype = torch.bfloat16 if args.workload.endswith("_bf16") else torch.float32
    ms = timed(lambda: rlk.gemm_bf16_nt(A, B, out_dtype=out_dtype), args.steps, args.warmup)
    kern = rlk.profile_end()
    clock_power = None if args.no_clock_power else clock_power_window(
        torch, lambda: rlk.gemm_bf16_nt(A, B, out_dtype=out_dtype))
    n, tot = kern["gemm_tiles"]
    k_ms = tot / n
    Bt = B.t()
    vendor_ms = timed(lambda: torch.matmul(A, Bt), args.steps, args.warmup)
    achieved = flops / (k_ms * 1e-3)
    out = {
        "metric": "deterministic bf16 GEMM TFLOP/s (rlk_gemm_bf16_nt)",
        "value": flops / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "M": M, "N": N, "K": K},
        "clock_power": clock_power,
        "roofline": {"bound": "mfma", "kernel": "gemm_tiles", "achieved": achieved / 1e12,
                     "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16,
                     "traffic": traffic_for("gemm_tiles"), "flops_per_launch": flops,
                     "avg_launch_ms": k_ms},
        "context": {"vendor_bf16_gemm": "torch.matmul (hipBLASLt), same operands, not deterministic by contract",
                    "vendor_ms": vendor_ms, "vendor_tflops": flops / (vendor_ms * 1e-3) / 1e12},
        "kernel_digest": kernel_digest("gemm_tiles"),
    }
    print(json.dumps(out), flush=True)


def rebatch_bench(args):
    """Times the forward over the ragged batches of synth.rebatch_plan: one
    step runs every batch once (rows gathered ahead, resident in HBM);
    reports rows/s over the step and the median latency per batch size."""
    import numpy as np
    import torch

    import selected_token_lm_amd as rlk
    import synth

    T, H, V, mask = synth.CONFIGS["qwen3_8b"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(T, H, V, mask)
    h = torch.from_numpy(inp.h.view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(inp.W.view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.from_numpy(inp.y).to(dev)
    plan = synth.rebatch_plan(T)
    batches = []
    for rows in plan:
        r = torch.from_numpy(rows).to(dev)
        hb, yb = h.index_select(0, r).contiguous(), y.index_select(0, r).contiguous()
        ws = torch.empty(rlk.workspace_bytes(rlk.OP_FWD, len(rows), H, V), dtype=torch.uint8, device=dev)
        batches.append((len(rows), int((inp.y[rows] != -100).sum()), hb, yb, ws))
    rows_step = sum(b[0] for b in batches)
    act_step = sum(b[1] for b in batches)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(batches) + 1)] for _ in range(args.steps)]

    def step(k=None):
        for j, (_, _, hb, yb, ws) in enumerate(batches):
            if k is not None:
                ev[k][j].record(stream)
            rlk.linear_logp_fwd(hb, W, yb, ws=ws)
        if k is not None:
            ev[k][len(batches)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    rlk.profile_begin()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = rlk.profile_end()
    clock_power = None if args.no_clock_power else clock_power_window(torch, step)
    ms_ev = sum(ev[k][0].elapsed_time(ev[k][-1]) for k in range(args.steps)) / args.steps
    ms = max(ms_ev, (t1 - t0) * 1e3 / args.steps)
    lat = {}
    for j, b in enumerate(batches):
        v = sorted(ev[k][j].elapsed_time(ev[k][j + 1]) for k in range(args.steps))
        lat[str(b[0])] = {"active_rows": b[1], "median_ms": v[len(v) // 2], "min_ms": v[0]}
    n, tot = kern["fwd_tiles"]
    k_ms = tot / n
    fl = 2.0 * act_step * H * V / (n / args.steps)  # algorithmic FLOPs per fwd_tiles launch, averaged
    out = {
        "metric": f"{args.workload}: tokens/s",
        "value": rows_step / (ms * 1e-3),
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
        "config": {"workload": REBATCH_DESC, "rows_per_step": rows_step, "active_rows_per_step": act_step,
                   "H": H, "V": V, "batches": [b[0] for b in batches], "parallelism": "single GPU"},
        "batch_latency_ms": lat,
        "clock_power": clock_power,
        "mfma_frac_step": 2.0 * act_step * H * V / (ms * 1e-3) / PEAK_BF16,
        "roofline": {"bound": "mfma", "kernel": "fwd_tiles", "achieved": fl / (k_ms * 1e-3) / 1e12,
                     "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": fl / (k_ms * 1e-3) / PEAK_BF16,
                     "traffic": None, "flops_per_launch": fl, "avg_launch_ms": k_ms},
        "kernels": {name: {"launches_per_step": c / args.steps, "avg_ms": t / c} for name, (c, t) in kern.items()},
        "kernel_digest": kernel_digest("fwd_tiles"),
    }
    print(json.dumps(out), flush=True)


def _oracle_sample(inp, rows, backward):
    """Times the fp64 oracle on the first `rows` rows of a workload (same W);
    returns (seconds, logp, grad_h) of the sample."""
    import numpy as np
    import oracle

    sel = np.arange(rows)
    hs, ys, gs = inp.h[sel], inp.y[sel], inp.g[sel]
    t0 = time.perf_counter()
    logp, _ = oracle.forward(hs, inp.W, ys)
    gh = oracle.backward(hs, inp.W, ys, gs, want_grad_W=True)[0] if backward else None
    return time.perf_counter() - t0, logp, gh


def cpu_baseline(inp, rows, backward, gpu_logp=None, gpu_grad_h=None, other_configs=True):
    """The fp64 oracle as it stands, on the host cores (all of this process's
    CPU affinity, BLAS threads set to that count), on bounded samples: the
    first `rows` rows of the benchmarked workload, and when `other_configs`
    the Qwen3-8B-shaped forward and the Qwen3-30B-A3B-shaped forward +
    backward on their first `rows` rows.  A reported baseline, not a target.
    Also compares the GPU's outputs on the sample rows with the oracle's."""
    import contextlib

    import numpy as np

    import synth

    model, cores = host_cpu()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limiter = contextlib.nullcontext()
    with limiter:
        dt, logp, gh = _oracle_sample(inp, rows, backward)
        act = int((inp.y[:rows] != -100).sum())
        res = {
            "value": rows / dt,
            "unit": "tokens/s",
            "cores": int(cores),
            "cpu_model": model,
            "kind": "oracle",
            "sample": f"first {rows} of the {inp.T} rows ({act} active) through the fp64 oracle's "
                      f"forward{' and backward (grad_h and the sample rows full grad_W)' if backward else ''}, "
                      f"same W; {dt:.1f} s",
            "seconds": dt,
        }
        if gpu_logp is not None:
            res["parity_on_sample"] = {"max_abs_dlogp": float(np.max(np.abs(gpu_logp[:rows] - logp)))}
            if gh is not None and gpu_grad_h is not None:
                a = inp.y[:rows] != -100
                d = gpu_grad_h[:rows][a] - gh[a]
                res["parity_on_sample"]["grad_h_rel_l2"] = float(np.linalg.norm(d) / np.linalg.norm(gh[a]))
        if other_configs:
            others = {}
            for name, bwd in (("qwen3_8b", False), ("qwen3_30b_a3b", True)):
                T, H, V, mask = synth.CONFIGS[name]
                if (T, H, V) == (inp.T, inp.H, inp.V) and bwd == backward:
                    continue
                sub = synth.Inputs(name, rows, H, V, synth.normal_bf16(synth.SEED_H, rows, H),
                                   inp.W if (H, V) == (inp.H, inp.V) else
                                   synth.normal_bf16(synth.SEED_W, V, H, float(np.float32(1.0 / np.sqrt(H)))),
                                   synth.targets(T, V, mask)[:rows], synth.upstream_grad(T)[:rows], mask)
                t, _, _ = _oracle_sample(sub, rows, bwd)
                others[f"{name}_{'fwd_bwd' if bwd else 'fwd'}"] = {
                    "value": rows / t, "unit": "tokens/s", "seconds": t,
                    "sample": f"first {rows} of the {T} rows (T={T}, H={H}, V={V}, "
                              f"{int((sub.y != -100).sum())} active), forward{' and backward' if bwd else ''}"}
            res["other_configs"] = others
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_fwd_bwd",
                    choices=sorted(WORKLOADS) + sorted(GEMM_WORKLOADS) + [REBATCH_WORKLOAD])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--no-cpu-other-configs", action="store_true",
                    help="time the oracle on the benchmarked workload's sample only")
    ap.add_argument("--no-clock-power", action="store_true",
                    help="skip the extra steps that sample the GFX clock and socket power (use under a profiler)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run plain copies of a known size (HBM counter calibration)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="no GPU: turn the FETCH_SIZE / WRITE_SIZE counter runs under DIR into profiles/traffic_*.json")
    ap.add_argument("--traffic-command", default="", help="command recorded with --traffic-from")
    ap.add_argument("--rows", type=int, default=None,
                    help="override the workload's row count T (throughput against batch size; "
                         "not the headline configuration)")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from, args.traffic_command)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the operator is measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import selected_token_lm_amd as rlk
    import synth

    if args.rows is not None and (args.workload in GEMM_WORKLOADS or args.workload == REBATCH_WORKLOAD
                                  or args.rows < 1):
        print("--rows takes a positive row count and applies to the linear_logp workloads only",
              file=sys.stderr)
        sys.exit(2)
    if args.workload in GEMM_WORKLOADS:
        gemm_bench(args)
        return
    if args.workload == REBATCH_WORKLOAD:
        rebatch_bench(args)
        return

    T, H, V, mask, do_bwd, desc = WORKLOADS[args.workload]
    if args.rows is not None:
        desc = desc.replace(f"T={T},", f"T={args.rows},") + f" [rows overridden: T={args.rows}]"
        T = args.rows
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(T, H, V, mask)
    h = torch.from_numpy(inp.h.view(np.int16)).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(inp.W.view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.from_numpy(inp.y).to(dev)
    g = torch.from_numpy(inp.g).to(dev)
    T_act = inp.n_active
    # memory around the operator: everything it needs beyond its resident
    # inputs (workspaces, outputs, the saved logits of the save-logits
    # variant) counts, as in the pages' "peak reserved delta" of a call
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    reserved0 = torch.cuda.memory_reserved()
    ws_f = torch.empty(rlk.workspace_bytes(rlk.OP_FWD, T, H, V), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(rlk.workspace_bytes(rlk.OP_BWD, T, H, V), dtype=torch.uint8, device=dev)

    saved = args.workload.endswith("_saved")
    zsave = torch.empty((T, rlk.saved_logits_ld(V)), dtype=torch.float32, device=dev) if saved else None
    sharded = args.workload.endswith("_tp2_partials")
    half = V // 2
    if sharded:
        W_sh = [W[:half].contiguous(), W[half:].contiguous()]
        parts = torch.empty((2, T, 4), dtype=torch.float32, device=dev)

    def step(keep=None):
        """One step; `keep` (a dict) receives its logp and grad_h."""
        gh = None
        if sharded:
            for r in range(2):
                rlk.lse_partial(h, W_sh[r], y, r * half, V, ws=ws_f, out=parts[r])
            logp, _ = rlk.lse_merge(parts, y)
        elif saved:
            logp, lse, _ = rlk.linear_logp_fwd_save(h, W, y, ws=ws_f, zsave=zsave)
            gh, _ = rlk.linear_logp_bwd_saved(h, W, y, lse, g, zsave, ws=ws_b)
        else:
            logp, lse = rlk.linear_logp_fwd(h, W, y, ws=ws_f)
            if do_bwd:
                gh, _ = rlk.linear_logp_bwd(h, W, y, lse, g, ws=ws_b)
        if keep is not None:
            keep["logp"], keep["grad_h"] = logp, gh

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    peak_reserved = torch.cuda.max_memory_reserved()

    stream = torch.cuda.current_stream()

    def timed_pass(profile):
        """K steps between synchronisations; per-step HIP events on the stream;
        with `profile` every library launch is also bracketed by HIP events."""
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        if profile:
            rlk.profile_begin()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for k in range(args.steps):
            step_ev[k].record(stream)
            step()
        step_ev[args.steps].record(stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kern = rlk.profile_end() if profile else None
        per = sorted(step_ev[k].elapsed_time(step_ev[k + 1]) for k in range(args.steps))
        return max((t1 - t0) * 1e3 / args.steps, ev0.elapsed_time(ev1) / args.steps), per, kern

    # headline: library timing off; then the same K steps with every launch
    # timed by HIP events on its stream, for the per-kernel figures
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ms, per_step, _ = timed_pass(False)
    print(f"[bench] timing {args.steps} steps with per-kernel events", file=sys.stderr, flush=True)
    ms_prof, _, kern = timed_pass(True)
    clock_power = None if args.no_clock_power or args.copy_calibration else clock_power_window(torch, step)
    if args.copy_calibration:
        copy_calibration(dev)
    # the part's MFMA ceiling on this machine right now (pure MFMA, random
    # operands, no memory traffic): context for the roofline fraction
    ceiling = rlk.bench_mfma_ceiling()

    # algorithmic contractions per step: forward, recompute (not in the
    # save-logits variant), grad_W, grad_h
    flops_step = 2.0 * T_act * H * V * ((3 if saved else 4) if do_bwd else 1)

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
        "traffic": traffic_for(dom),
        "flops_per_launch": dom_fl,
        "avg_launch_ms": kernels[dom]["avg_ms"],
    }
    if roofline["traffic"]:
        # diagnostic beside the MFMA bound: the dominant kernel's measured HBM
        # bytes per launch over its launch time, against the HBM3E peak
        roofline["traffic_gbps"] = roofline["traffic"] / (kernels[dom]["avg_ms"] * 1e-3) / 1e9
        roofline["traffic_frac_of_hbm_peak"] = roofline["traffic_gbps"] * 1e9 / PEAK_HBM

    out = {
        "metric": (METRIC if args.workload == "qwen3_8b_fwd_bwd" and args.rows is None
                   else f"{args.workload}{'' if args.rows is None else f' at T={T}'}: tokens/s"),
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
        "active_tokens_per_s": T_act / (ms * 1e-3),
        "ms_per_step_kernel_timing_pass": ms_prof,
        "step_ms_median_p10_p90": [per_step[len(per_step) // 2], per_step[len(per_step) // 10],
                                   per_step[min(len(per_step) - 1, (9 * len(per_step)) // 10)]],
        "device": device_info(torch),
        "clock_power": clock_power,
        "mfma_frac_step": flops_step / (ms * 1e-3) / PEAK_BF16,
        "algorithmic_tflop_per_step": flops_step / 1e12,
        "roofline": roofline,
        "kernels": kernels,
        "peak_at_measured_clock": None if not clock_power else {
            "what": "the 2.5 PFLOP/s bf16 peak scaled by the median GFX clock under this workload over the "
                    "2.4 GHz it assumes (clock_power)",
            "tflops": PEAK_BF16 / 1e12 * clock_power["gfx_clock_mhz"]["median"] / 2400.0,
            "dominant_kernel_frac": achieved / (PEAK_BF16 * clock_power["gfx_clock_mhz"]["median"] / 2400.0)},
        "mfma_ceiling": {"what": "pure loop of the tile engine's MFMA instruction on random bf16 operands, eight waves "
                                 "per compute unit with the tile kernels' 64 x 128 wave tile, no memory traffic, "
                                 "same box after the timed steps (rlk_bench_mfma_ceiling)",
                         "best_tflops": ceiling["best_tflops"], "median_tflops": ceiling["median_tflops"],
                         "dominant_kernel_frac_of_ceiling": achieved / 1e12 / ceiling["median_tflops"]},
        "workspace_bytes": int(ws_f.numel() + (ws_b.numel() if do_bwd else 0)
                               + (zsave.numel() * 4 if saved else 0)),
        "workspace_bytes_fwd_bwd": [int(ws_f.numel()), int(ws_b.numel()) if do_bwd else 0],
        "dz_budget_mb_env": os.environ.get("RLK_DZ_BUDGET_MB"),
        "peak_reserved_delta_mb": (peak_reserved - reserved0) / 2**20,
        "peak_reserved_delta_what": "torch max_memory_reserved after the warmup steps minus memory_reserved "
                                    "before the workspaces were allocated: workspaces, outputs (logp, lse, "
                                    "grad_h, grad_W) and saved logits, the inputs being resident before",
        "kernel_digest": kernel_digest(dom),
        "kernel_digests": {k: kernel_digest(k) for k in GEMM_KERNELS if k in kernels},
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline ({args.cpu_rows} rows)", file=sys.stderr, flush=True)
        last = {}
        step(last)
        gpu_logp = last["logp"].cpu().numpy().astype(np.float64)
        gpu_gh = last["grad_h"].float().cpu().numpy() if last["grad_h"] is not None else None
        del h, W, y, g, ws_f, ws_b, last
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows, do_bwd, gpu_logp, gpu_gh,
                                           other_configs=not args.no_cpu_other_configs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
