#!/usr/bin/env python3
"""One-GPU benchmark of the block-quantized matmul path on MI355X.

Main line (the JSON `value`): the Qwen3-0.6B-shaped linear set of one layer
for a 4096-token prefill, MXFP8 weights and activations.  q/k/v read the
same hidden state and gate/up the same MLP input, as in the model, so a step
is four groups -- qkv (1024 -> 2048 + 1024 + 1024), o (2048 -> 1024),
gate_up (1024 -> 3072 + 3072), down (3072 -> 1024) -- each one dynamic
per-32 MXFP8 quantization of the group's BF16 input (rq_quantize) and one
block-scaled GEMM (rq_gemm, BF16 output) against the members' weights,
quantized once and stacked along N.  value = GEMM FLOP per step (128.85
GFLOP, all seven linears) / wall time per step, in TFLOP/s, inputs resident
in HBM.

`roofline` covers the dominant kernel (the exact MXFP8 GEMM, which runs on
BF16 MFMAs, so its peak is the BF16 one): algorithmic FLOP (2 M N K per
launch) over its average launch time, from HIP events around back-to-back
launches of each of the step's four GEMMs on the same inputs, averaged over
the four; `traffic` is the HBM bytes per launch from the committed counter
summary (write it with --traffic-from).  The same GEMMs on the FP8 scaled
instruction and both paths' distance from the oracle are reported beside
it.  `rows` measures the other steps of the path on their own workloads:
single MXFP4 GEMM (128 x 1024 x 1024), 4096^3 MXFP4 plain / ARC (K' =
4224) / BF16, the exact MXFP8 GEMM's K sweep, quantization bandwidth, the
recurrent prefill (8 steps, RAMP vs all-BF16; 32 steps with 24 in MXFP8)
and the nibble GEMV (LM head, the 28-layer sweep grouped and in layer
order, escalation, gate).  `cpu_baseline` times the CPU oracle on a bounded
sample of the main workload.

Every figure is timed after at least 50 ms of sustained calls of the same
work: after an idle spell the GPU runs about 10% slower for its first
25-30 ms.  The main line's timed steps come right after its per-launch
figures and the W warm-up steps.

    python bench.py [--steps K] [--warmup W] [--no-rows] [--no-cpu-baseline]
    python bench.py --only square|gemv|ksweep   # one group of rows, for profiling
    python bench.py --traffic-from gpurun_out   # after the --pmc runs

"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"mxfp4": 10.1e15, "mxfp8": 5.0e15, "bf16": 2.5e15, "hbm": 8.0e12}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_mxfp8_qwen3_linear_set.json")
GEMM_SRCS = [os.path.join(ROOT, "mixed_precision_block_amd", "csrc", f) for f in ("gemm.hip", "gemm_pipe.hip", "rq_cvt.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the main GEMM from the committed counter
    summary, or None when the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256_16") != source_hash(GEMM_SRCS):
        return None
    return t.get("hbm_bytes_per_launch")


class Timer:
    """HIP events on torch's current stream (where librq launches)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def total_ms(self):
        self.torch.cuda.synchronize()
        return sum(s.elapsed_time(e) for s, e in self.pairs)


WARM_MS = 50.0  # sustained work before a timing: the clocks settle within about 30 ms


def warm_clocks(torch, fns, before=None, ms=WARM_MS):
    """Calls fns round-robin (each after `before` when given) until `ms` of
    wall time has passed, in batches that double up to about 2 ms, so the
    GPU has left the lower clocks it drops to while idle (about 10% slower
    over the first 25-30 ms of work) before anything is timed."""
    n, spent = 1, 0.0
    while spent < ms:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            for fn in fns:
                if before:
                    before()
                fn()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) * 1e3
        spent += dt
        if dt < 2.0:
            n *= 2


def time_calls(torch, fn, iters, warmup=10, before=None, batches=5, graph=False):
    """Per-call milliseconds of fn().  Without `before`: the median over
    `batches` batches of iters back-to-back calls, each batch bracketed by
    one pair of events.  Eager calls are device time only while the host
    issues them faster than the GPU runs them (about 7 us per library call
    from Python); for shorter kernels graph=True captures the iters calls
    once in a HIP graph and times its replays.  With `before`: events
    bracket each call, the untimed `before` work runs in between, and the
    mean is returned."""
    warm_clocks(torch, [fn], before)
    for _ in range(warmup):
        if before:
            before()
        fn()
    if before is None:
        if graph:
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(iters):
                    fn()
            g.replay()
            run = g.replay
        else:
            def run():
                for _ in range(iters):
                    fn()
        per = []
        for _ in range(batches):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / iters)
        return sorted(per)[len(per) // 2]
    tm = Timer(torch)
    for _ in range(iters):
        before()
        s = tm.start()
        fn()
        tm.stop(s)
    return tm.total_ms() / iters


def time_interleaved(torch, fns, iters, warmup=10, batches=9):
    """Per-call milliseconds of each function in fns, for comparisons whose
    difference is a few percent: batches of iters back-to-back calls (one
    pair of events per batch) alternate between the functions, so drifts of
    the clock (which follows power on random operands) reach them alike;
    the median over each function's batches."""
    warm_clocks(torch, fns)
    for fn in fns:
        for _ in range(warmup):
            fn()
    per = [[] for _ in fns]
    for _ in range(batches):
        for i, fn in enumerate(fns):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            per[i].append(e0.elapsed_time(e1) / iters)
    return [sorted(p)[len(p) // 2] for p in per]


COPY_BYTES = 256 << 20


def write_traffic(pmc_dir):
    """HBM bytes per launch of the main-line GEMM from FETCH_SIZE /
    WRITE_SIZE counter runs (KiB per dispatch), each scaled by what the same
    counter reads for a plain device copy of COPY_BYTES."""
    import csv
    from synthetic import workloads as W

    def per_dispatch(run, counter):
        path = os.path.join(pmc_dir, f"pmc_{run}_{counter}", "p_counter_collection.csv")
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]))
            out[key] = out.get(key, 0.0) + float(r["Counter_Value"]) * 1024  # KiB summed over instances
        return out

    scale = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        copies = [v for (d, name, g), v in per_dispatch("copy", counter).items() if "copy" in name.lower()]
        copy_kib = sorted(copies)[len(copies) // 2]
        scale[counter] = COPY_BYTES / copy_kib
    grids = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        for (d, name, g), v in per_dispatch("main", counter).items():
            # the main line's exact MXFP8 GEMMs with BF16 output (template
            # arguments <2, 0, ...>); the run also holds the FP8-instruction
            # and FP32-output launches of the bench's other figures
            if "gemm_pipe_kernel<2, 0," not in name:
                continue
            tmpl = name[name.index("<") + 1:name.index(">")]
            e = grids.setdefault((tmpl, g), {"grid_threads": g, "template": tmpl, "dispatches": 0, "FETCH_SIZE": 0.0,
                                             "WRITE_SIZE": 0.0})
            e[counter] += v * scale[counter]
            if counter == "FETCH_SIZE":
                e["dispatches"] += 1
    per_grid = []
    for g, e in sorted(grids.items()):
        n = e["dispatches"]
        per_grid.append({"template": e["template"], "grid_threads": e["grid_threads"], "dispatches": n,
                         "read_bytes": round(e["FETCH_SIZE"] / n), "write_bytes": round(e["WRITE_SIZE"] / n)})
    total = sum((e["read_bytes"] + e["write_bytes"]) * e["dispatches"] for e in per_grid)
    nd = sum(e["dispatches"] for e in per_grid)
    M = 4096
    alg = [M * g["a"].shape[1] * 33 // 32 + g["w"].shape[0] * g["a"].shape[1] * 33 // 32 + M * g["w"].shape[0] * 2
           for g in W.c2_layer(M=M)]
    summary = {"kernel": "gemm_pipe_kernel<MXFP8 exact, BF16 out>",
               "workload": "qwen3-0.6b linear set of one layer, 4096 tokens, MXFP8, four GEMMs per step",
               "gemm_source_sha256_16": source_hash(GEMM_SRCS),
               "hbm_bytes_per_launch": round(total / nd),
               "algorithmic_bytes_per_launch": round(sum(alg) / len(alg)),
               "fetch_scale": scale["FETCH_SIZE"], "write_scale": scale["WRITE_SIZE"], "per_grid": per_grid}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(summary, f, indent=1)
    print(json.dumps(summary, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain 256 MiB device copies (the reference for HBM byte counters)")
    ap.add_argument("--only", choices=["square", "gemv", "ksweep", "probes"],
                    help="run only one group of rows (4096^3 GEMMs and the ARC front end, the nibble GEMV "
                         "kernels without the escalation gate, the exact MXFP8 GEMM's K sweep, or the "
                         "hardware probes of libprobe.so: matrix-instruction rate and shader clock on "
                         "constant and random operands, dequantization against BF16 MFMAs) "
                         "and print them; for profiling runs")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="write the traffic summary from rocprofv3 --pmc CSV runs under DIR (pmc_main_FETCH_SIZE, "
                         "pmc_main_WRITE_SIZE, pmc_copy_FETCH_SIZE, pmc_copy_WRITE_SIZE) and exit (no GPU needed)")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (no multi-GPU path is built).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixed_precision_block_amd import api
    from mixed_precision_block_amd import _lib as L
    from synthetic import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.only:
        to_dev_only = (lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev))
        if args.only == "square":
            out = measure_square(torch, api, L, W, to_dev_only, dev)
        elif args.only == "probes":
            out = {"hardware_probes": measure_probes(torch, np, dev)}
        elif args.only == "ksweep":
            out = {"mxfp8_exact_gemm_k_sweep_4096x4096": measure_ksweep(torch, np, api, L, W, to_dev_only, dev)}
        else:
            out = measure_gemv(torch, np, api, L, W, dev, gate=False)
        print(json.dumps(out), flush=True)
        return
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel(), "copies": 5}), flush=True)
        return

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    # ------------------------------------------------------ main workload --
    log("generating the Qwen3-0.6B linear set of one layer at 4096 tokens (seeded)")
    M = 4096
    groups = []
    for g in W.c2_layer(M=M):
        K, N = g["a"].shape[1], g["w"].shape[0]
        wq = api.quantize(to_dev(g["w"]), L.RQ_MXFP8)  # weights: quantized once (per row: stacking commutes)
        groups.append(dict(name=g["name"], K=K, N=N, a=to_dev(g["a"]), wc=wq[0], ws=wq[1],
                           ac=torch.empty((M, K), dtype=torch.uint8, device=dev),
                           as_=torch.empty((M, K // 32), dtype=torch.uint8, device=dev),
                           y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    flops_step = sum(2.0 * M * g["K"] * g["N"] for g in groups)

    def step():
        for g in groups:
            L.rq_quantize(g["a"], M, g["K"], L.RQ_MXFP8, None, 0, L.RQ_APPEND_NONE, g["ac"], g["as_"])
            L.rq_gemm(L.RQ_MXFP8, g["ac"], g["as_"], g["wc"], g["ws"], M, g["N"], g["K"], L.RQ_OUT_BF16, g["y"])

    step()  # the quantized inputs that the per-launch figures run on
    # the GEMM's average launch duration: each of the step's GEMMs launched
    # back to back between one pair of events (events around every launch
    # would add their own packets to the measured time), averaged over them
    per_gemm, per_quant = {}, {}
    for g in groups:
        ms_g = time_calls(torch, lambda g=g: L.rq_gemm(L.RQ_MXFP8, g["ac"], g["as_"], g["wc"], g["ws"], M, g["N"],
                                                      g["K"], L.RQ_OUT_BF16, g["y"]), max(args.steps, 20),
                          graph=True)
        f_g = 2.0 * M * g["N"] * g["K"]
        per_gemm[f"{g['name']} {M}x{g['N']}x{g['K']}"] = {
            "us": round(ms_g * 1e3, 2), "tflops": round(f_g / (ms_g * 1e-3) / 1e12, 1),
            "frac_mxfp8_peak": round(f_g / (ms_g * 1e-3) / PEAK["mxfp8"], 4)}
        ms_q = time_calls(torch, lambda g=g: L.rq_quantize(g["a"], M, g["K"], L.RQ_MXFP8, None, 0,
                                                          L.RQ_APPEND_NONE, g["ac"], g["as_"]), max(args.steps, 20),
                          graph=True)
        qb = M * g["K"] * (2 + 1) + M * g["K"] // 32
        per_quant[f"{g['name']} input {M}x{g['K']}"] = {
            "us": round(ms_q * 1e3, 2), "gb_s": round(qb / (ms_q * 1e-3) / 1e9, 1),
            "frac_hbm": round(qb / (ms_q * 1e-3) / PEAK["hbm"], 4)}
    # the same codes on the FP8 scaled instruction (RQ_MXFP8_F8MFMA): faster,
    # but it truncates products inside runs of 8 (about 4e-5 relative)
    per_gemm_f8 = {}
    for g in groups:
        ms_g = time_calls(torch, lambda g=g: L.rq_gemm(L.RQ_MXFP8_F8MFMA, g["ac"], g["as_"], g["wc"], g["ws"], M,
                                                      g["N"], g["K"], L.RQ_OUT_BF16, g["y"]), max(args.steps, 20),
                          graph=True)
        f_g = 2.0 * M * g["N"] * g["K"]
        per_gemm_f8[f"{g['name']} {M}x{g['N']}x{g['K']}"] = {
            "us": round(ms_g * 1e3, 2), "tflops": round(f_g / (ms_g * 1e-3) / 1e12, 1),
            "frac_mxfp8_peak": round(f_g / (ms_g * 1e-3) / PEAK["mxfp8"], 4)}
    # The step's own timing follows the per-launch figures above, whose
    # ~100 ms of sustained work has brought the clocks up from where they
    # sit while the GPU is idle (otherwise the first ~30 ms run about 10%
    # slower, and a short warm-up would leave the timed steps inside that).
    for _ in range(args.warmup):
        step()
    # timed region: the steps alone, wall clock between synchronizations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # FP32 outputs of the first rows, for the accuracy check in the oracle leg
    acc_rows = 256
    gpu_f32 = {}
    for g in groups:
        for fmt, tag in ((L.RQ_MXFP8, "exact"), (L.RQ_MXFP8_F8MFMA, "f8mfma")):
            y32 = torch.empty((M, g["N"]), dtype=torch.float32, device=dev)
            L.rq_gemm(fmt, g["ac"], g["as_"], g["wc"], g["ws"], M, g["N"], g["K"], L.RQ_OUT_F32, y32)
            gpu_f32[(g["name"], tag)] = y32[:acc_rows].cpu().numpy()
            del y32
    gemm_ms = sum(v["us"] for v in per_gemm.values()) / 1e3 / len(groups)
    achieved = flops_step / len(groups) / (gemm_ms * 1e-3)
    log(f"main: {ms_step:.3f} ms/step, GEMM avg launch {gemm_ms * 1e3:.1f} us")
    value = flops_step / (ms_step * 1e-3) / 1e12
    traffic = measured_traffic()

    line = {
        "metric": "MXFP4/MXFP8 GEMM TFLOPS & % MFMA peak; nibble-GEMV GB/s & % HBM peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 codes, bf16 mfma, fp32 accumulation",
        "data": "synthetic (seeded, shapes and distributions of the Qwen3-0.6B linear set)",
        "config": {"workload": "qwen3-0.6b linear set of one layer (q,k,v,o,gate,up,down), 4096-token prefill, "
                               "MXFP8 W/A, dynamic per-32 activation quantization + block-scaled GEMM; "
                               "q/k/v and gate/up share their inputs and run as one GEMM each",
                   "tokens": M, "gemm_gflop_per_step": round(flops_step / 1e9, 2),
                   "gemms_per_step": [f"{g['name']} {M}x{g['N']}x{g['K']}" for g in groups]},
        # the exact MXFP8 GEMM runs its contraction on the BF16 matrix
        # instruction (codes dequantized in registers), so its peak is the
        # BF16 one; the MXFP8 (FP8 instruction) peak is given beside it
        "roofline": {"bound": "mfma", "kernel": "gemm_pipe_kernel<MXFP8 exact, BF16 out> (256x256 tiles for qkv, "
                               "256x192 for gate_up, 128x128 for o and down)",
                     "achieved": round(achieved / 1e12, 2), "peak": PEAK["bf16"] / 1e12, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK["bf16"], 4), "traffic": traffic,
                     "frac_of_mxfp8_peak": round(achieved / PEAK["mxfp8"], 4),
                     "avg_launch_us": round(gemm_ms * 1e3, 2), "per_gemm": per_gemm,
                     "per_gemm_fp8_instruction": per_gemm_f8},
        "quantize_per_input": per_quant,
    }
    for g in groups:
        del g["ac"], g["as_"], g["y"], g["a"]
    if not args.no_rows:
        line["rows"] = measure_rows(torch, np, api, L, W, to_dev, dev)
        line["hardware_ceilings"] = hardware_ceilings(measure_probes(torch, np, dev))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(np, W, gpu_f32, acc_rows)
        line["accuracy_rel_frobenius"] = line["cpu_baseline"].pop("accuracy")
    print(json.dumps(line), flush=True)


def measure_probes(torch, np, dev, blocks=512, seed=20261204):
    """Matrix-instruction and conversion probes (probes/probes.hip, built as
    libprobe.so): eight independent instructions per loop iteration per
    wave, two waves per SIMD, on operands loaded once.  For each kind the
    sustained rate, its fraction of the datasheet peak, the shader clock
    (shader cycle counter over the 100 MHz real-time counter, median over
    workgroups) and the SIMD's shader cycles per matrix instruction (event
    time x that clock / instructions per SIMD; for the conversions alone,
    per conversion)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mixed_precision_block_amd", "libprobe.so"))
    lib.rqp_probe.restype = ctypes.c_int
    lib.rqp_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    rng = np.random.default_rng(seed)
    n = blocks * 256

    def fp8_codes(size):  # random E4M3FN codes, NaN (0x7F / 0xFF) excluded
        c = rng.integers(0, 256, size, dtype=np.uint32)
        return np.where((c & 0x7F) == 0x7F, c ^ 1, c)

    def pack8(b):  # uint32 bytes [n, 12, 4] -> dwords [n, 12]
        b = b.astype(np.uint32)
        return b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)

    ops = {
        "fp4_constant": np.full((n, 12), 0x22222222, np.uint32),           # every E2M1 code 1.0
        "fp4_random": rng.integers(0, 2 ** 32, (n, 12), dtype=np.uint64).astype(np.uint32),
        "fp8_constant": np.full((n, 12), 0x38383838, np.uint32),           # every E4M3 code 1.0
        "fp8_random": pack8(fp8_codes((n, 12, 4))),
        "bf16_constant": np.full((n, 12), 0x3F803F80, np.uint32),          # every BF16 value 1.0
    }
    g = rng.standard_normal((n, 12, 2)).astype(np.float32).view(np.uint32) >> 16  # N(0, 1) in BF16
    ops["bf16_random"] = (g[..., 0] | (g[..., 1] << 16)).astype(np.uint32)
    ops["fp8_random_dequant"] = ops["fp8_random"]
    # kind, operands, FLOP per instruction, peak, iterations
    runs = [("fp4_constant", 0, 131072, PEAK["mxfp4"], 40000), ("fp4_random", 0, 131072, PEAK["mxfp4"], 40000),
            ("fp8_constant", 1, 131072, PEAK["mxfp8"], 20000), ("fp8_random", 1, 131072, PEAK["mxfp8"], 20000),
            ("bf16_constant", 2, 32768, PEAK["bf16"], 40000), ("bf16_random", 2, 32768, PEAK["bf16"], 40000),
            ("bf16_random_fed_by_24_fp8_dequant_per_8", 3, 32768, PEAK["bf16"], 40000),
            ("fp8_dequant_24_per_iteration_alone", 4, 0, None, 40000)]
    scales = torch.from_numpy(np.full(n, 0x7F7F, np.uint32).view(np.int32)).to(dev)  # both scales 1.0
    out = torch.empty(n, dtype=torch.float32, device=dev)
    stamps = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for name, kind, flop, peak, iters in runs:
        key = "fp8_random" if kind in (3, 4) else name
        o = torch.from_numpy(ops[key].view(np.int32).copy()).to(dev)

        def call():
            rc = lib.rqp_probe(kind, o.data_ptr(), scales.data_ptr(), blocks, iters, out.data_ptr(),
                               stamps.data_ptr(), st)
            if rc:
                raise RuntimeError(f"rqp_probe({kind}) returned {rc}")
        call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        t = stamps.cpu().numpy().view(np.uint64).reshape(blocks, 4).astype(np.float64)
        clk = (t[:, 2] - t[:, 0]) / np.maximum(t[:, 3] - t[:, 1], 1.0) * 100e6
        ghz = float(np.median(clk)) / 1e9
        per_simd = iters * (8 if flop else 24) * blocks * 4 / 1024  # instructions of one SIMD
        r = {"ms": round(ms, 3), "shader_clock_ghz": round(ghz, 3),
             ("shader_cycles_per_instruction" if flop else "shader_cycles_per_conversion"):
                 round(ms * 1e-3 * ghz * 1e9 / per_simd, 1)}
        if flop:
            rate = blocks * 4 * iters * 8 * flop / (ms * 1e-3)
            r.update({"tflops": round(rate / 1e12, 1), "frac_peak": round(rate / peak, 4)})
        res[name] = r
        del o
    res.update(measure_stream_and_launch_probes(torch, lib, dev))
    res["setup"] = (f"{blocks} workgroups of 4 waves (2 waves per SIMD), eight independent matrix instructions "
                    "per iteration (FP4 / FP8: v_mfma_scale_f32_32x32x64_f8f6f4 with both scales 1.0; BF16: "
                    "v_mfma_f32_32x32x16_bf16); the dequant kinds add 24 v_cvt_scalef32_pk_bf16_fp8 per iteration "
                    "(the ratio of the exact MXFP8 GEMM's 128 x 64 wave tiles)")
    return res


def hardware_ceilings(p):
    """The probes' figures that bound this line's fractions: the matrix
    instructions' sustained rate on random operands (the clock drops on
    random bits), the BF16 instruction fed by the exact MXFP8 path's
    dequantization, streaming rates and launch costs."""
    return {
        "mfma_random_operands_frac_of_peak": {k: p[f"{k}_random"]["frac_peak"] for k in ("fp4", "fp8", "bf16")},
        "mfma_random_shader_clock_ghz": {k: p[f"{k}_random"]["shader_clock_ghz"] for k in ("fp4", "fp8", "bf16")},
        "bf16_mfma_fed_by_fp8_dequant_frac_of_bf16_peak": p["bf16_random_fed_by_24_fp8_dequant_per_8"]["frac_peak"],
        "l2_to_lds_tb_s": p["stream_l2_private_two_64k_stages"]["tb_s"],
        "hbm_to_lds_tb_s": p["stream_hbm_two_64k_stages"]["tb_s"],
        "launch_us": {"empty": p["launch_empty_kernel"]["us_per_launch"],
                      "arrival_64_tiles_16_slices": p["launch_arrival_counter_64_tiles_16_slices_one_counter_per_128b"]
                      ["us_per_launch"]},
        "source": "bench.py --only probes (mixed_precision_block_amd/probes/probes.hip)"}


def measure_stream_and_launch_probes(torch, lib, dev):
    """L2 -> LDS streaming the way the pipelined GEMM loads (rqp_stream: one
    512-thread workgroup per CU, buffer-to-LDS loads into a ring of stages,
    one wait and barrier per stage, no compute), from data resident in each
    XCD's L2 (shared windows read in step by an XCD's 32 CUs, or a private
    64 KiB window per CU; the dispatcher deals workgroups round-robin over
    the 8 XCDs) and from HBM (each workgroup its own 4 MiB window of
    1 GiB); and the per-launch cost of back-to-back
    launches in a captured HIP graph (rqp_launch: an empty kernel, one that
    reads and writes 2 MiB, arrival launches of 1 and 64 tiles whose 16
    workgroups each meet at a device-scope counter, as the split-K GEMV's
    do)."""
    import ctypes
    import numpy as np
    lib.rqp_stream.restype = ctypes.c_int
    lib.rqp_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                               ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.rqp_launch.restype = ctypes.c_int
    lib.rqp_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    res = {}
    blocks = 256
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    stamps = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    kinds = {0: ("two_64k_stages", 2, 65536), 1: ("three_32k_stages", 3, 32768), 2: ("four_32k_stages", 4, 32768)}
    # l2_shared: the 32 workgroups of an XCD read one 2 MiB window in step
    # (each line read by all of them); l2_private: each workgroup streams its
    # own 64 KiB window (2 MiB per XCD, each line read by one CU); hbm: each
    # workgroup its own 4 MiB window of 1 GiB
    for where, win, nwin, stages in (("l2_shared", 2 << 20, 8, 4000), ("l2_private", 64 << 10, 256, 4000),
                                     ("hbm", 4 << 20, 256, 1000)):
        for kind, (name, nstg, sb) in kinds.items():
            n_st = stages * 65536 // sb

            def call():
                rc = lib.rqp_stream(kind, src.data_ptr(), src.numel(), win, nwin, blocks, n_st, out.data_ptr(),
                                    stamps.data_ptr(), st)
                if rc:
                    raise RuntimeError(f"rqp_stream({kind}) returned {rc}")
            call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            t = stamps.cpu().numpy().view(np.uint64).reshape(blocks, 4).astype(np.float64)
            ghz = float(np.median((t[:, 2] - t[:, 0]) / np.maximum(t[:, 3] - t[:, 1], 1.0))) * 0.1
            nbytes = blocks * (n_st + nstg - 1) * sb
            res[f"stream_{where}_{name}"] = {
                "ms": round(ms, 3), "tb_s": round(nbytes / (ms * 1e-3) / 1e12, 2), "shader_clock_ghz": round(ghz, 3),
                "bytes_per_clk_per_cu": round(nbytes / (ms * 1e-3) / (ghz * 1e9) / 256, 1)}
    del src
    x = torch.ones(1 << 19, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    tiles = 64
    part = torch.empty(tiles * 16 * 256, dtype=torch.float32, device=dev)
    counter = torch.zeros(tiles * 32, dtype=torch.int32, device=dev)
    ysum = torch.empty(tiles * 256, dtype=torch.float32, device=dev)
    p3 = (part.data_ptr(), counter.data_ptr(), ysum.data_ptr())
    # counters 4 bytes apart (64 tiles' counters in two 128-byte lines) or
    # one per 128-byte line
    launches = {"empty_kernel": (0, 1, 1, 1, 0, 0, 0), "touch_2mib": (1, 2048, 1, 1, x.data_ptr(), y.data_ptr(), 0),
                "arrival_counter_1_tile_16_slices": (2, 1, 16, 1, *p3),
                "arrival_counter_64_tiles_16_slices_packed_counters": (2, tiles, 16, 1, *p3),
                "arrival_counter_64_tiles_16_slices_one_counter_per_128b": (2, tiles, 16, 32, *p3)}
    n = 200
    for name, (kind, nb, sl, cs, a, b, c) in launches.items():
        def one():
            rc = lib.rqp_launch(kind, nb, sl, cs, a, b, c, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc:
                raise RuntimeError(f"rqp_launch({kind}) returned {rc}")
        one()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                one()
        g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / n)
        res[f"launch_{name}"] = {"us_per_launch": round(sorted(per)[2], 2), "launches_per_graph": n}
        del g
    # LDS reads: 1, 2 and 4 waves per SIMD (one, two and four 256-thread
    # workgroups per CU)
    lib.rqp_lds.restype = ctypes.c_int
    lib.rqp_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    for per_cu in (1, 2, 4):
        nb = 256 * per_cu
        lo = torch.empty(nb * 256, dtype=torch.float32, device=dev)
        st_l = torch.zeros(nb * 4, dtype=torch.int64, device=dev)
        iters = 20000

        def lds_call():
            rc = lib.rqp_lds(nb, iters, lo.data_ptr(), st_l.data_ptr(),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc:
                raise RuntimeError(f"rqp_lds returned {rc}")
        lds_call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lds_call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        t = st_l.cpu().numpy().view(np.uint64).reshape(nb, 4).astype(np.float64)
        ghz = float(np.median((t[:, 2] - t[:, 0]) / np.maximum(t[:, 3] - t[:, 1], 1.0))) * 0.1
        nbytes = nb * 256 * iters * 8 * 16
        res[f"lds_read_{per_cu}_waves_per_simd"] = {
            "ms": round(ms, 3), "shader_clock_ghz": round(ghz, 3),
            "bytes_per_clk_per_cu": round(nbytes / (ms * 1e-3) / (ghz * 1e9) / 256, 1)}
    if float(ysum[1].item()) != 16.0 or float(ysum[(tiles - 1) * 256 + 3].item()) != 48.0:
        raise RuntimeError("arrival probe: the last workgroup's sum is wrong")
    return res


def measure_rows(torch, np, api, L, W, to_dev, dev):
    rows = {}

    def tflops(flop, ms):
        return flop / (ms * 1e-3) / 1e12

    # ---- single MXFP4 GEMM, 128 x 1024 x 1024 (launch/latency bound)
    d = W.c1_gemm_mxfp4()
    ac, as_ = api.quantize(to_dev(d["a"]), L.RQ_MXFP4)
    wc, ws = api.quantize(to_dev(d["w"]), L.RQ_MXFP4)
    y = torch.empty((128, 1024), dtype=torch.bfloat16, device=dev)
    ms = time_calls(torch, lambda: L.rq_gemm(L.RQ_MXFP4, ac, as_, wc, ws, 128, 1024, 1024, 0, y), 200, graph=True)
    f = 2.0 * 128 * 1024 * 1024
    rows["single_mxfp4_gemm_128x1024x1024"] = {"us": round(ms * 1e3, 2), "tflops": round(tflops(f, ms), 2),
                                               "frac_mxfp4_peak": round(tflops(f, ms) * 1e12 / PEAK["mxfp4"], 5)}
    a1, w1 = to_dev(d["a"]), to_dev(d["w"])
    for name, x1, r1 in (("a_128x1024", a1, 128), ("w_1024x1024", w1, 1024)):
        c1, s1 = api.quantize(x1, L.RQ_MXFP4)
        ms_q = time_calls(torch, lambda: L.rq_quantize(x1, r1, 1024, L.RQ_MXFP4, None, 0, 0, c1, s1), 100,
                          graph=True)
        qb = r1 * 1024 * 2 + r1 * 512 + r1 * 32
        rows[f"single_mxfp4_quantize_{name}"] = {"us": round(ms_q * 1e3, 2),
                                                 "gb_s": round(qb / (ms_q * 1e-3) / 1e9, 1), "bytes": qb}
    log(f"rows: config-1 {ms * 1e3:.1f} us")

    # ---- 4096^3: plain MXFP4, ARC (K' = 4224), BF16; quantization bandwidth; ARC front end
    rows.update(measure_square(torch, api, L, W, to_dev, dev))
    rows["mxfp8_exact_gemm_k_sweep_4096x4096"] = measure_ksweep(torch, np, api, L, W, to_dev, dev)

    # ---- recurrent prefill, 4096 x 2048, FFN 5632, 8 steps
    rows.update(measure_ramp(torch, api, L, W, to_dev, dev, time_calls))
    rows["recurrent_prefill_schedule_study"] = measure_ramp_study(torch, np, api, L, W, to_dev, dev, time_calls)

    # ---- nibble GEMV: weights drawn on the GPU with the same recipe
    rows.update(measure_gemv(torch, np, api, L, W, dev))

    # ---- FP8 KV tiles: one 4096-token prefill's keys, 8 heads of 128
    rows["kv_quantize_fp8_tile128_4096x8x128"] = measure_kv(torch, L, dev)
    return rows


def measure_kv(torch, L, dev, T=4096, H=8, D=128):
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261209)
    x = torch.randn((T, H, D), generator=gen, device=dev).to(torch.bfloat16)
    codes = torch.empty((T, H, D), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, H, D // 128), dtype=torch.float32, device=dev)
    ms = time_calls(torch, lambda: L.rq_kv_quantize(x, T, H, D, codes, scales), 100, graph=True)
    nbytes = T * H * D * 3 + T * H * (D // 128) * 4
    return {"us": round(ms * 1e3, 2), "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / PEAK["hbm"], 4), "bytes": nbytes}


def measure_square(torch, api, L, W, to_dev, dev):
    """Config 3 at 4096^3: plain MXFP4, ARC (K' = 4224) and BF16 GEMMs, the
    MXFP4 quantization bandwidth and the ARC fused front end."""
    rows = {}

    def tflops(flop, ms):
        return flop / (ms * 1e-3) / 1e12

    d = W.c3_arc()
    a = to_dev(d["a"])
    w = to_dev(d["w"])
    n = 4096
    f = 2.0 * n ** 3
    pc, ps = api.quantize(a, L.RQ_MXFP4)
    qc, qs = api.quantize(w, L.RQ_MXFP4)
    y = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    ms_plain = time_calls(torch, lambda: L.rq_gemm(L.RQ_MXFP4, pc, ps, qc, qs, n, n, n, 0, y), 50)
    ms_q = time_calls(torch, lambda: L.rq_quantize(a, n, n, L.RQ_MXFP4, None, 0, 0, pc, ps), 50, graph=True)
    idx = api.select_channels(api.channel_amax(a), 128).to(dev)
    w_aug = api.quantize(w, L.RQ_MXFP4, idx, L.RQ_APPEND_COPY)
    ws_bytes = L.rq_gemm_arc_workspace_bytes(n, n, 128)
    wsp = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    # ARC against the plain path timed alike: each call launches a
    # quantization and a GEMM back to back (rq_gemm_arc: the one-pass
    # residual quantization into the workspace, then the GEMM over K + S),
    # in interleaved batches
    def plain_pair():
        L.rq_quantize(a, n, n, L.RQ_MXFP4, None, 0, 0, pc, ps)
        L.rq_gemm(L.RQ_MXFP4, pc, ps, qc, qs, n, n, n, 0, y)
    ms_arc, ms_pair = time_interleaved(
        torch, [lambda: L.rq_gemm_arc(a, n, n, idx, 128, w_aug[0], w_aug[1], n, wsp, ws_bytes, 0, y), plain_pair], 50)
    ms_bf = time_calls(torch, lambda: L.rq_gemm(L.RQ_BF16, a, None, w, None, n, n, n, 0, y), 20)
    qbytes = n * n * 2 + n * n // 2 + n * n // 32
    f_arc = 2.0 * n * n * (n + 128)
    rows["mxfp4_gemm_4096cubed"] = {"us": round(ms_plain * 1e3, 1), "tflops": round(tflops(f, ms_plain), 1),
                                    "frac_mxfp4_peak": round(tflops(f, ms_plain) * 1e12 / PEAK["mxfp4"], 4)}
    rows["arc_gemm_4096cubed_kprime4224"] = {
        "us_quant_plus_gemm": round(ms_arc * 1e3, 1), "tflops_gemm_flop": round(tflops(f_arc, ms_arc), 1),
        "us_plain_quant_plus_gemm": round(ms_pair * 1e3, 1),
        "overhead_vs_plain_quant_plus_gemm": round(ms_arc / ms_pair - 1, 4)}
    rows["bf16_gemm_4096cubed"] = {"us": round(ms_bf * 1e3, 1), "tflops": round(tflops(f, ms_bf), 1),
                                   "frac_bf16_peak": round(tflops(f, ms_bf) * 1e12 / PEAK["bf16"], 4)}
    rows["quantize_mxfp4_4096x4096"] = {"us": round(ms_q * 1e3, 2), "gb_s": round(qbytes / (ms_q * 1e-3) / 1e9, 1),
                                        "frac_hbm": round(qbytes / (ms_q * 1e-3) / PEAK["hbm"], 4)}
    log(f"rows: 4096^3 plain {ms_plain * 1e3:.1f} us, ARC {ms_arc * 1e3:.1f} us, BF16 {ms_bf * 1e3:.1f} us, "
        f"quant {ms_q * 1e3:.1f} us")
    rows["arc_front_end_4096x4096_s128"] = measure_front_end(torch, api, L, a, w, qc, qs, dev, time_calls)
    del a, w, pc, ps, qc, qs, y, w_aug, wsp

    return rows


def measure_ksweep(torch, np, api, L, W, to_dev, dev):
    """The exact MXFP8 GEMM at 4096 x 4096 x K for K = 1024 .. 8192 (the qkv
    group's seeded operands repeated along K), and the least-squares line
    t = fixed + K / rate through the four times: the per-launch cost that
    does not grow with K (pipeline fill, the output write, launch) and the
    steady-state rate of the K loop."""
    g = W.c2_layer(M=4096)[0]
    a0, w0 = g["a"], g["w"]
    M, N = a0.shape[0], w0.shape[0]
    ks, ts, out = [], [], {}
    for rep in (1, 2, 4, 8):
        K = a0.shape[1] * rep
        a = to_dev(np.tile(a0, (1, rep)))
        w = to_dev(np.tile(w0, (1, rep)))
        ac, as_ = api.quantize(a, L.RQ_MXFP8)
        wc, ws = api.quantize(w, L.RQ_MXFP8)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ms = time_calls(torch, lambda: L.rq_gemm(L.RQ_MXFP8, ac, as_, wc, ws, M, N, K, 0, y), 20)
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out[f"k{K}"] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                        "frac_bf16_peak": round(tf * 1e12 / PEAK["bf16"], 4)}
        ks.append(K)
        ts.append(ms * 1e3)
        del a, w, ac, as_, wc, ws, y
    slope, fixed = np.polyfit(np.array(ks, float), np.array(ts, float), 1)
    rate = 2.0 * M * N / (slope * 1e-6) / 1e12  # TFLOP/s of the K loop
    out["fit"] = {"fixed_us": round(float(fixed), 1), "steady_tflops": round(float(rate), 1),
                  "steady_frac_bf16_peak": round(float(rate) * 1e12 / PEAK["bf16"], 4)}
    log(f"rows: exact MXFP8 K sweep {[round(t, 1) for t in ts]} us, fixed {fixed:.1f} us, steady {rate:.0f} TF")
    return out


def measure_front_end(torch, api, L, a, w, qc, qs, dev, time_calls):
    """The ARC fused front end on config 3's activations read as the hidden
    state before RMSNorm: channel order calibrated on the normalized rows;
    the fused pass (RMSNorm + reorder + primary + residual) against RMSNorm
    followed by the gather-form quantize, alone and with the GEMM over
    K + S; errors of fused ARC, gather ARC and plain MXFP4 against the BF16
    product of the normalized rows."""
    n, S = a.shape[0], 128
    Kp = n + S
    nb = torch.empty_like(a)
    L.rq_rmsnorm(a, n, n, 1e-6, nb)
    perm = api.reorder_permutation(nb)
    idx = perm[:S].contiguous()
    fc = torch.empty((n, Kp // 2), dtype=torch.uint8, device=dev)
    fs = torch.empty((n, Kp // 32), dtype=torch.uint8, device=dev)
    gc, gs = torch.empty_like(fc), torch.empty_like(fs)
    wf = api.arc_frontend(w, perm, S, append=L.RQ_APPEND_COPY, rmsnorm=False)
    wg = api.quantize(w, L.RQ_MXFP4, idx, L.RQ_APPEND_COPY)
    y = torch.empty((n, n), dtype=torch.float32, device=dev)

    def fused():
        L.rq_arc_frontend(a, n, n, perm, S, L.RQ_MXFP4, L.RQ_APPEND_RESIDUAL, 1, 1e-6, fc, fs)

    def unfused():
        L.rq_rmsnorm(a, n, n, 1e-6, nb)
        L.rq_quantize(nb, n, n, L.RQ_MXFP4, idx, S, L.RQ_APPEND_RESIDUAL, gc, gs)

    def fused_gemm():
        fused()
        L.rq_gemm(L.RQ_MXFP4, fc, fs, wf[0], wf[1], n, n, Kp, L.RQ_OUT_BF16, y)

    # the same pass without ARC (identity order, no appended channels): the
    # plain normalize-and-quantize front end, then the GEMM over K
    ident = torch.arange(n, dtype=torch.int32, device=dev)
    pc = torch.empty((n, n // 2), dtype=torch.uint8, device=dev)
    pcs = torch.empty((n, n // 32), dtype=torch.uint8, device=dev)

    def plain_gemm():
        L.rq_arc_frontend(a, n, n, ident, 0, L.RQ_MXFP4, L.RQ_APPEND_NONE, 1, 1e-6, pc, pcs)
        L.rq_gemm(L.RQ_MXFP4, pc, pcs, qc, qs, n, n, n, L.RQ_OUT_BF16, y)

    ms_f = time_calls(torch, fused, 50, graph=True)
    ms_u = time_calls(torch, unfused, 50, graph=True)
    ms_fg, ms_pg = time_interleaved(torch, [fused_gemm, plain_gemm], 50)
    ref = torch.empty((n, n), dtype=torch.float32, device=dev)
    L.rq_gemm(L.RQ_BF16, nb, None, w, None, n, n, n, L.RQ_OUT_F32, ref)

    def rel():
        return round(float((y - ref).norm() / ref.norm()), 5)

    fused()
    L.rq_gemm(L.RQ_MXFP4, fc, fs, wf[0], wf[1], n, n, Kp, L.RQ_OUT_F32, y)
    e_fused = rel()
    unfused()
    L.rq_gemm(L.RQ_MXFP4, gc, gs, wg[0], wg[1], n, n, Kp, L.RQ_OUT_F32, y)
    e_gather = rel()
    pa = api.quantize(nb, L.RQ_MXFP4)
    L.rq_gemm(L.RQ_MXFP4, pa[0], pa[1], qc, qs, n, n, n, L.RQ_OUT_F32, y)
    e_plain = rel()
    nbytes = n * n * 2 + n * Kp // 2 + n * Kp // 32 + 4 * n
    out = {"us_fused_front_end": round(ms_f * 1e3, 2), "gb_s": round(nbytes / (ms_f * 1e-3) / 1e9, 1),
           "frac_hbm": round(nbytes / (ms_f * 1e-3) / PEAK["hbm"], 4), "bytes": nbytes,
           "us_unfused_rmsnorm_then_quantize_gather": round(ms_u * 1e3, 2),
           "us_fused_front_end_plus_gemm_kprime4224": round(ms_fg * 1e3, 1),
           "us_plain_front_end_plus_gemm_k4096": round(ms_pg * 1e3, 1),
           "arc_overhead_vs_plain": round(ms_fg / ms_pg - 1, 4),
           "rel_err_vs_bf16_fused_arc": e_fused, "rel_err_vs_bf16_gather_arc": e_gather,
           "rel_err_vs_bf16_plain_mxfp4": e_plain}
    log(f"rows: ARC front end {out}")
    return out


_C4 = {}


def c4_block(W, tied=False):
    """The recurrent block's inputs, generated once per run."""
    if tied not in _C4:
        _C4[tied] = W.c4_ramp(tied=tied)
    return _C4[tied]


def measure_ramp(torch, api, L, W, to_dev, dev, time_calls):
    """Recurrent prefill rows: the four 8-step schedules (bit t-1 set = step
    t quantized) on the random-weight block and on the tied, contractive
    block; the block's per-step perturbation gain; the 32-step schedule with
    steps 1-24 in MXFP8."""
    S, D, F = 4096, 2048, 5632
    out = {}
    schedules = (("all_bf16", 0x00), ("ramp_steps1_6_mxfp4", 0x3F), ("uniform_mxfp4", 0xFF),
                 ("early_bf16_steps1_2", 0xFC))

    def run_block(d, tag, timed):
        h0 = to_dev(d["h0"])
        w1, w2 = to_dev(d["w1"]), to_dev(d["w2"])
        w1q, w2q = api.quantize(w1, L.RQ_MXFP4), api.quantize(w2, L.RQ_MXFP4)
        wsb = L.rq_recurrent_prefill_workspace_bytes(S, D, F, L.RQ_MXFP4)
        wsp = torch.empty(wsb, dtype=torch.uint8, device=dev)
        h = torch.empty_like(h0)
        res, outs = {}, {}

        def run(sched, steps=8, src=h0):
            h.copy_(src)
            L.rq_recurrent_prefill(h, S, D, F, w1, w2, w1q[0], w1q[1], w2q[0], w2q[1], L.RQ_MXFP4, sched, steps,
                                   1e-6, wsp, wsb)

        for name, sched in schedules:
            if timed:
                ms = time_calls(torch, lambda: L.rq_recurrent_prefill(h, S, D, F, w1, w2, w1q[0], w1q[1], w2q[0],
                                                                      w2q[1], L.RQ_MXFP4, sched, 8, 1e-6, wsp, wsb),
                                5, warmup=1, before=lambda: h.copy_(h0))
                res[name] = {"ms": round(ms, 3)}
            else:
                res[name] = {}
            run(sched)
            outs[name] = h.clone()
        ref = outs["all_bf16"].view(torch.bfloat16).float()
        for name in res:
            x = outs[name].view(torch.bfloat16).float()
            res[name]["final_state_rel_err_vs_all_bf16"] = float((x - ref).norm() / ref.norm())
        # per-step perturbation gain of one BF16 step: ||f(h + d) - f(h)|| / ||d||
        gen = torch.Generator(device=dev)
        gen.manual_seed(20261204)
        hp = (h0.view(torch.bfloat16).float() + 1e-2 * torch.randn(h0.shape, generator=gen, device=dev))
        hp = hp.to(torch.bfloat16).view(torch.int16)
        run(0x00, 1, h0)
        f0 = h.view(torch.bfloat16).float().clone()
        run(0x00, 1, hp)
        f1 = h.view(torch.bfloat16).float()
        dlt = hp.view(torch.bfloat16).float() - h0.view(torch.bfloat16).float()
        res["per_step_perturbation_gain"] = round(float((f1 - f0).norm() / dlt.norm()), 4)
        log(f"rows: RAMP {tag} {res}")
        return res, (h0, w1, w2, wsp, wsb, h)

    res, (h0, w1, w2, wsp, wsb, h) = run_block(c4_block(W), "random W", True)
    res["ramp_speedup_vs_all_bf16"] = round(res["all_bf16"]["ms"] / res["ramp_steps1_6_mxfp4"]["ms"], 4)
    out["recurrent_prefill_4096x2048_ffn5632_r8"] = res

    # 32 steps, 1-24 in MXFP8 (the long fixed-budget schedule), against 32 BF16 steps
    w1q8, w2q8 = api.quantize(w1, L.RQ_MXFP8), api.quantize(w2, L.RQ_MXFP8)
    wsb8 = L.rq_recurrent_prefill_workspace_bytes(S, D, F, L.RQ_MXFP8)
    wsp8 = torch.empty(wsb8, dtype=torch.uint8, device=dev)
    r32 = {}
    finals = {}
    # MXFP8 steps with exact block-scaled GEMMs (BF16 MFMAs) and on the FP8 scaled instruction
    for name, sched, gf in (("all_bf16", 0, L.RQ_MXFP8), ("steps1_24_mxfp8", (1 << 24) - 1, L.RQ_MXFP8),
                            ("uniform_mxfp8", (1 << 32) - 1, L.RQ_MXFP8),
                            ("steps1_24_mxfp8_fp8_instruction", (1 << 24) - 1, L.RQ_MXFP8_F8MFMA),
                            ("uniform_mxfp8_fp8_instruction", (1 << 32) - 1, L.RQ_MXFP8_F8MFMA)):
        def run32(sched=sched, gf=gf):
            L.rq_recurrent_prefill(h, S, D, F, w1, w2, w1q8[0], w1q8[1], w2q8[0], w2q8[1], gf, sched, 32,
                                   1e-6, wsp8, wsb8)
        ms = time_calls(torch, run32, 3, warmup=1, before=lambda: h.copy_(h0))
        h.copy_(h0)
        run32()
        finals[name] = h.view(torch.bfloat16).float().clone()
        r32[name] = {"ms": round(ms, 3)}
    for name in r32:
        r32[name]["final_state_rel_err_vs_all_bf16"] = float((finals[name] - finals["all_bf16"]).norm()
                                                             / finals["all_bf16"].norm())
    r32["speedup_vs_all_bf16"] = round(r32["all_bf16"]["ms"] / r32["steps1_24_mxfp8"]["ms"], 4)
    r32["speedup_vs_all_bf16_fp8_instruction"] = round(
        r32["all_bf16"]["ms"] / r32["steps1_24_mxfp8_fp8_instruction"]["ms"], 4)
    out["recurrent_prefill_4096x2048_ffn5632_t32_k24_mxfp8"] = r32
    log(f"rows: RAMP T=32 K=24 MXFP8 {r32}")
    del h0, w1, w2, wsp, h, w1q8, w2q8, wsp8, finals

    tied, _ = run_block(c4_block(W, True), "tied W2 = -W1^T", False)
    out["recurrent_prefill_tied_contractive_r8"] = tied
    return out


def measure_ramp_study(torch, np, api, L, W, to_dev, dev, time_calls):
    """Fixed-budget schedule study of the 8-step recurrent prefill (MXFP4):
    the switch point (steps 1..k quantized, BF16 after) for k = 0..8;
    twenty seeded random schedules with six of eight steps quantized (the
    RAMP budget) against RAMP's steps 1-6, on the random-weight and on the
    tied, contractive block; and RAMP's speedup over all-BF16 as the
    sequence grows from 128 to 4096 tokens."""
    S, D, F = 4096, 2048, 5632
    rng = np.random.default_rng(20261205)
    masks = []
    while len(masks) < 20:
        m = int(sum(1 << int(b) for b in rng.choice(8, 6, replace=False)))
        if m != 0x3F and m not in masks:
            masks.append(m)
    out = {"random_schedules": [f"0x{m:02X}" for m in masks]}
    for tag, d in (("random_w", c4_block(W)), ("tied_contractive", c4_block(W, True))):
        h0 = to_dev(d["h0"])
        w1, w2 = to_dev(d["w1"]), to_dev(d["w2"])
        w1q, w2q = api.quantize(w1, L.RQ_MXFP4), api.quantize(w2, L.RQ_MXFP4)
        wsb = L.rq_recurrent_prefill_workspace_bytes(S, D, F, L.RQ_MXFP4)
        wsp = torch.empty(wsb, dtype=torch.uint8, device=dev)
        h = torch.empty_like(h0)

        def final(sched):
            h.copy_(h0)
            L.rq_recurrent_prefill(h, S, D, F, w1, w2, w1q[0], w1q[1], w2q[0], w2q[1], L.RQ_MXFP4, sched, 8, 1e-6,
                                   wsp, wsb)
            return h.view(torch.bfloat16).float().clone()

        ref = final(0)

        def err(sched):
            return float((final(sched) - ref).norm() / ref.norm())

        r = {"switch_point_err": [round(err((1 << k) - 1), 5) for k in range(9)]}
        e_ramp = err(0x3F)
        e_rand = sorted(err(m) for m in masks)
        r["ramp_steps1_6_err"] = round(e_ramp, 5)
        r["random_6_of_8_err_min_median_max"] = [round(e_rand[0], 5), round(e_rand[10], 5), round(e_rand[-1], 5)]
        r["random_schedules_below_ramp"] = sum(e < e_ramp for e in e_rand)
        out[tag] = r
        del h0, w1, w2, w1q, w2q, wsp, h, ref
    # sequence sweep on the random-weight block: the token-wise block's cost
    # scales with S, the weight quantization is done once outside
    d = c4_block(W)
    w1, w2 = to_dev(d["w1"]), to_dev(d["w2"])
    w1q, w2q = api.quantize(w1, L.RQ_MXFP4), api.quantize(w2, L.RQ_MXFP4)
    sweep = {}
    for s_tok in (128, 256, 512, 1024, 2048, 4096):
        h0 = to_dev(d["h0"][:s_tok])
        h = torch.empty_like(h0)
        wsb = L.rq_recurrent_prefill_workspace_bytes(s_tok, D, F, L.RQ_MXFP4)
        wsp = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
        t = {}
        for name, sched in (("all_bf16", 0x00), ("ramp", 0x3F)):
            t[name] = time_calls(torch, lambda sched=sched: L.rq_recurrent_prefill(
                h, s_tok, D, F, w1, w2, w1q[0], w1q[1], w2q[0], w2q[1], L.RQ_MXFP4, sched, 8, 1e-6, wsp, wsb),
                5, warmup=1, before=lambda: h.copy_(h0))
        sweep[str(s_tok)] = {"all_bf16_ms": round(t["all_bf16"], 3), "ramp_ms": round(t["ramp"], 3),
                             "speedup": round(t["all_bf16"] / t["ramp"], 3)}
    out["sequence_sweep_r8"] = sweep
    log(f"rows: RAMP schedule study {out}")
    return out


def gpu_int8_weights(torch, gen, N, K, dev):
    w = torch.randn((N, K), generator=gen, device=dev) * 0.02
    blk = w.view(N, K // 32, 32)
    s = (blk.abs().amax(-1) / 127.0).to(torch.float16)
    s = torch.where(s == 0, torch.ones_like(s), s)
    q = torch.round(blk / s.float()[..., None]).clamp(-127, 127).to(torch.int8).view(N, K)
    return q, s.view(torch.int16)


GROUPED_NOTE = ("upper bound for a decode: the 197 linears in one launch treat their inputs as independent; "
                "a model runs its layers in order (the layer-ordered rows)")


def measure_gemv(torch, np, api, L, W, dev, gate=True):
    out = {}
    B = 16
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261208)
    lins = W.c5_linear_list()
    xs = {}
    for K in (1024, 2048, 3072):
        xs[K] = torch.randn((B, K), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    flags = torch.from_numpy(W.c5_flags(B)).to(dev)
    planes = []
    for name, K, N in lins:
        q, s = gpu_int8_weights(torch, gen, N, K, dev)
        planes.append((N, K, api.pack_nibble_planes(q, s)))
        del q, s
    ys = {N: torch.empty((B, N), dtype=torch.int16, device=dev) for _, _, N in lins}
    out["gemv_inputs"] = ("int8 weights, FP16 scales and x drawn on the GPU by torch's generator (seed 20261208) "
                          "with the config-5 recipe (w ~ N(0, 0.02^2), per-32 scales amax/127, x ~ N(0, 1)), "
                          "not the seeded NumPy streams the parity tests use; flags from the seeded permutation "
                          "(2 of 16 tokens)")
    # one split-K workspace, large enough for every shape (launches are stream-ordered)
    wsb = max(L.rq_gemv_workspace_bytes(B, N, K) for _, K, N in lins)
    wsp = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)  # arrival counters start at zero

    def low_bytes(N, K):
        return N * K // 2 + N * K // 32 * 2 + B * K * 2 + B * N * 2

    def esc_bytes(N, K, nf):
        return N * K + N * K // 32 * 2 + nf * K * 2 + nf * N * 2

    # with the FP32 carry: the low pass also writes every row's FP32 sum; the
    # escalation reads the lo plane, the scales, the flagged rows' x and
    # carry, and writes their y
    def low_carry_bytes(N, K):
        return low_bytes(N, K) + B * N * 4

    def esc_lo_bytes(N, K, nf):
        return N * K // 2 + N * K // 32 * 2 + nf * K * 2 + nf * N * 2 + nf * N * 4

    # LM head alone, low pass; four rotating copies so the 256 MB MALL does not serve it
    N, K, p = planes[-1]
    copies = [p] + [tuple(t.clone() for t in p) for _ in range(3)]
    it = [0]

    def lm_low():
        c = copies[it[0] % 4]
        it[0] += 1
        L.rq_gemv_nibble_escalate(xs[K], B, K, N, c[0], c[1], c[2], None, L.RQ_LOW, wsp, wsb, None, ys[N])

    ms = time_calls(torch, lm_low, 40)
    gb = low_bytes(N, K) / (ms * 1e-3) / 1e9
    out["gemv_lm_head_low_pass_b16"] = {"us": round(ms * 1e3, 2), "gb_s": round(gb, 1),
                                        "frac_hbm": round(gb * 1e9 / PEAK["hbm"], 4),
                                        "bytes": low_bytes(N, K)}
    nf_lm = int(flags.sum().item())

    def lm_esc():
        c = copies[it[0] % 4]
        it[0] += 1
        L.rq_gemv_nibble_escalate(xs[K], B, K, N, c[0], c[1], c[2], flags, L.RQ_ESCALATE, wsp, wsb, None, ys[N])

    ms = time_calls(torch, lm_esc, 40)
    gb = esc_bytes(N, K, nf_lm) / (ms * 1e-3) / 1e9
    out["gemv_lm_head_escalation_2_of_16"] = {"us": round(ms * 1e3, 2), "gb_s": round(gb, 1),
                                              "frac_hbm": round(gb * 1e9 / PEAK["hbm"], 4),
                                              "bytes": esc_bytes(N, K, nf_lm)}
    # the same two passes through the FP32 carry (the copies hold the same
    # weights, so one carry serves them all)
    carry = torch.empty((B, N), dtype=torch.float32, device=dev)

    def lm_low_carry():
        c = copies[it[0] % 4]
        it[0] += 1
        L.rq_gemv_nibble_escalate(xs[K], B, K, N, c[0], c[1], c[2], None, L.RQ_LOW, wsp, wsb, carry, ys[N])

    def lm_esc_lo():
        c = copies[it[0] % 4]
        it[0] += 1
        L.rq_gemv_nibble_escalate(xs[K], B, K, N, None, c[1], c[2], flags, L.RQ_ESCALATE, wsp, wsb, carry, ys[N])

    ms = time_calls(torch, lm_low_carry, 40)
    out["gemv_lm_head_low_pass_b16_with_carry"] = {
        "us": round(ms * 1e3, 2), "gb_s": round(low_carry_bytes(N, K) / (ms * 1e-3) / 1e9, 1),
        "frac_hbm": round(low_carry_bytes(N, K) / (ms * 1e-3) / PEAK["hbm"], 4), "bytes": low_carry_bytes(N, K)}
    ms = time_calls(torch, lm_esc_lo, 40)
    out["gemv_lm_head_escalation_2_of_16_lo_plane_from_carry"] = {
        "us": round(ms * 1e3, 2), "gb_s": round(esc_lo_bytes(N, K, nf_lm) / (ms * 1e-3) / 1e9, 1),
        "frac_hbm": round(esc_lo_bytes(N, K, nf_lm) / (ms * 1e-3) / PEAK["hbm"], 4),
        "bytes": esc_lo_bytes(N, K, nf_lm)}
    if gate:
        parts_us = (out["gemv_lm_head_low_pass_b16_with_carry"]["us"]
                    + out["gemv_lm_head_escalation_2_of_16_lo_plane_from_carry"]["us"])
        out.update(measure_gate(torch, L, dev, N, K, xs, ys, copies, it, carry, wsp, wsb, lm_low_carry, parts_us))
    del copies, carry

    def sweep(phase):
        for N, K, (hi, lo, st) in planes:
            L.rq_gemv_nibble_escalate(xs[K], B, K, N, hi, lo, st, flags, phase, wsp, wsb, None, ys[N])

    tot_low = sum(low_bytes(N, K) for N, K, _ in planes)
    nf = int(flags.sum().item())
    tot_esc = sum(esc_bytes(N, K, nf) for N, K, _ in planes)
    ms_low = time_calls(torch, lambda: sweep(L.RQ_LOW), 10)
    ms_esc = time_calls(torch, lambda: sweep(L.RQ_ESCALATE), 10)
    # the same 197-launch sweeps captured once in a HIP graph and replayed
    graphs = {}
    for phase in (L.RQ_LOW, L.RQ_ESCALATE):
        sweep(phase)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sweep(phase)
        graphs[phase] = g
    ms_low_g = time_calls(torch, graphs[L.RQ_LOW].replay, 10)
    ms_esc_g = time_calls(torch, graphs[L.RQ_ESCALATE].replay, 10)
    out["gemv_full_sweep_197_linears_low_pass_b16_hip_graph"] = {
        "us": round(ms_low_g * 1e3, 1), "gb_s": round(tot_low / (ms_low_g * 1e-3) / 1e9, 1),
        "frac_hbm": round(tot_low / (ms_low_g * 1e-3) / PEAK["hbm"], 4), "bytes": tot_low}
    out["gemv_full_sweep_escalation_2_of_16_hip_graph"] = {
        "us": round(ms_esc_g * 1e3, 1), "gb_s": round(tot_esc / (ms_esc_g * 1e-3) / 1e9, 1),
        "frac_hbm": round(tot_esc / (ms_esc_g * 1e-3) / PEAK["hbm"], 4), "bytes": tot_esc}
    del graphs
    # the same sweeps as one grouped launch per phase (a problem table in
    # device memory; no split-K: the 197 problems give 7750 row tiles)
    gys = [torch.empty((B, N), dtype=torch.bfloat16, device=dev) for N, _, _ in planes]
    table = api.gemv_group([(xs[K], p, y) for (N, K, p), y in zip(planes, gys)], dev)
    ms_low_grp = time_calls(torch, lambda: api.gemv_nibble_escalate_grouped(table, B, None, L.RQ_LOW), 10)
    ms_esc_grp = time_calls(torch, lambda: api.gemv_nibble_escalate_grouped(table, B, flags, L.RQ_ESCALATE), 10)
    out["gemv_full_sweep_197_linears_low_pass_b16_grouped"] = {
        "us": round(ms_low_grp * 1e3, 1), "gb_s": round(tot_low / (ms_low_grp * 1e-3) / 1e9, 1),
        "frac_hbm": round(tot_low / (ms_low_grp * 1e-3) / PEAK["hbm"], 4), "bytes": tot_low,
        "launches": 1, "tiles": table[2], "bound": GROUPED_NOTE}
    out["gemv_full_sweep_escalation_2_of_16_grouped"] = {
        "us": round(ms_esc_grp * 1e3, 1), "gb_s": round(tot_esc / (ms_esc_grp * 1e-3) / 1e9, 1),
        "frac_hbm": round(tot_esc / (ms_esc_grp * 1e-3) / PEAK["hbm"], 4), "bytes": tot_esc,
        "bound": GROUPED_NOTE}
    del table
    # grouped, through the FP32 carries: the escalation reads only the lo planes
    carries = [torch.empty((B, N), dtype=torch.float32, device=dev) for N, _, _ in planes]
    table = api.gemv_group([(xs[K], p, y, c) for (N, K, p), y, c in zip(planes, gys, carries)], dev)
    tot_low_c = sum(low_carry_bytes(N, K) for N, K, _ in planes)
    tot_esc_lo = sum(esc_lo_bytes(N, K, nf) for N, K, _ in planes)
    ms_low_c = time_calls(torch, lambda: api.gemv_nibble_escalate_grouped(table, B, None, L.RQ_LOW), 10)
    ms_esc_lo = time_calls(torch, lambda: api.gemv_nibble_escalate_grouped(table, B, flags, L.RQ_ESCALATE), 10)
    out["gemv_full_sweep_197_linears_low_pass_b16_grouped_with_carry"] = {
        "us": round(ms_low_c * 1e3, 1), "gb_s": round(tot_low_c / (ms_low_c * 1e-3) / 1e9, 1),
        "frac_hbm": round(tot_low_c / (ms_low_c * 1e-3) / PEAK["hbm"], 4), "bytes": tot_low_c,
        "bound": GROUPED_NOTE}
    out["gemv_full_sweep_escalation_2_of_16_grouped_lo_plane_from_carry"] = {
        "us": round(ms_esc_lo * 1e3, 1), "gb_s": round(tot_esc_lo / (ms_esc_lo * 1e-3) / 1e9, 1),
        "frac_hbm": round(tot_esc_lo / (ms_esc_lo * 1e-3) / PEAK["hbm"], 4), "bytes": tot_esc_lo,
        "bound": GROUPED_NOTE}
    del table, gys, carries
    out.update(measure_decode_layer_ordered(torch, api, L, W, dev, gen, xs, flags, planes[-1], low_bytes, esc_bytes))
    out["gemv_full_sweep_197_linears_low_pass_b16"] = {
        "us": round(ms_low * 1e3, 1), "gb_s": round(tot_low / (ms_low * 1e-3) / 1e9, 1),
        "frac_hbm": round(tot_low / (ms_low * 1e-3) / PEAK["hbm"], 4), "bytes": tot_low,
        "launches": len(planes)}
    out["gemv_full_sweep_escalation_2_of_16"] = {
        "us": round(ms_esc * 1e3, 1), "gb_s": round(tot_esc / (ms_esc * 1e-3) / 1e9, 1),
        "frac_hbm": round(tot_esc / (ms_esc * 1e-3) / PEAK["hbm"], 4), "bytes": tot_esc}
    log(f"rows: GEMV {out}")
    return out


def measure_decode_layer_ordered(torch, api, L, W, dev, gen, xs, flags, lm, low_bytes, esc_bytes):
    """The decode step in layer order, as a model runs it: per layer q/k/v
    (one GEMV on the stacked weights, as they share their input), o,
    gate/up (stacked), down, then the LM head -- 28 x 4 + 1 = 113 launches
    on one stream, each waiting for the one before (no batching across
    layers).  Small-N shapes split K inside their launch.  The low pass over
    all 16 tokens, and the escalation of the 2 flagged tokens with both
    planes (their hidden states differ from the low pass's, so no carry);
    eager, and captured once in a HIP graph and replayed."""
    out = {}
    B = 16
    shapes = [("qkv", 1024, 2048 + 1024 + 1024), ("o", 2048, 1024), ("gate_up", 1024, 2 * 3072),
              ("down", 3072, 1024)]
    layer = []
    for _ in range(len(W.c5_linear_list()) // 7):
        for name, K, N in shapes:
            q, sc = gpu_int8_weights(torch, gen, N, K, dev)
            layer.append((N, K, api.pack_nibble_planes(q, sc)))
            del q, sc
    seq = layer + [lm]
    ys = {N: torch.empty((B, N), dtype=torch.int16, device=dev) for N, _, _ in seq}
    wsb = max(L.rq_gemv_workspace_bytes(B, N, K) for N, K, _ in seq)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)  # arrival counters start at zero

    def step(phase):
        for N, K, (hi, lo, st) in seq:
            L.rq_gemv_nibble_escalate(xs[K], B, K, N, hi, lo, st, flags, phase, ws, wsb, None, ys[N])

    nf = int(flags.sum().item())
    tot = {L.RQ_LOW: sum(low_bytes(N, K) for N, K, _ in seq), L.RQ_ESCALATE: sum(esc_bytes(N, K, nf) for N, K, _ in seq)}
    tag = {L.RQ_LOW: "low_pass_b16", L.RQ_ESCALATE: "escalation_2_of_16"}
    for phase in (L.RQ_LOW, L.RQ_ESCALATE):
        ms = time_calls(torch, lambda: step(phase), 10)
        step(phase)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(phase)
        ms_g = time_calls(torch, g.replay, 10)
        del g
        for form, t in (("eager", ms), ("hip_graph", ms_g)):
            out[f"gemv_decode_step_layer_ordered_{tag[phase]}_{form}"] = {
                "us": round(t * 1e3, 1), "gb_s": round(tot[phase] / (t * 1e-3) / 1e9, 1),
                "frac_hbm": round(tot[phase] / (t * 1e-3) / PEAK["hbm"], 4), "bytes": tot[phase],
                "launches": len(seq), "split_k_launches": sum(L.rq_gemv_workspace_bytes(B, N, K) > 0 for N, K, _ in seq)}
    del layer, seq, ys, ws
    log(f"rows: layer-ordered decode step {out}")
    return out


def measure_gate(torch, L, dev, N, K, xs, ys, copies, it, carry, wsp, wsb, lm_low_carry, parts_us):
    """The escalation gate rows; parts_us: the carry low pass plus the
    lo-plane escalation of the LM head, microseconds."""
    out = {}
    B = ys[N].shape[0]
    # the escalation gate over the LM head's low-pass logits [16 x 151936]
    # (softmax entropy and top-1 / top-2 margin per token), alone and as the
    # middle of the LM head's whole decode step on the device: low pass with
    # the carry, gate, lo-plane escalation of the tokens it flags.  tau sits
    # between the second and third largest entropy, so the gate flags two
    # tokens as the seeded flags above do; delta = 0 leaves the margin test
    # off (random logits have no confident tokens).
    lm_low_carry()
    logits = ys[N]
    gflags = torch.empty(B, dtype=torch.uint8, device=dev)
    gstats = torch.empty((B, 2), dtype=torch.float32, device=dev)
    gwsb = L.rq_escalation_gate_workspace_bytes(B, N)
    gws = torch.empty(max(gwsb, 16), dtype=torch.uint8, device=dev)
    L.rq_escalation_gate(logits, B, N, 0.0, 0.0, gflags, gstats, gws, gwsb)
    ent = sorted(gstats[:, 0].tolist(), reverse=True)
    tau = 0.5 * (ent[1] + ent[2])
    ms = time_calls(torch, lambda: L.rq_escalation_gate(logits, B, N, tau, 0.0, gflags, gstats, gws, gwsb), 100,
                    graph=True)
    gate_bytes = B * N * 2
    out["escalation_gate_lm_head_logits_16x151936"] = {
        "us": round(ms * 1e3, 2), "gb_s": round(gate_bytes / (ms * 1e-3) / 1e9, 1),
        "frac_hbm": round(gate_bytes / (ms * 1e-3) / PEAK["hbm"], 4), "bytes": gate_bytes}

    def lm_decode_step():
        lm_low_carry()
        L.rq_escalation_gate(logits, B, N, tau, 0.0, gflags, gstats, gws, gwsb)
        c = copies[it[0] % 4]
        it[0] += 1
        L.rq_gemv_nibble_escalate(xs[K], B, K, N, None, c[1], c[2], gflags, L.RQ_ESCALATE, wsp, wsb, carry, ys[N])

    ms = time_calls(torch, lm_decode_step, 40)
    out["gemv_lm_head_decode_step_low_gate_escalate_b16"] = {
        "us": round(ms * 1e3, 2), "flagged": int(gflags.sum().item()),
        "us_parts_sum": round(parts_us + out["escalation_gate_lm_head_logits_16x151936"]["us"], 2)}
    return out


def cpu_baseline(np, W, gpu_f32=None, acc_rows=256):
    """The CPU oracle (float64 NumPy) on a bounded sample of the main
    workload: 256 rows of each group's input, quantize + GEMM against the
    group's stacked weights (dequantized outside the timed region),
    repeated for about 10 s.  The oracle's products of those rows also give
    the relative Frobenius error of the GPU's FP32 outputs (exact MXFP8 path
    and the FP8 instruction) on them."""
    import threadpoolctl
    from oracle import formats as F
    from oracle import quant as Q
    from oracle import gemm as G

    rows = 256
    work = []
    for g in W.c2_layer(M=rows):
        work.append((g["a"], Q.quantize_dequantize(g["w"], F.FMT_MXFP8)))
    flop = sum(2.0 * rows * a.shape[1] * wd.shape[0] for a, wd in work)
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] or [1])
    n = 0
    t0 = time.perf_counter()
    while True:
        for a, wd in work:
            y = G.matmul_f64(Q.quantize_dequantize(a, F.FMT_MXFP8), wd)
            F.f64_to_bf16(y)
        n += 1
        if time.perf_counter() - t0 >= 10.0:
            break
    dt = (time.perf_counter() - t0) / n
    accuracy = {}
    if gpu_f32:
        for g, (a, wd) in zip(W.c2_layer(M=rows), work):
            ref = G.matmul_f64(Q.quantize_dequantize(a[:acc_rows], F.FMT_MXFP8), wd)
            for tag in ("exact", "f8mfma"):
                y = gpu_f32[(g["name"], tag)].astype(np.float64)
                accuracy[f"{g['name']} {tag}"] = float(f"{G.rel_frobenius(y, ref):.3e}")
    return {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "accuracy": accuracy,
            "sample": f"{rows} of 4096 rows of each of the 4 layer inputs (quantize + float64 GEMM against the "
                      f"stacked weights + BF16 rounding), {n} repetitions, {dt:.3f} s each",
            "rows": cpu_rows(np, W)}


def cpu_rows(np, W):
    """The oracle's other steps on bounded samples (a baseline only): MXFP4
    quantization, one decode GEMV with escalation, one RAMP step; each the
    median of three timed runs after one warm-up."""
    from oracle import formats as F
    from oracle import quant as Q
    from oracle import gemv as V
    from oracle import ramp as R

    def med3(fn):
        fn()
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[1]

    out = {}
    a = W.c3_arc(M=256, N=32)["a"]
    t = med3(lambda: Q.quantize_mx(a, F.FMT_MXFP4))
    qb = a.size * 2 + a.size // 2 + a.size // 32
    out["quantize_mxfp4_256x4096"] = {"s": round(t, 4), "gb_s": round(qb / t / 1e9, 4)}
    d = W.c5_linear(0)
    flags = d["flags"]
    t = med3(lambda: V.gemv_nibble_escalate(d["x"], d["w"], d["scales"], flags))
    wb = d["w"].size
    out[f"gemv_nibble_escalate_{d['name']}_{d['w'].shape[0]}x{d['w'].shape[1]}_b16"] = {
        "s": round(t, 4), "gb_s_of_int8_weights": round(wb / t / 1e9, 4)}
    c4 = W.c4_ramp(S=64)
    w1d = R.quantize_weights(c4["w1"], F.FMT_MXFP4)
    w2d = R.quantize_weights(c4["w2"], F.FMT_MXFP4)
    t = med3(lambda: R.ramp_step(c4["h0"], c4["w1"], c4["w2"], True, F.FMT_MXFP4, w1d, w2d))
    out["ramp_step_mxfp4_64_of_4096_rows"] = {"s": round(t, 4), "s_per_step_at_4096_rows": round(t * 64, 2)}
    return out


if __name__ == "__main__":
    main()
