#!/usr/bin/env python3
"""Benchmark of the BF16x9 emulated SGEMM on one MI355X.

One step is one pass of the whole path over the large PET-like workload
(17,280 atoms x 32 neighbour tokens = 552,960 rows, d = 256, FFN = 1024):
    split W1 [256 x 1024] and W2 [1024 x 256] into BF16 planes   (standalone split)
    C1 = X [552960 x 256]  . W1     (A split inside the GEMM, nine products)
    C2 = H [552960 x 1024] . W2     (H = GELU(X W1), computed once before timing)
Inputs are seeded synthetic data already resident in HBM when timing starts.
Reported value: effective FP32 TFLOP/s = (2 M N1 K1 + 2 M N2 K2) / t_step.

Also reported on the same line:
  roofline      the GEMM kernel against the BF16 dense MFMA peak, counting the
                nine BF16 products (18 M N K flops per launch), from HIP events
                recorded around every GEMM launch of the timed steps on the
                stream the kernels run on;
  cpu_baseline  the oracle's naive FP32 SGEMM on a bounded sample of the same
                rows, timed on this host's cores;
  context       torch.matmul FP32 (rocBLAS/hipBLASLt) on the same GEMMs and
                the fused-B entry point sgemm_bf16x9, for comparison only.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-context]
"""
import argparse
import json
import os
import sys
import time

MI355X_BF16_DENSE_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 flop/clk/CU
MI355X_FP32_VECTOR_TFLOPS = 157.3
MI355X_HBM_GBS = 8000.0
METRIC = "BF16x9 SGEMM effective FP32 TFLOP/s (2MNK/t) and % of bf16 MFMA peak"
HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCE = os.path.join(HERE, "fp32_emulated_gemm_amd", "csrc", "gemm.hip")

# HBM traffic of the timed GEMM kernel per launch ([X@W1, H@W2], bytes), from two
# rocprofv3 --pmc runs of `python3 bench.py --traffic-probe` (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for
# the probe's cold 2 GiB device copy (FETCH_SIZE reads half the copied bytes:
# x2.0; WRITE_SIZE reads all of them: x1.0).  The figures belong to the kernel
# source they were taken on; once gemm.hip has changed, roofline.traffic is null.
GEMM_TRAFFIC = {"gemm_hip_sha256": "75195d81894525a370e411dd08d3e74a307f23e645ba9ed56e41630d4769eaeb",
                "bytes_per_launch": [2843925792, 3264026398]}

# MFMA activity of the same launches, from one rocprofv3 --pmc run of the same
# probe (SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_BUSY_CYCLES GRBM_GUI_ACTIVE).
# busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs): the
# share of the kernel's active cycles in which a SIMD's matrix pipe was busy
# (one 32x32x16 BF16 MFMA keeps it busy 32 cycles).  GRBM_GUI_ACTIVE per XCD
# divided by the kernel's own time in this run gives the shader clock the chip
# held under the load; roofline.frac = busy x clock / 2.4 GHz.
GEMM_MFMA_PMC = {"gemm_hip_sha256": GEMM_TRAFFIC["gemm_hip_sha256"],
                 "mfma_busy": [0.6544, 0.7188],
                 "active_cycles_per_xcd": [3815687, 3465315]}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # ten untimed steps: the engine clock ramps down under this load for the
    # first eight or so GEMM launches (kernel traces), so the timed steps start
    # on a settled clock
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-context", action="store_true", help="skip torch.matmul / fused-B context timings")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--calibrate", action="store_true",
                   help="only time the platform's BF16 and FP32 GEMMs (torch.matmul) on the square and "
                        "PET shapes and print them as one JSON line")
    p.add_argument("--calibrate-reps", type=int, default=10)
    p.add_argument("--sustain", type=float, default=None,
                   help="SECONDS: only run the vendor BF16 GEMM, sgemm_bf16x9 and the vendor FP32 GEMM on "
                        "4096^3 and 8192^3 for SECONDS each (normal and uniform operands), sampling the "
                        "engine clock with rocm-smi, and print them as one JSON line")
    p.add_argument("--shape", type=str, default=None,
                   help="M,N,K: only time the library's entry points (and torch.matmul FP32) on this one "
                        "shape, random N(0,1) operands, and print them as one JSON line (for kernel traces)")
    p.add_argument("--shape-reps", type=int, default=20)
    p.add_argument("--shape-warmup", type=float, default=1.0,
                   help="seconds of untimed calls of every entry point before --shape times them")
    p.add_argument("--shape-rounds", type=int, default=2,
                   help="timed rounds of --shape (each entry point in turn); the fastest round is kept")
    p.add_argument("--traffic-probe", action="store_true",
                   help="for HBM counter runs: two steps, one split of X, then one plain 2 GiB device copy "
                        "whose FETCH/WRITE counts calibrate the counters; prints no JSON line")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.calibrate:
        calibrate(args.calibrate_reps)
        return
    if args.sustain:
        sustained(args.sustain)
        return
    if args.shape:
        one_shape(tuple(int(x) for x in args.shape.split(",")), args.shape_reps, args.shape_warmup,
                  args.shape_rounds)
        return

    import numpy as np
    import torch
    import fp32_emulated_gemm_amd as fe
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")

    t0 = time.perf_counter()
    w = workloads.pet_large()
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s")
    X, W1, W2 = w["X"], w["W1"], w["W2"]
    M, D = X.shape
    F = W1.shape[1]
    Xd = torch.from_numpy(X).to(dev)
    W1d = torch.from_numpy(W1).to(dev)
    W2d = torch.from_numpy(W2).to(dev)
    # The weights as a linear layer stores them, [out_features][in_features].
    W1t = W1d.t().contiguous()
    W2t = W2d.t().contiguous()
    C1 = torch.empty((M, F), dtype=torch.float32, device=dev)
    C2 = torch.empty((M, D), dtype=torch.float32, device=dev)
    P1 = [torch.empty((F, D), dtype=torch.int16, device=dev) for _ in range(3)]
    P2 = [torch.empty((D, F), dtype=torch.int16, device=dev) for _ in range(3)]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    # The hidden layer H = GELU(X W1), chained as in the network: computed once,
    # before timing, by the library's linear layer with its fused GELU epilogue
    # (within a few ulp of fp32(GELU) of the exact product).
    Hd = torch.empty((M, F), dtype=torch.float32, device=dev)
    fe.split_f32_bf16x3(F, D, W1t, D, *P1, D, sp)
    fe.sgemm_emu_linear(M, F, D, Xd, D, *P1, D, None, fe.SGEMM_EMU_ACT_GELU, Hd, F, 5, sp)
    torch.cuda.synchronize()

    ev = []

    def step(record):
        if record:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            e[4].record(stream)
        fe.split_f32_bf16x3(F, D, W1t, D, *P1, D, sp)
        fe.split_f32_bf16x3(D, F, W2t, F, *P2, F, sp)
        if record:
            e[0].record(stream)
        fe.sgemm_emu_presplit_b(M, F, D, Xd, D, *P1, D, fe.SGEMM_EMU_B_NK, C1, F, 5, sp)
        if record:
            e[1].record(stream)
            e[2].record(stream)
        fe.sgemm_emu_presplit_b(M, D, F, Hd, F, *P2, F, fe.SGEMM_EMU_B_NK, C2, D, 5, sp)
        if record:
            e[3].record(stream)
            ev.append(e)

    if args.traffic_probe:
        for _ in range(2):
            step(False)
        # the standalone split kernel on X (552960 x 256): 4 + 6 bytes per element
        Xp = [torch.empty((M, D), dtype=torch.int16, device=dev) for _ in range(3)]
        fe.split_f32_bf16x3(M, D, Xd, D, *Xp, D, sp)
        torch.cuda.synchronize()
        del Xp
        # Calibration: a plain device copy of known size whose source is cold.
        # The source is written first, then a 1 GiB fill evicts it from the
        # 256 MB last-level cache, then the copy reads and writes 2 GiB.
        src = torch.empty(512 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        evict = torch.empty(256 << 20, dtype=torch.float32, device=dev).fill_(2.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"traffic probe done: 2 steps, then a {src.numel() * 4}-byte copy "
            f"(evict buffer {evict.numel() * 4} bytes)")
        return

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step(True)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / args.steps

    flops_eff = 2.0 * M * F * D + 2.0 * M * D * F
    value = flops_eff / (ms_step * 1e-3) / 1e12
    g1 = [e[0].elapsed_time(e[1]) for e in ev]
    g2 = [e[2].elapsed_time(e[3]) for e in ev]
    wsplit = [e[4].elapsed_time(e[0]) for e in ev]        # both weight splits of a step
    g1_ms, g2_ms = float(np.mean(g1)), float(np.mean(g2))
    # roofline of the GEMM kernel: nine BF16 products per FP32 multiply-add pair
    bf16_flops_per_launch = [18.0 * M * F * D, 18.0 * M * D * F]
    achieved = sum(bf16_flops_per_launch) / ((g1_ms + g2_ms) * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms (wall {wall / args.steps * 1e3:.3f} ms); GEMM1 {g1_ms:.3f} ms, GEMM2 {g2_ms:.3f} ms")
    # bytes each GEMM must move at least: A (FP32) + three BF16 planes of B + C (FP32)
    algo_bytes = [4 * M * D + 6 * D * F + 4 * M * F, 4 * M * F + 6 * F * D + 4 * M * D]
    traffic_per_launch = None
    if GEMM_TRAFFIC["gemm_hip_sha256"] == source_sha256(GEMM_SOURCE):
        traffic_per_launch = GEMM_TRAFFIC["bytes_per_launch"]
    traffic = None if traffic_per_launch is None else sum(traffic_per_launch) / len(traffic_per_launch)
    mfma_busy = sclk = None
    if GEMM_MFMA_PMC["gemm_hip_sha256"] == source_sha256(GEMM_SOURCE):
        mfma_busy = GEMM_MFMA_PMC["mfma_busy"]
        sclk = [round(c / (t * 1e-3) / 1e9, 3) for c, t in zip(GEMM_MFMA_PMC["active_cycles_per_xcd"], (g1_ms, g2_ms))]

    # correctness spot check of the timed outputs against torch FP32 (sanity, not parity)
    ref1 = torch.matmul(Xd[:256], W1d)
    rel = float((C1[:256] - ref1).norm() / ref1.norm())
    if not rel < 1e-5:
        raise SystemExit(f"bench: output check failed (relative error {rel:.3g})")

    context = None
    if not args.no_context:
        context = context_timings(fe, torch, Xd, Hd, W1d, W2d, C1, C2, M, D, F, stream, sp)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(X, W1, Hd.cpu().numpy(), W2, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "pet_large: X[552960x256] @ W1[256x1024] and H[552960x1024] @ W2[1024x256] "
                        "(17280 atoms x 32 tokens), H = GELU(X W1) chained once before timing, "
                        "weights held [out][in] and split once per step, all nine products",
            "M": M, "d": D, "ffn": F, "nbands": 5,
            "entry": "split_f32_bf16x3 + sgemm_emu_presplit_b(SGEMM_EMU_B_NK)",
        },
        "pct_bf16_peak_9products": round(100.0 * value * 9 / MI355X_BF16_DENSE_TFLOPS, 2),
        "pct_fp32_vector_peak": round(100.0 * value / MI355X_FP32_VECTOR_TFLOPS, 2),
        "gemm_ms": {"X@W1": round(g1_ms, 4), "H@W2": round(g2_ms, 4)},
        "gemm_ms_per_launch": {name: {"median": round(float(np.median(v)), 4), "min": round(float(np.min(v)), 4),
                                      "max": round(float(np.max(v)), 4)} for name, v in (("X@W1", g1), ("H@W2", g2))},
        "weight_split_ms_per_step": round(float(np.mean(wsplit)), 4),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MI355X_BF16_DENSE_TFLOPS, 4),
            "traffic": traffic,
            "traffic_per_launch": traffic_per_launch,
            "algorithmic_bytes_per_launch": algo_bytes,
            "kernel": "gemm_bf16x9_dma_kernel<Cfg<2,4,64,32,sched>, 5 bands>: N x K planes copied to LDS by DMA, A split in-kernel",
            "flops_per_launch": bf16_flops_per_launch,
            "mfma_busy_per_launch_pmc": mfma_busy,
            "sclk_ghz_under_load": sclk,
        },
        "cpu_baseline": cpu,
        "context": context,
    }
    print(json.dumps(out), flush=True)


def source_sha256(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def timed(fn, stream, reps):
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def settled_ms(entries, stream, reps, warmup_s=1.0, rounds=2):
    """Milliseconds per call of each entry point: every entry in turn for
    warmup_s seconds first, so the clock has settled under load before anything
    is timed; then `rounds` timed rounds in turn, the fastest of each entry
    point's kept (the order of the entries then no longer decides which of them
    meets a ramping clock)."""
    import time
    import torch
    t0 = time.time()
    while time.time() - t0 < warmup_s:
        for fn in entries.values():
            fn()
        torch.cuda.synchronize()
    times = [{name: timed(fn, stream, reps) for name, fn in entries.items()} for _ in range(max(rounds, 1))]
    return {name: min(t[name] for t in times) for name in entries}


def vendor_bf16(torch, stream, shapes, reps=10):
    """Context for the ceiling: the platform's own BF16 GEMM (torch.matmul on BF16
    operands, i.e. hipBLASLt; run, never inspected) on the given M x N x K shapes,
    random operands, HIP events on the same stream.  One BF16 product per FP32
    multiply-add pair, so its rate compares with the roofline's achieved rate."""
    res = {}
    g = torch.Generator(device="cuda").manual_seed(7)
    for name, (m, n, k) in shapes.items():
        A = (torch.rand((m, k), device="cuda", generator=g) * 2 - 1).to(torch.bfloat16)
        B = (torch.rand((k, n), device="cuda", generator=g) * 2 - 1).to(torch.bfloat16)
        C = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        t = timed(lambda: torch.matmul(A, B, out=C), stream, reps)
        tf = 2.0 * m * n * k / t / 1e9
        res[name] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / MI355X_BF16_DENSE_TFLOPS, 4)}
        del A, B, C
    log(f"vendor BF16 GEMM (torch.matmul, hipBLASLt): {res}")
    return res


def one_shape(shape, reps, warmup_s=1.0, rounds=2):
    """--shape: every entry point on one M x N x K shape, effective TFLOP/s."""
    import torch
    import fp32_emulated_gemm_amd as fe
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    m, n, k = shape
    g = torch.Generator(device="cuda").manual_seed(5)
    A = torch.randn((m, k), device="cuda", generator=g)
    B = torch.randn((k, n), device="cuda", generator=g) / max(k, 1) ** 0.5
    C = torch.empty((m, n), device="cuda")
    Bt_planes = fe.split(B.t().contiguous())
    fl = 2.0 * m * n * k
    entries = {
        "sgemm_bf16x9": lambda: fe.sgemm_bf16x9(m, n, k, A, k, B, n, C, n, sp),
        "presplit_nk": lambda: fe.sgemm_emu_presplit_b(m, n, k, A, k, *Bt_planes, k, fe.SGEMM_EMU_B_NK, C, n, 5, sp),
        "native_fp32": lambda: fe.sgemm_emu_ex(m, n, k, A, k, B, n, C, n, 5, fe.SGEMM_EMU_NATIVE_FP32, sp),
        "performant": lambda: fe.sgemm_emu_ex(m, n, k, A, k, B, n, C, n, 5, fe.SGEMM_EMU_PERFORMANT, sp),
        "torch_fp32": lambda: torch.matmul(A, B, out=C),
    }
    ms = settled_ms(entries, stream, reps, warmup_s, rounds)
    res = {name: round(fl / ms[name] / 1e9, 2) for name in entries}
    print(json.dumps({"shape": [m, n, k], "reps": reps, "tflops": res,
                      "split_k": fe.sgemm_emu_split_k(m, n, k, 5),
                      "split_k_fp32_b": fe.sgemm_emu_split_k_fp32_b(m, n, k, 5)}), flush=True)


CALIBRATION_SHAPES = {"4096^3": (4096, 4096, 4096), "8192^3": (8192, 8192, 8192),
                      "X@W1 552960x1024x256": (552960, 1024, 256), "H@W2 552960x256x1024": (552960, 256, 1024)}


def calibrate(reps):
    """--calibrate: the platform's BF16 and FP32 GEMMs on the square and PET shapes,
    one JSON line (the ceiling the chip reaches with a vendor BF16 kernel on random
    data; for rocprofv3 counter runs beside the emulated GEMM's)."""
    import torch
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    bf16 = vendor_bf16(torch, stream, CALIBRATION_SHAPES, reps)
    fp32 = {}
    g = torch.Generator(device="cuda").manual_seed(8)
    for name, (m, n, k) in CALIBRATION_SHAPES.items():
        A = torch.rand((m, k), device="cuda", generator=g) * 2 - 1
        B = torch.rand((k, n), device="cuda", generator=g) * 2 - 1
        C = torch.empty((m, n), device="cuda")
        t = timed(lambda: torch.matmul(A, B, out=C), stream, reps)
        fp32[name] = round(2.0 * m * n * k / t / 1e9, 1)
        del A, B, C
    print(json.dumps({"calibration": "torch.matmul BF16 / FP32 (hipBLASLt), random operands",
                      "reps": reps, "bf16": bf16, "fp32_tflops": fp32,
                      "bf16_dense_peak_tflops": MI355X_BF16_DENSE_TFLOPS}), flush=True)


def engine_clock_mhz():
    """The engine clock rocm-smi reports now (MHz), or None where it cannot be read."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "-g", "--json"], capture_output=True, text=True, timeout=30).stdout
        level = json.loads(out[out.index("{"):])["card0"]["sclk clock level"]
        return int(level.split("(")[1].split("M")[0])
    except Exception:
        return None


def sustained(seconds):
    """--sustain: each GEMM back to back for `seconds` (the clock settles under a
    sustained load), the effective rate from HIP events around all the calls, the
    engine clock sampled twice in the second half.  Square shapes, operands
    N(0,1) and U(-1,1): the vendor BF16 GEMM (one product, the ceiling a BF16
    kernel reaches), sgemm_bf16x9 (nine products) and the vendor FP32 GEMM."""
    import time
    import torch
    import fp32_emulated_gemm_amd as fe
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    out = {}

    def run(name, f, flops, products):
        f()
        torch.cuda.synchronize()
        clocks, calls = [], 0
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.time()
        e0.record(stream)
        while time.time() - t0 < seconds:
            for _ in range(5):
                f()
            calls += 5
            if time.time() - t0 > seconds / 2 and len(clocks) < 2:
                clocks.append(engine_clock_mhz())
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / calls
        tf = flops / ms / 1e9
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "calls": calls,
                     "bf16_frac_of_peak": round(tf * products / MI355X_BF16_DENSE_TFLOPS, 4) if products else None,
                     "sclk_mhz": clocks}
        print(name, out[name], file=sys.stderr, flush=True)

    g = torch.Generator(device="cuda").manual_seed(11)
    for n in (8192, 4096):
        fl = 2.0 * n ** 3
        for dist in ("normal", "uniform"):
            if dist == "normal":
                A = torch.randn((n, n), device="cuda", generator=g)
                B = torch.randn((n, n), device="cuda", generator=g)
            else:
                A = torch.rand((n, n), device="cuda", generator=g) * 2 - 1
                B = torch.rand((n, n), device="cuda", generator=g) * 2 - 1
            Ab, Bb = A.bfloat16(), B.bfloat16()
            Cb = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
            C = torch.empty((n, n), device="cuda")
            run(f"torch_bf16_{n}^3_{dist}", lambda: torch.matmul(Ab, Bb, out=Cb), fl, 1)
            run(f"sgemm_bf16x9_{n}^3_{dist}", lambda: fe.sgemm_bf16x9(n, n, n, A, n, B, n, C, n, sp), fl, 9)
            if dist == "normal":
                run(f"torch_fp32_{n}^3_{dist}", lambda: torch.matmul(A, B, out=C), fl, 0)
            del A, B, Ab, Bb, Cb, C
            torch.cuda.empty_cache()
    print(json.dumps({"sustained_seconds_each": seconds, "bf16_dense_peak_tflops": MI355X_BF16_DENSE_TFLOPS,
                      "runs": out}), flush=True)


def context_timings(fe, torch, Xd, Hd, W1d, W2d, C1, C2, M, D, F, stream, sp):
    """torch.matmul FP32 and the fused-B entry point on the same GEMMs (context only)."""
    res = {}
    fl = 2.0 * M * F * D
    # the platform's BF16 GEMM on the same shapes: one product per multiply-add
    # (memory-bound here), against the emulation's nine on the same bytes
    res["torch_bf16_same_shapes"] = vendor_bf16(torch, stream, {"X@W1": (M, F, D), "H@W2": (M, D, F)}, 5)
    t = timed(lambda: torch.matmul(Xd, W1d, out=C1), stream, 5)
    res["torch_fp32_X@W1_tflops"] = round(fl / t / 1e9, 2)
    t = timed(lambda: torch.matmul(Hd, W2d, out=C2), stream, 5)
    res["torch_fp32_H@W2_tflops"] = round(fl / t / 1e9, 2)
    t = timed(lambda: fe.sgemm_bf16x9(M, F, D, Xd, D, W1d, F, C1, F, sp), stream, 5)
    res["sgemm_bf16x9_X@W1_tflops"] = round(fl / t / 1e9, 2)
    t = timed(lambda: fe.sgemm_bf16x9(M, D, F, Hd, F, W2d, D, C2, D, sp), stream, 5)
    res["sgemm_bf16x9_H@W2_tflops"] = round(fl / t / 1e9, 2)
    # the linear layer built on the same planes: forward with bias, and the input
    # gradient dX = dY W1 (W1's N x K planes read as K x N)
    W1t_ = W1d.t().contiguous()                      # [out][in]
    W1t_planes = fe.split(W1t_)
    bias1 = torch.zeros(F, dtype=torch.float32, device=Xd.device)
    t = timed(lambda: fe.sgemm_emu_linear(M, F, D, Xd, D, *W1t_planes, D, bias1, fe.SGEMM_EMU_ACT_NONE, C1, F, 5, sp), stream, 5)
    res["linear_fwd_X@W1^T+b_tflops"] = round(fl / t / 1e9, 2)
    t = timed(lambda: fe.sgemm_emu_linear(M, F, D, Xd, D, *W1t_planes, D, bias1, fe.SGEMM_EMU_ACT_GELU, C1, F, 5,
                                          sp), stream, 5)
    res["linear_fwd_gelu(X@W1^T+b)_tflops"] = round(fl / t / 1e9, 2)
    t = timed(lambda: fe.sgemm_emu_presplit_b(M, D, F, C1, F, *W1t_planes, D, fe.SGEMM_EMU_B_KN, C2, D, 5, sp),
              stream, 5)
    res["linear_dX=dY@W1_kn_planes_tflops"] = round(fl / t / 1e9, 2)
    W1_planes = fe.split_t(W1t_)                    # planes of (W1t_)^T: N x K for dY W1t_
    t = timed(lambda: fe.sgemm_emu_presplit_b(M, D, F, C1, F, *W1_planes, F, fe.SGEMM_EMU_B_NK, C2, D, 5, sp),
              stream, 5)
    res["linear_dX=dY@W1_tflops"] = round(fl / t / 1e9, 2)
    # band-drop / product-count ablations on X @ W1 (bf16 work scales with the product count)
    for nb in (4, 3, 2, 1):
        t = timed(lambda: fe.sgemm_emu_presplit_b(M, F, D, Xd, D, *W1t_planes, D, fe.SGEMM_EMU_B_NK, C1, F, nb,
                                                  sp), stream, 5)
        res[f"ablation_X@W1_nbands{nb}_{fe.sgemm_emu_products(nb)}products_tflops"] = round(fl / t / 1e9, 2)
    # the standalone split kernel on X (552960 x 256): 4 bytes read + 6 written per element
    Xp = [torch.empty((M, D), dtype=torch.int16, device=Xd.device) for _ in range(3)]
    t = timed(lambda: fe.split_f32_bf16x3(M, D, Xd, D, *Xp, D, sp), stream, 10)
    res["split_X_ms"] = round(t, 4)
    res["split_X_GBps"] = round(10.0 * M * D / t / 1e6, 1)
    res["split_X_frac_of_8TBps"] = round(10.0 * M * D / t / 1e6 / MI355X_HBM_GBS, 3)
    # what a plain device copy of the same bytes reaches on this GPU (8 B per element
    # of X moved), the practical ceiling for an HBM-bound stream
    Xc = torch.empty_like(Xd)
    t = timed(lambda: Xc.copy_(Xd), stream, 10)
    res["copy_X_GBps"] = round(8.0 * M * D / t / 1e6, 1)
    res["split_X_vs_copy"] = round(res["split_X_GBps"] / res["copy_X_GBps"], 3)
    del Xp, Xc
    q = 4096
    Q = torch.rand((q, q), device="cuda") * 2 - 1
    Qp = [torch.empty((q, q), dtype=torch.int16, device="cuda") for _ in range(3)]
    t = timed(lambda: fe.split_f32_bf16x3(q, q, Q, q, *Qp, q, sp), stream, 20)
    res["split_4096^2_GBps"] = round(10.0 * q * q / t / 1e6, 1)
    del Q, Qp
    # the small shapes: 256^3, the PET GEMMs of a 192-atom system (6144 rows) and a
    # grid of 1.1 waves of tiles (stream-K by the cost model)
    for name, (m, nn, k) in (("256^3", (256, 256, 256)), ("6144x1024x256", (6144, 1024, 256)),
                             ("6144x256x1024", (6144, 256, 1024)), ("3072x1536x1024", (3072, 1536, 1024))):
        A = torch.randn((m, k), device="cuda")
        B = torch.randn((k, nn), device="cuda") / k ** 0.5
        C = torch.empty((m, nn), device="cuda")
        Bt_planes = fe.split(B.t().contiguous())
        fs = 2.0 * m * nn * k
        ms = settled_ms({
            "sgemm_bf16x9": lambda: fe.sgemm_bf16x9(m, nn, k, A, k, B, nn, C, nn, sp),
            "presplit_nk": lambda: fe.sgemm_emu_presplit_b(m, nn, k, A, k, *Bt_planes, k, fe.SGEMM_EMU_B_NK, C, nn,
                                                           5, sp),
            "performant": lambda: fe.sgemm_emu_ex(m, nn, k, A, k, B, nn, C, nn, 5, fe.SGEMM_EMU_PERFORMANT, sp),
            "torch_fp32": lambda: torch.matmul(A, B, out=C)}, stream, 20, warmup_s=0.3)
        for entry, t in ms.items():
            res[f"{entry}_{name}_tflops"] = round(fs / t / 1e9, 2)
        del A, B, C, Bt_planes
    n = 4096
    g = torch.Generator(device="cuda").manual_seed(1)
    A = torch.rand((n, n), device="cuda", generator=g) * 2 - 1
    B = torch.rand((n, n), device="cuda", generator=g) * 2 - 1
    C = torch.empty((n, n), device="cuda")
    t = timed(lambda: fe.sgemm_bf16x9(n, n, n, A, n, B, n, C, n, sp), stream, 10)
    res["sgemm_bf16x9_4096^3_tflops"] = round(2.0 * n ** 3 / t / 1e9, 2)
    # cold: A and B (128 MB) fit in the 256 MB last-level cache, so each timed
    # call follows a 512 MB write that evicts them (median of 5)
    flush = torch.empty(128 * 1024 * 1024, device="cuda")
    cold = []
    for _ in range(5):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fe.sgemm_bf16x9(n, n, n, A, n, B, n, C, n, sp)
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    res["sgemm_bf16x9_4096^3_cold_tflops"] = round(2.0 * n ** 3 / sorted(cold)[2] / 1e9, 2)
    del flush
    t = timed(lambda: torch.matmul(A, B, out=C), stream, 10)
    res["torch_fp32_4096^3_tflops"] = round(2.0 * n ** 3 / t / 1e9, 2)
    for nb in (4, 3, 2):
        t = timed(lambda: fe.sgemm_emu(n, n, n, A, n, B, n, C, n, nb, sp), stream, 10)
        res[f"ablation_4096^3_nbands{nb}_{fe.sgemm_emu_products(nb)}products_tflops"] = round(2.0 * n ** 3 / t / 1e9, 2)
    del A, B, C
    n = 8192
    A = torch.rand((n, n), device="cuda", generator=g) * 2 - 1
    B = torch.rand((n, n), device="cuda", generator=g) * 2 - 1
    C = torch.empty((n, n), device="cuda")
    t = timed(lambda: fe.sgemm_bf16x9(n, n, n, A, n, B, n, C, n, sp), stream, 5)
    res["sgemm_bf16x9_8192^3_tflops"] = round(2.0 * n ** 3 / t / 1e9, 2)
    t = timed(lambda: torch.matmul(A, B, out=C), stream, 5)
    res["torch_fp32_8192^3_tflops"] = round(2.0 * n ** 3 / t / 1e9, 2)
    del A, B, C
    # the accuracy-stress workload (scales 2^-20..2^20, near-cancelling rows,
    # subnormals) at 8192^3, all nine products and the band-drop ablations
    import workloads
    w = workloads.stress8192()
    A = torch.from_numpy(w["A"]).to("cuda")
    B = torch.from_numpy(w["B"]).to("cuda")
    C = torch.empty((n, n), device="cuda")
    for nb in (5, 4, 3, 2):
        t = timed(lambda: fe.sgemm_emu(n, n, n, A, n, B, n, C, n, nb, sp), stream, 5)
        res[f"stress8192_nbands{nb}_{fe.sgemm_emu_products(nb)}products_tflops"] = round(2.0 * n ** 3 / t / 1e9, 2)
    del A, B, C, w
    # speed-up over the platform's own FP32 GEMM on the same shapes, next to the
    # ratios the pages quote for other hardware (context only)
    res["speedup_vs_torch_fp32"] = {
        "X@W1": round(res["sgemm_bf16x9_X@W1_tflops"] / res["torch_fp32_X@W1_tflops"], 3),
        "H@W2": round(res["sgemm_bf16x9_H@W2_tflops"] / res["torch_fp32_H@W2_tflops"], 3),
        "4096^3": round(res["sgemm_bf16x9_4096^3_tflops"] / res["torch_fp32_4096^3_tflops"], 3),
        "8192^3": round(res["sgemm_bf16x9_8192^3_tflops"] / res["torch_fp32_8192^3_tflops"], 3),
        "6144x1024x256": round(res["sgemm_bf16x9_6144x1024x256_tflops"] / res["torch_fp32_6144x1024x256_tflops"], 3),
        "6144x256x1024": round(res["sgemm_bf16x9_6144x256x1024_tflops"] / res["torch_fp32_6144x256x1024_tflops"], 3),
        "3072x1536x1024": round(res["sgemm_bf16x9_3072x1536x1024_tflops"] / res["torch_fp32_3072x1536x1024_tflops"], 3),
    }
    res["pages_quoted_speedups_other_hardware"] = {
        "BF16x9_vs_FP32_B300_large_PET_GEMMs": "2.2-2.5x", "BF16x9_vs_FP32_B300_4096^3": "2.41x",
        "TF32x3_vs_FP32_A100_PET_GEMMs": "1.7-1.9x"}
    log(f"context: {res}")
    return res


def cpu_baseline(X, W1, H, W2, target_s):
    """The oracle's naive FP32 SGEMM on a row sample of both GEMMs, all host cores."""
    import numpy as np
    import oracle
    M = X.shape[0]
    flops_per_row = 2.0 * (W1.shape[0] * W1.shape[1] + W2.shape[0] * W2.shape[1])

    def run(nrows, fn=oracle.sgemm_naive_f32):
        rows = np.linspace(0, M - 1, nrows).astype(np.int64)
        t = time.perf_counter()
        fn(X, W1, rows=rows)
        fn(H, W2, rows=rows)
        return time.perf_counter() - t

    def sized(fn, seconds):
        probe_rows = 128
        tp = run(probe_rows, fn)
        return int(min(M, max(probe_rows, probe_rows * seconds / max(tp, 1e-6))))

    nrows = sized(oracle.sgemm_naive_f32, target_s)
    t = run(nrows)
    val = flops_per_row * nrows / t / 1e12
    log(f"cpu baseline: {nrows} rows in {t:.2f} s on {oracle.num_threads()} threads")
    # beside it, the oracle's other two products on smaller samples (same rate unit)
    others = {}
    for name, fn in (("fp64_reference", lambda A, B, rows: oracle.gemm_f64(A, B, rows=rows, want_g=False)),
                     ("band_emulation_9_products", oracle.gemm_emu)):
        n = sized(fn, target_s / 4)
        tt = run(n, fn)
        others[name] = {"value": round(flops_per_row * n / tt / 1e12, 5), "rows": n, "seconds": round(tt, 2)}
    log(f"cpu oracle, other products: {others}")
    return {"value": round(val, 5), "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"naive FP32 SGEMM (oracle) on {nrows} of {M} rows of X@W1 and H@W2, "
                      f"{t:.1f} s; value = 2*rows*(256*1024+1024*256)/t",
            "other_oracle_products": others}


if __name__ == "__main__":
    main()
