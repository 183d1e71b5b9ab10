"""Benchmark of the fine-grained FP8 linear layer on one MI355X.

One step = the DeepSeek-V3 dense projections at M = 8192 tokens (q_a
7168->1536, q_b 1536->24576, kv_a 7168->576, o_proj 16384->7168, MLP up
7168->18432 and down 18432->7168; 7.12 TFLOP): for each projection, dynamic
per-token-group activation quantization of x followed by the block-scaled
FP8 GEMM (weights quantized once, before timing).  This is the largest
single-GPU workload of the library.  Inputs are resident in HBM before the
timed region; two input/output sets are rotated between steps so that the
256 MB last-level cache does not hold a step's working set.

Before it, the same measurement runs on the Llama-3-8B prefill linear layers
(M = 4096; q/o 4096x4096, kv 1024x4096, gate/up 14336x4096, down
4096x14336), reported under ``llama_prefill``.

    python bench.py [--gpus 1] [--steps 20] [--warmup 10] [--no-cpu-baseline]
                    [--rows]  (also time weight quant, decode, MoE (grouped
                               and batched layouts), the DeepSeek-V3 shapes
                               at M = 512, the tiny configuration, the
                               power-of-two (UE8M0), static-activation-scale
                               and row-wise (fp8r) rows)

Prints one JSON line.  ``value`` is the whole step's throughput in TFLOP/s
(GEMM FLOPs of the six projections / step time, the activation
quantization included); ``roofline`` is for the GEMM kernels alone (FLOPs /
their launch times measured with HIP events on the launch stream, against
the dense fp8 MFMA peak); ``ceilings`` gives what the matrix cores sustain
on this chip with operands in registers (plain fp8 MFMAs, and the same with
the GEMM's fp32 promotion FMAs), as context for that fraction;
``cpu_baseline`` times the CPU oracle on a row sample of the step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
M_PREFILL = 4096
PREFILL_SHAPES = (("qo", 4096, 4096), ("kv", 1024, 4096), ("gate_up", 14336, 4096),
                  ("down", 4096, 14336))
M_DSV3 = 8192
DSV3_SHAPES = (("q_a", 1536, 7168), ("q_b", 24576, 1536), ("kv_a", 576, 7168),
               ("o_proj", 7168, 16384), ("mlp_up", 18432, 7168), ("mlp_down", 7168, 18432))
CPU_SAMPLE_ROWS = 256    # rows of each DeepSeek-V3 projection the oracle runs
ACT_BYTES_PER_ELEM = 2 + 1 + 4 / 128   # bf16 in, e4m3 out, one fp32 scale per 128


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rows", action="store_true", help="also time the other hot-path rows")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with a plain 512 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


GEMM_SOURCE = os.path.join(ROOT, "block_scaled_fp8_act_amd", "csrc", "gemm_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "block_gemm_dsv3_m8192_traffic.md")


def progress(msg):
    """One line on stderr per finished part of the run (stdout carries only
    the result line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def source_digest(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per GEMM launch of this workload from the committed rocprofv3
    --pmc summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy kernel),
    or None when the GEMM source has changed since the counters were taken."""
    try:
        fields = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
        if fields.get("gemm_source_sha256_16") != source_digest(GEMM_SOURCE):
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def gen_inputs(torch, dev, seed):
    """Seeded synthetic Llama-3-8B-shaped inputs generated on the device:
    x ~ N(0,1) with 1 % of channels x20 (bf16); W ~ N(0, 0.02) (bf16)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    xs, ws = [], []
    for name, N, K in PREFILL_SHAPES:
        x = torch.randn((M_PREFILL, K), generator=g, device=dev, dtype=torch.float32)
        cols = torch.randperm(K, generator=g, device=dev)[: round(0.01 * K)]
        x[:, cols] *= 20.0
        xs.append(x.to(torch.bfloat16))
        ws.append((torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * 0.02)
                  .to(torch.bfloat16))
    return xs, ws


def gen_inputs_dsv3(torch, dev, seed):
    """Seeded synthetic DeepSeek-V3-shaped inputs generated on the device:
    x ~ N(0,1) with 0.5 % of entries (i.i.d. positions) replaced by
    10 * t(3) (Student t with 3 degrees of freedom, drawn as Z / sqrt(V/3)
    with V a sum of three squared normals); W ~ N(0, 0.01); both bf16."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    xs, ws = [], []
    for name, N, K in DSV3_SHAPES:
        x = torch.randn((M_DSV3, K), generator=g, device=dev, dtype=torch.float32)
        mask = torch.rand((M_DSV3, K), generator=g, device=dev) < 0.005
        n = int(mask.sum())
        z = torch.randn(n, generator=g, device=dev)
        v = torch.randn((n, 3), generator=g, device=dev).square().sum(1)
        x[mask] = 10.0 * z / torch.sqrt(v / 3.0)
        xs.append(x.to(torch.bfloat16))
        del x, mask
        ws.append((torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * 0.01)
                  .to(torch.bfloat16))
    return xs, ws


def cpu_baseline():
    """The CPU oracle (as it stands) on a row sample of the step: for each
    DeepSeek-V3 projection, activation quantization + fp64
    dequantize-then-matmul of CPU_SAMPLE_ROWS rows (weights quantized
    beforehand, as on the GPU; same input distributions).  Returns TFLOP/s
    (GEMM FLOPs of the sample / oracle time) and the BLAS thread count."""
    import numpy as np
    import synth
    from oracle import gemm as og
    from oracle import quant as oq
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    dt, flops = 0.0, 0.0
    for i, (_, N, K) in enumerate(DSV3_SHAPES):
        x, w = synth.dsv3_inputs(i, CPU_SAMPLE_ROWS)
        wq, ws = oq.weight_block_quant(w)
        del w
        t0 = time.perf_counter()
        xq, xs = oq.act_quant_group(x)
        y = og.block_gemm(xq, xs, wq, ws)
        dt += time.perf_counter() - t0
        og.bf16_rne_bits(y)
        flops += 2.0 * CPU_SAMPLE_ROWS * N * K
        del x, wq, ws, xq, xs, y
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except Exception:  # pragma: no cover
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{CPU_SAMPLE_ROWS} of the {M_DSV3} rows of each of the six DeepSeek-V3 "
                      f"projections ({flops / 1e12:.3f} TFLOP, 1/{M_DSV3 // CPU_SAMPLE_ROWS} of "
                      f"the step): act quant + fp64 dequantize-then-matmul, {dt:.1f} s on {cpu} "
                      f"({len(os.sched_getaffinity(0))} CPUs in the affinity mask)"}


def linear_leg(torch, fb, dev, stream, shapes, M, xs0, ws_bf16, steps, warmup):
    """Time a step of linear layers: for each (name, N, K) of `shapes`, the
    activation quantizer on x [M, K] then the block-scaled GEMM against the
    quantized weight, two rotated input sets.  Returns (ms_per_step,
    per-projection act-quant and GEMM times in s, GEMM FLOPs of the step,
    act-quant bytes of the step)."""
    sets = [xs0, [torch.roll(x, 1, 0) for x in xs0]]
    wq, wsc = [], []
    for w in ws_bf16:
        q, s = fb.weight_block_quant(w)
        wq.append(q); wsc.append(s)
    outs = [[(torch.empty((M, K), dtype=torch.uint8, device=dev),
              torch.empty((M, K // 128), dtype=torch.float32, device=dev),
              torch.empty((M, N), dtype=torch.bfloat16, device=dev))
             for (_, N, K) in shapes] for _ in sets]
    # the GEMM's workspace (stream-K tail or K split, when the library plans
    # one for a shape), allocated once before timing
    need = max(fb.fp8_block_gemm_workspace_bytes(M, N, K) for (_, N, K) in shapes)
    work = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def launch(i, p, ev):
        xq, xsc, y = outs[i % 2][p]
        if ev is not None:
            ev[0].record(stream)
        fb.fp8_act_quant_group(sets[i % 2][p], xq, xsc)
        if ev is not None:
            ev[1].record(stream)
        fb.fp8_block_gemm_ws(xq, xsc, wq[p], wsc[p], y, work)
        if ev is not None:
            ev[2].record(stream)

    wall, act_s, gemm_s = run_leg(torch, stream, launch, len(shapes), steps, warmup)
    flops = sum(2.0 * M * N * K for (_, N, K) in shapes)
    act_bytes = sum(M * K * ACT_BYTES_PER_ELEM for (_, N, K) in shapes)
    del sets, outs, wq, wsc, work
    return wall, act_s, gemm_s, flops, act_bytes


def leg_summary(shapes, M, wall, act_s, gemm_s, flops, act_bytes):
    gemm_tflops = flops / sum(gemm_s) / 1e12
    act_gbs = act_bytes / sum(act_s) / 1e9
    return {
        "ms_per_step": round(wall * 1e3, 4),
        "TFLOP/s": round(flops / wall / 1e12, 2),
        "gemm": {"achieved": round(gemm_tflops, 2), "unit": "TFLOP/s",
                 "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4)},
        "act_quant": {"achieved": round(act_gbs, 1), "unit": "GB/s",
                      "frac": round(act_gbs / PEAK_HBM_GBS, 4)},
        "per_projection": {
            name: {"act_quant_us": round(act_s[p] * 1e6, 2),
                   "act_quant_GB/s": round(M * K * ACT_BYTES_PER_ELEM / act_s[p] / 1e9, 1),
                   "gemm_us": round(gemm_s[p] * 1e6, 2),
                   "gemm_TFLOP/s": round(2.0 * M * N * K / gemm_s[p] / 1e12, 1),
                   "gemm_frac": round(2.0 * M * N * K / gemm_s[p] / 1e12 / PEAK_FP8_TFLOPS, 4)}
            for p, (name, N, K) in enumerate(shapes)},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding of this path is designed, not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_fp8_act_amd as fb

    if not os.path.exists(fb.lib_path()):
        raise RuntimeError("libfp8blk.so is not built (python -m block_scaled_fp8_act_amd.build)")
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    # --- Llama-3-8B prefill (reported beside the headline) ------------------
    xs0, ws_bf16 = gen_inputs(torch, dev, 3000)
    llama = leg_summary(PREFILL_SHAPES, M_PREFILL,
                        *linear_leg(torch, fb, dev, stream, PREFILL_SHAPES, M_PREFILL, xs0,
                                    ws_bf16, args.steps, args.warmup))
    del xs0, ws_bf16
    progress("Llama-3-8B prefill leg done")

    # --- headline: DeepSeek-V3 dense projections at M = 8192 ---------------
    xs0, ws_bf16 = gen_inputs_dsv3(torch, dev, 4000)
    wall, act_s, gemm_s, step_flops, act_bytes = linear_leg(
        torch, fb, dev, stream, DSV3_SHAPES, M_DSV3, xs0, ws_bf16, args.steps, args.warmup)
    del xs0, ws_bf16
    torch.cuda.empty_cache()
    head = leg_summary(DSV3_SHAPES, M_DSV3, wall, act_s, gemm_s, step_flops, act_bytes)
    progress("DeepSeek-V3 M = 8192 leg done")
    gemm_tflops = step_flops / sum(gemm_s) / 1e12
    act_gbs = act_bytes / sum(act_s) / 1e9
    value = step_flops / wall / 1e12

    out = {
        "metric": "fp8_block_gemm TFLOP/s (% dense-fp8 MFMA peak); act-quant GB/s (% HBM)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp8_e4m3 -> fp32 accumulate, bf16 out",
        "data": "synthetic (seeded; DeepSeek-V3 dense projection shapes, x ~ N(0,1) with 0.5% "
                "entries 10*t(3), W ~ N(0,0.01))",
        "config": {"workload": "DeepSeek-V3 dense projections at M=8192: act quant + "
                               "block-scaled FP8 GEMM per projection",
                   "M": M_DSV3, "shapes_NxK": [[N, K] for (_, N, K) in DSV3_SHAPES],
                   "block": 128, "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "kernel": "block-scaled GEMM (block_gemm_kernel; o_proj and MLP down: "
                      "block_gemm_sk_kernel + sk_reduce_kernel, the stream-K tail; kv_a: "
                      "the 128x128 tile)",
            "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "traffic": measured_traffic(),
            "traffic_unit": "HBM bytes per launch (mean over the 6 projections)",
            "algorithmic": "2*M*N*K FLOP per launch, summed over the six projections",
        },
        "act_quant": {"achieved": round(act_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(act_gbs / PEAK_HBM_GBS, 4), "bound": "hbm"},
        "per_projection": head["per_projection"],
        "llama_prefill": llama,
    }
    out["act_quant"]["standalone"] = act_quant_alone(torch, fb, dev, stream)
    out["ceilings"] = ceilings(torch, stream, gemm_tflops)
    progress("quantizer alone and matrix-core ceilings done")
    if args.rows:
        out["rows"] = other_rows(torch, fb, dev, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
        progress("CPU baseline done")
    if args.calibrate_copy:
        src = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        t = _time(torch, stream, lambda: dst.copy_(src), iters=10, warm=1)
        out["copy_512MiB_GBps"] = round(2 * src.numel() / t / 1e9, 1)
    print(json.dumps(out), flush=True)


def run_leg(torch, stream, launch, n_proj, steps, warmup):
    """Time one prefill leg.  launch(i, p, ev) enqueues projection p of step
    i (activation quantization, then GEMM), recording ev[0] before, ev[1]
    between and ev[2] after the two kernels when ev is given.  Returns the
    wall time per step (s) and the mean in-step event times of each
    projection's two kernels (s); all event-timed steps are enqueued back to
    back with one synchronisation at the end."""
    for i in range(warmup):
        for p in range(n_proj):
            launch(i, p, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for p in range(n_proj):
            launch(i, p, None)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_proj)]
           for _ in range(steps)]
    for i in range(steps):
        for p in range(n_proj):
            launch(i, p, evs[i][p])
    torch.cuda.synchronize()
    quant = [sum(ev[p][0].elapsed_time(ev[p][1]) for ev in evs) / steps * 1e-3 for p in range(n_proj)]
    gemm = [sum(ev[p][1].elapsed_time(ev[p][2]) for ev in evs) / steps * 1e-3 for p in range(n_proj)]
    return wall, quant, gemm


ROTATE_BYTES = 600 * 2 ** 20   # > twice the 256 MB MALL


def _weight_copies(wq, *extra):
    """Enough copies of a quantized weight (codes and scales) that the bytes
    touched between two uses of one copy exceed twice the MALL: the decode
    timings then stream the weights from HBM, not from the cache."""
    n = max(2, -(-ROTATE_BYTES // wq.numel()))
    return [(wq.clone(), *[e.clone() for e in extra]) for _ in range(n)]


def _rotating(copies, fn):
    """fn(*copy) over the copies in turn, one per call."""
    k = [0]

    def call():
        c = copies[k[0] % len(copies)]
        k[0] += 1
        fn(*c)
    return call


def act_quant_alone(torch, fb, dev, stream):
    """The activation quantizer on its own at the step's two shapes: 20
    launches back to back between two HIP events, cycling through input
    copies that add up to over 400 MB (so each call reads from HBM, not the
    256 MB MALL).  The in-step figure brackets each launch with events, which
    adds the dispatch gap to every ~11 us kernel.  Beside each, the runtime's
    own device-to-device copy of the same byte count (read + write), the
    practical HBM ceiling at that size."""
    res = {}
    g = torch.Generator(device=dev)
    g.manual_seed(4000)
    for K in (4096, 14336):
        ncopy = max(2, -(-400 * 2**20 // (M_PREFILL * K * 2)))
        xs = [torch.randn((M_PREFILL, K), generator=g, device=dev, dtype=torch.float32)
              .to(torch.bfloat16) for _ in range(ncopy)]
        xq = torch.empty((M_PREFILL, K), dtype=torch.uint8, device=dev)
        xsc = torch.empty((M_PREFILL, K // 128), dtype=torch.float32, device=dev)
        k = [0]

        def run():
            fb.fp8_act_quant_group(xs[k[0] % ncopy], xq, xsc)
            k[0] += 1
        t = min(_time(torch, stream, run, iters=20, warm=4) for _ in range(3))
        gbs = M_PREFILL * K * ACT_BYTES_PER_ELEM / t / 1e9
        del xs, xq, xsc
        # context: the runtime's device-to-device copy moving the same bytes
        # (half read, half written), sources cycled the same way
        nb = int(M_PREFILL * K * ACT_BYTES_PER_ELEM) // 2
        srcs = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(ncopy)]
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        k[0] = 0

        def copy():
            dst.copy_(srcs[k[0] % ncopy])
            k[0] += 1
        tc = min(_time(torch, stream, copy, iters=20, warm=4) for _ in range(3))
        del srcs, dst
        res[f"{M_PREFILL}x{K}"] = {"us": round(t * 1e6, 2), "GB/s": round(gbs, 1),
                                   "frac": round(gbs / PEAK_HBM_GBS, 4),
                                   "copy_same_bytes_us": round(tc * 1e6, 2),
                                   "frac_of_copy": round(tc / t, 4)}
    return res


CEIL_BLOCKS = 2048   # 8 workgroups of 8 waves per CU
CEIL_ITERS = 500     # 32 MFMAs per wave per iteration (~3.5 ms per launch)


def ceilings(torch, stream, gemm_tflops):
    """Ceilings measured on this chip.  Matrix cores (libfp8ceil.so; every
    operand in registers, no memory traffic in the loop): back-to-back fp8
    MFMAs, and the same MFMAs each followed by the fp32 promotion (one FMA per
    output per 128-wide K block) that the block GEMM's inner loop carries;
    each once on near-constant operand registers and once on operands that
    take fresh random bits every iteration (the switching activity of real
    data), with the engine clock each held (shader-clock over wall-clock
    ticks, read inside the kernel).  HBM: a plain 512 MiB device-to-device
    copy.  roofline.frac and act_quant.frac stay against the published
    peaks; these are context."""
    import ctypes
    path = os.path.join(ROOT, "block_scaled_fp8_act_amd", "lib", "libfp8ceil.so")
    if not os.path.exists(path):
        from block_scaled_fp8_act_amd import build
        build.build()
    lib = ctypes.CDLL(path)
    f = lib.fp8ceil_mfma
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    lib.fp8ceil_wall_clock_khz.restype = ctypes.c_int
    wall_khz = lib.fp8ceil_wall_clock_khz()
    out = torch.empty(CEIL_BLOCKS * 512, dtype=torch.float32, device="cuda")
    clk = torch.zeros(CEIL_BLOCKS * 2, dtype=torch.int64, device="cuda")
    flops = CEIL_BLOCKS * 8 * CEIL_ITERS * 32 * 65536.0
    res = {}
    clocks = {}
    for mode, key in ((0, "mfma_fp8"), (1, "mfma_fp8_with_fp32_promotion"),
                      (2, "mfma_fp8_random_operands"),
                      (3, "mfma_fp8_with_fp32_promotion_random_operands")):
        def run(c=None):
            rc = f(mode, out.data_ptr(), c, CEIL_BLOCKS, CEIL_ITERS, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"fp8ceil_mfma failed ({rc})")
        best = min(_time(torch, stream, run, iters=3, warm=1) for _ in range(3))
        res[key] = round(flops / best / 1e12, 1)
        if wall_khz > 0:
            run(clk.data_ptr())
            torch.cuda.synchronize()
            ticks = clk.view(CEIL_BLOCKS, 2).double().sum(0)
            clocks[key] = round(float(ticks[0] / ticks[1]) * wall_khz / 1e6, 3)
    res["unit"] = "TFLOP/s"
    res["clock_GHz"] = clocks
    res["gemm_frac_of_mfma_fp8"] = round(gemm_tflops / res["mfma_fp8"], 4)
    res["gemm_frac_of_promotion_ceiling"] = round(gemm_tflops / res["mfma_fp8_with_fp32_promotion"], 4)
    res["gemm_frac_of_promotion_ceiling_random_operands"] = round(
        gemm_tflops / res["mfma_fp8_with_fp32_promotion_random_operands"], 4)
    # HBM: the runtime's own device-to-device copy of 512 MiB (read + write)
    src = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t = min(_time(torch, stream, lambda: dst.copy_(src), iters=5, warm=1) for _ in range(3))
    res["hbm_copy_512MiB_GBps"] = round(2 * src.numel() / t / 1e9, 1)
    del src, dst
    return res


def _time(torch, stream, fn, iters=20, warm=3):
    for _ in range(warm):
        fn()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(iters):
        fn()
    e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters * 1e-3


def other_rows(torch, fb, dev, stream):
    """Weight quantization, decode GEMMs and the grouped MoE GEMM."""
    import numpy as np
    import synth
    rows = {}
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    # weight quant: DeepSeek-V3 18432x7168 (largest single weight)
    w = (torch.randn((18432, 7168), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    q = torch.empty((18432, 7168), dtype=torch.uint8, device=dev)
    s = torch.empty((144, 56), dtype=torch.float32, device=dev)
    t = _time(torch, stream, lambda: fb.fp8_weight_block_quant(w, q, s))
    rows["weight_quant_18432x7168"] = {"us": round(t * 1e6, 2), "GB/s": round(18432 * 7168 * 3 / t / 1e9, 1)}
    del w, q, s
    # decode GEMMs (HBM-bound): M = 1, 4, 16 (the Llama-3-8B decode
    # configuration) and 32, 64 (small batches, still the decode kernel),
    # weights rotated through HBM
    for name, N, K in PREFILL_SHAPES:
        wq, wsc = fb.weight_block_quant((torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16))
        copies = _weight_copies(wq, wsc)
        for Md in (1, 4, 16, 32, 64):
            x = torch.randn((Md, K), generator=g, device=dev).to(torch.bfloat16)
            xq, xsc = fb.act_quant_group(x)
            y = torch.empty((Md, N), dtype=torch.bfloat16, device=dev)
            t = _time(torch, stream, _rotating(copies, lambda w, s: fb.fp8_block_gemm(xq, xsc, w, s, y)))
            byts = N * K + Md * K + 2 * Md * N
            rows[f"decode_M{Md}_{name}"] = {"us": round(t * 1e6, 2), "GB/s": round(byts / t / 1e9, 1),
                                            "frac_hbm": round(byts / t / 1e9 / PEAK_HBM_GBS, 4)}
            need = fb.fp8_block_gemm_workspace_bytes(Md, N, K)
            if need:
                # long K: four slabs per workgroup, K split over workgroups
                work = torch.empty(need, dtype=torch.uint8, device=dev)
                t = _time(torch, stream, _rotating(
                    copies, lambda w, s: fb.fp8_block_gemm_ws(xq, xsc, w, s, y, work)))
                rows[f"decode_M{Md}_{name}"].update(
                    {"split_k_us": round(t * 1e6, 2), "split_k_GB/s": round(byts / t / 1e9, 1)})
                del work
        del copies
    progress("rows: weight quant and decode GEMMs done")
    rows.update(ue8m0_rows(torch, fb, dev, stream, g))
    rows.update(static_rows(torch, fb, dev, stream))
    rows.update(rowwise_rows(torch, fb, dev, stream))
    progress("rows: UE8M0, static and row-wise legs done")
    # the whole decode linear layer from bf16 x (M = 16): one fused kernel
    # against the two launches (act quant + GEMM); weights rotated
    for name, N, K in PREFILL_SHAPES:
        x = torch.randn((16, K), generator=g, device=dev).to(torch.bfloat16)
        wq, wsc = fb.weight_block_quant((torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16))
        y = torch.empty((16, N), dtype=torch.bfloat16, device=dev)
        xq = torch.empty((16, K), dtype=torch.uint8, device=dev)
        xsc = torch.empty((16, K // 128), dtype=torch.float32, device=dev)
        copies = _weight_copies(wq, wsc)

        def two(w, s):
            fb.fp8_act_quant_group(x, xq, xsc)
            fb.fp8_block_gemm(xq, xsc, w, s, y)
        t1 = _time(torch, stream, _rotating(copies, lambda w, s: fb.fp8_linear(x, w, s, y)))
        t2 = _time(torch, stream, _rotating(copies, two))
        t3 = _time(torch, stream, _rotating(copies, lambda w, s: fb.fp8_linear(x, w, s, y, xq, xsc)))
        del copies
        rows[f"decode_linear_M16_{name}"] = {"fused_us": round(t1 * 1e6, 2),
                                             "two_launch_us": round(t2 * 1e6, 2),
                                             "fp8_linear_with_workspace_us": round(t3 * 1e6, 2)}
    # the decode step (the four projections at M = 16, each one fp8_linear
    # call) launched eagerly and replayed as one captured HIP graph; the same
    # fixed weights in both legs
    lin = []
    for name, N, K in PREFILL_SHAPES:
        x = torch.randn((16, K), generator=g, device=dev).to(torch.bfloat16)
        wq, wsc = fb.weight_block_quant((torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16))
        lin.append((x, wq, wsc, torch.empty((16, N), dtype=torch.bfloat16, device=dev),
                    torch.empty((16, K), dtype=torch.uint8, device=dev),
                    torch.empty((16, K // 128), dtype=torch.float32, device=dev)))

    def dec_step():
        for x, wq, wsc, y, xq, xsc in lin:
            fb.fp8_linear(x, wq, wsc, y, xq, xsc)
    t_eager = _time(torch, stream, dec_step)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        dec_step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            dec_step()
    torch.cuda.synchronize()
    t_graph = _time(torch, stream, graph.replay)
    rows["decode_step_M16"] = {"eager_us": round(t_eager * 1e6, 2), "graph_us": round(t_graph * 1e6, 2)}
    del lin, graph
    progress("rows: decode linear layers done")
    # grouped MoE (32 experts, Zipf top-8 routing of 4096 tokens)
    _, off = synth.moe_routing()
    total = int(off[-1])
    offd = torch.from_numpy(off).to(dev)
    for which, (name, N, K) in enumerate(synth.MOE_SHAPES):
        x = torch.randn((total, K), generator=g, device=dev).to(torch.bfloat16)
        xq, xsc = fb.act_quant_group(x)
        wq = torch.empty((32, N, K), dtype=torch.uint8, device=dev)
        wsc = torch.empty((32, -(-N // 128), K // 128), dtype=torch.float32, device=dev)
        for e in range(32):
            fb.fp8_weight_block_quant((torch.randn((N, K), generator=g, device=dev) * 0.01).to(torch.bfloat16),
                                      wq[e], wsc[e])
        y = torch.empty((total, N), dtype=torch.bfloat16, device=dev)
        t = _time(torch, stream, lambda: fb.fp8_grouped_block_gemm(xq, xsc, wq, wsc, offd, y), iters=10)
        rows[f"moe_{name}"] = {"us": round(t * 1e6, 2), "TFLOP/s": round(2.0 * total * N * K / t / 1e12, 1)}
        # the same tokens in the batched layout: capacity = the largest load
        # rounded up to 256 rows, counts = the loads
        counts = np.diff(off).astype(np.int32)
        cap = int(-(-int(counts.max()) // 256) * 256)
        xb = torch.zeros((32, cap, K), dtype=torch.uint8, device=dev)
        sb = torch.zeros((32, cap, K // 128), dtype=torch.float32, device=dev)
        for e in range(32):
            xb[e, :counts[e]] = xq[off[e]:off[e + 1]]
            sb[e, :counts[e]] = xsc[off[e]:off[e + 1]]
        yb = torch.empty((32, cap, N), dtype=torch.bfloat16, device=dev)
        cnt = torch.from_numpy(counts).to(dev)
        t = _time(torch, stream, lambda: fb.fp8_batched_block_gemm(xb, sb, wq, wsc, cnt, yb), iters=10)
        rows[f"moe_batched_{name}"] = {"us": round(t * 1e6, 2), "capacity": cap,
                                       "TFLOP/s": round(2.0 * total * N * K / t / 1e12, 1)}
        del xb, sb, yb
    # SwiGLU + activation quantizer ahead of the MoE down projection: the
    # gate/up output [32768, 2 * 2048] -> codes [32768, 2048] and scales in
    # one kernel, against torch's SwiGLU (bf16 h through memory) followed by
    # the activation quantizer; three rotating inputs (805 MB)
    I = synth.MOE_INTERMEDIATE
    gus = [(torch.randn((total, 2 * I), generator=g, device=dev) * synth.MOE_GATE_UP_STD).to(torch.bfloat16)
           for _ in range(3)]
    xq = torch.empty((total, I), dtype=torch.uint8, device=dev)
    xsc = torch.empty((total, I // 128), dtype=torch.float32, device=dev)
    h = torch.empty((total, I), dtype=torch.bfloat16, device=dev)
    k = [0]

    def fused():
        k[0] += 1
        fb.fp8_swiglu_act_quant(gus[k[0] % 3], xq, xsc)

    def unfused():
        k[0] += 1
        gu = gus[k[0] % 3]
        torch.mul(torch.nn.functional.silu(gu[:, :I]), gu[:, I:], out=h)
        fb.fp8_act_quant_group(h, xq, xsc)
    t1 = _time(torch, stream, fused)
    t2 = _time(torch, stream, unfused)
    byts = total * I * (4 + 1) + total * (I // 128) * 4
    rows["moe_swiglu_act_quant_32768x2048"] = {
        "us": round(t1 * 1e6, 2), "GB/s": round(byts / t1 / 1e9, 1),
        "torch_swiglu_then_act_quant_us": round(t2 * 1e6, 2)}
    del gus, xq, xsc, h
    # DeepSeek-V3 dense projections at M = 512: act quant + GEMM per shape;
    # where the library plans a K split over workgroups (small grids), the
    # plain GEMM beside the split one (its workspace allocated before timing)
    M = 512
    for name, N, K in DSV3_SHAPES:
        x = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        xq, xsc = fb.act_quant_group(x)
        wq, wsc = fb.weight_block_quant(
            (torch.randn((N, K), generator=g, device=dev) * 0.01).to(torch.bfloat16))
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        need = fb.fp8_block_gemm_workspace_bytes(M, N, K)
        work = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        ta = _time(torch, stream, lambda: fb.fp8_act_quant_group(x, xq, xsc))
        t0 = _time(torch, stream, lambda: fb.fp8_block_gemm(xq, xsc, wq, wsc, y))
        fl = 2.0 * M * N * K
        r = {"act_quant_us": round(ta * 1e6, 2), "gemm_us": round(t0 * 1e6, 2),
             "gemm_TFLOP/s": round(fl / t0 / 1e12, 1),
             "gemm_frac": round(fl / t0 / 1e12 / PEAK_FP8_TFLOPS, 4)}
        if need:
            t1 = _time(torch, stream, lambda: fb.fp8_block_gemm_ws(xq, xsc, wq, wsc, y, work))
            r.update({"split_us": round(t1 * 1e6, 2), "split_TFLOP/s": round(fl / t1 / 1e12, 1),
                      "split_frac": round(fl / t1 / 1e12 / PEAK_FP8_TFLOPS, 4),
                      "workspace_MB": round(need / 1e6, 2)})
        rows[f"dsv3_{name}_M512"] = r
        del x, xq, xsc, wq, wsc, y, work
    progress("rows: MoE, SwiGLU and DeepSeek-V3 M = 512 done")
    # the tiny configuration (x[16,512], W[512,512]): one linear layer
    xt = torch.randn((16, 512), generator=g, device=dev).to(torch.bfloat16)
    wq, wsc = fb.weight_block_quant(torch.randn((512, 512), generator=g, device=dev).to(torch.bfloat16))
    yt = torch.empty((16, 512), dtype=torch.bfloat16, device=dev)
    xq = torch.empty((16, 512), dtype=torch.uint8, device=dev)
    xsc = torch.empty((16, 4), dtype=torch.float32, device=dev)
    t1 = _time(torch, stream, lambda: fb.fp8_linear(xt, wq, wsc, yt), iters=100)

    def two_tiny():
        fb.fp8_act_quant_group(xt, xq, xsc)
        fb.fp8_block_gemm(xq, xsc, wq, wsc, yt)
    t2 = _time(torch, stream, two_tiny, iters=100)
    rows["tiny_16x512x512"] = {"fp8_linear_us": round(t1 * 1e6, 2), "two_launch_us": round(t2 * 1e6, 2)}
    # decode K split (four slabs per workgroup, K over workgroups) against
    # the unsplit decode GEMM: DeepSeek-V3 o_proj at M = 16 and Llama down
    # at M = 9, 12, 16; weights rotated through HBM
    for name, N, K, Ms in (("dsv3_o_proj", 7168, 16384, (16,)), ("llama_down", 4096, 14336, (9, 12, 16))):
        wq, wsc = fb.weight_block_quant((torch.randn((N, K), generator=g, device=dev) * 0.01).to(torch.bfloat16))
        copies = _weight_copies(wq, wsc)
        for Md in Ms:
            x = torch.randn((Md, K), generator=g, device=dev).to(torch.bfloat16)
            xq, xsc = fb.act_quant_group(x)
            y = torch.empty((Md, N), dtype=torch.bfloat16, device=dev)
            need = fb.fp8_block_gemm_workspace_bytes(Md, N, K)
            work = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            tp = _time(torch, stream, _rotating(copies, lambda w, s: fb.fp8_block_gemm(xq, xsc, w, s, y)))
            ts = _time(torch, stream, _rotating(copies, lambda w, s: fb.fp8_block_gemm_ws(xq, xsc, w, s, y, work)))
            rows[f"decode_split_{name}_M{Md}"] = {"plain_us": round(tp * 1e6, 2),
                                                  "split_us": round(ts * 1e6, 2), "planned": bool(need)}
        del copies
    return rows


def rowwise_rows(torch, fb, dev, stream):
    """Row-wise ("fp8r") scales: the same prefill step with the row-wise
    quantizer (per token) and the row-scaled GEMM; weights quantized
    row-wise once."""
    xs0, ws_bf16 = gen_inputs(torch, dev, 3000)
    sets = [xs0, [torch.roll(x, 1, 0) for x in xs0]]
    wq, wsc = zip(*[fb.rowwise_quant(w) for w in ws_bf16])
    del ws_bf16
    outs = [[(torch.empty((M_PREFILL, K), dtype=torch.uint8, device=dev),
              torch.empty((M_PREFILL,), dtype=torch.float32, device=dev),
              torch.empty((M_PREFILL, N), dtype=torch.bfloat16, device=dev))
             for (_, N, K) in PREFILL_SHAPES] for _ in sets]
    flops = sum(2.0 * M_PREFILL * N * K for (_, N, K) in PREFILL_SHAPES)

    def launch(i, p, ev):
        xq, xs, y = outs[i % 2][p]
        if ev is not None:
            ev[0].record(stream)
        fb.fp8_rowwise_quant(sets[i % 2][p], xq, xs)
        if ev is not None:
            ev[1].record(stream)
        fb.fp8_rowwise_gemm(xq, xs, wq[p], wsc[p], y)
        if ev is not None:
            ev[2].record(stream)

    dt, ta, tg = run_leg(torch, stream, launch, len(PREFILL_SHAPES), 30, 10)
    per = {name: {"act_quant_us": round(ta[p] * 1e6, 2),
                  "act_quant_GB/s": round(3 * M_PREFILL * K / ta[p] / 1e9, 1),
                  "gemm_us": round(tg[p] * 1e6, 2),
                  "gemm_TFLOP/s": round(2.0 * M_PREFILL * N * K / tg[p] / 1e12, 1)}
           for p, (name, N, K) in enumerate(PREFILL_SHAPES)}
    return {"rowwise_prefill_step": {"ms_per_step": round(dt * 1e3, 4),
                                     "TFLOP/s": round(flops / dt / 1e12, 1),
                                     "gemm_TFLOP/s": round(flops / sum(tg) / 1e12, 1),
                                     "per_projection": per}}


def static_rows(torch, fb, dev, stream):
    """Static (calibrated, per-tensor) activation scale: the same prefill
    step with the static quantizer and GEMM, two rotated input sets."""
    xs0, ws_bf16 = gen_inputs(torch, dev, 3000)
    sets = [xs0, [torch.roll(x, 1, 0) for x in xs0]]
    wq, wsc = zip(*[fb.weight_block_quant(w) for w in ws_bf16])
    del ws_bf16
    # a calibrated scale: the largest |x| of the first set / 448
    scales = [(x.abs().amax().float() / 448.0).reshape(1).contiguous() for x in xs0]
    outs = [[(torch.empty((M_PREFILL, K), dtype=torch.uint8, device=dev),
              torch.empty((M_PREFILL, N), dtype=torch.bfloat16, device=dev))
             for (_, N, K) in PREFILL_SHAPES] for _ in sets]
    flops = sum(2.0 * M_PREFILL * N * K for (_, N, K) in PREFILL_SHAPES)

    def launch(i, p, ev):
        xq, y = outs[i % 2][p]
        if ev is not None:
            ev[0].record(stream)
        fb.fp8_act_quant_static(sets[i % 2][p], scales[p], xq)
        if ev is not None:
            ev[1].record(stream)
        fb.fp8_block_gemm_static(xq, scales[p], wq[p], wsc[p], y)
        if ev is not None:
            ev[2].record(stream)

    dt, ta, tg = run_leg(torch, stream, launch, len(PREFILL_SHAPES), 30, 10)
    per = {name: {"act_quant_us": round(ta[p] * 1e6, 2),
                  "act_quant_GB/s": round(3 * M_PREFILL * K / ta[p] / 1e9, 1),
                  "gemm_us": round(tg[p] * 1e6, 2),
                  "gemm_TFLOP/s": round(2.0 * M_PREFILL * N * K / tg[p] / 1e12, 1)}
           for p, (name, N, K) in enumerate(PREFILL_SHAPES)}
    return {"static_prefill_step": {"ms_per_step": round(dt * 1e3, 4),
                                    "TFLOP/s": round(flops / dt / 1e12, 1),
                                    "gemm_TFLOP/s": round(flops / sum(tg) / 1e12, 1),
                                    "per_projection": per}}


def ue8m0_rows(torch, fb, dev, stream, g):
    """Power-of-two (E8M0-byte) scales: the same prefill step (activation
    quantization + GEMM per projection, two rotated input sets), the weight
    quantizer on the largest weight, and the decode GEMMs."""
    rows = {}
    xs0, ws_bf16 = gen_inputs(torch, dev, 3000)
    sets = [xs0, [torch.roll(x, 1, 0) for x in xs0]]
    wq, we = zip(*[fb.weight_block_quant(w, "ue8m0") for w in ws_bf16])
    del ws_bf16
    outs = [[(torch.empty((M_PREFILL, K), dtype=torch.uint8, device=dev),
              torch.empty((M_PREFILL, K // 128), dtype=torch.uint8, device=dev),
              torch.empty((M_PREFILL, N), dtype=torch.bfloat16, device=dev))
             for (_, N, K) in PREFILL_SHAPES] for _ in sets]
    flops = sum(2.0 * M_PREFILL * N * K for (_, N, K) in PREFILL_SHAPES)

    def launch(i, p, ev):
        xq, xe, y = outs[i % 2][p]
        if ev is not None:
            ev[0].record(stream)
        fb.fp8_act_quant_group_ue8m0(sets[i % 2][p], xq, xe)
        if ev is not None:
            ev[1].record(stream)
        fb.fp8_block_gemm_ue8m0(xq, xe, wq[p], we[p], y)
        if ev is not None:
            ev[2].record(stream)

    dt, ta, tg = run_leg(torch, stream, launch, len(PREFILL_SHAPES), 30, 10)
    per = {name: {"act_quant_us": round(ta[p] * 1e6, 2), "gemm_us": round(tg[p] * 1e6, 2),
                  "gemm_TFLOP/s": round(2.0 * M_PREFILL * N * K / tg[p] / 1e12, 1)}
           for p, (name, N, K) in enumerate(PREFILL_SHAPES)}
    gemm_s = sum(tg)
    rows["ue8m0_prefill_step"] = {"ms_per_step": round(dt * 1e3, 4),
                                  "TFLOP/s": round(flops / dt / 1e12, 1),
                                  "gemm_TFLOP/s": round(flops / gemm_s / 1e12, 1),
                                  "per_projection": per}
    del sets, outs, wq, we
    w = (torch.randn((18432, 7168), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    q = torch.empty((18432, 7168), dtype=torch.uint8, device=dev)
    e = torch.empty((144, 56), dtype=torch.uint8, device=dev)
    t = _time(torch, stream, lambda: fb.fp8_weight_block_quant_ue8m0(w, q, e))
    rows["ue8m0_weight_quant_18432x7168"] = {"us": round(t * 1e6, 2),
                                             "GB/s": round(18432 * 7168 * 3 / t / 1e9, 1)}
    del w, q, e
    for name, N, K in PREFILL_SHAPES:
        x = torch.randn((16, K), generator=g, device=dev).to(torch.bfloat16)
        wq1, we1 = fb.weight_block_quant(
            (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16), "ue8m0")
        xq, xe = fb.act_quant_group(x, "ue8m0")
        y = torch.empty((16, N), dtype=torch.bfloat16, device=dev)
        copies = _weight_copies(wq1, we1)
        t = _time(torch, stream, _rotating(copies, lambda w, e: fb.fp8_block_gemm_ue8m0(xq, xe, w, e, y)))
        del copies
        byts = N * K + 16 * K + 2 * 16 * N
        rows[f"ue8m0_decode_M16_{name}"] = {"us": round(t * 1e6, 2), "GB/s": round(byts / t / 1e9, 1),
                                            "frac_hbm": round(byts / t / 1e9 / PEAK_HBM_GBS, 4)}
    return rows


if __name__ == "__main__":
    main()
