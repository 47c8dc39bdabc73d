#!/usr/bin/env python3
"""Benchmark of the fused dense GEMM + epilogue on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input already
resident in HBM: one fused GEMM + epilogue launch (for the FFN workload, the
up- and down-projection launches).  The deliberately unfused two-kernel path
is timed the same way in the same run for the fused-vs-unfused speedup.

The large shapes run the MI355X at its board power limit, where the clock
settles only after about a second of load; so every run first pre-heats with
1.5 s of fused steps (reported as preheat_s, also when --warmup is given),
then runs the W warm-up steps (unless given: about 1.5 s of work) and the
timed region (unless given: about 2 s of work; step counts derived from one
probe step).  The timed region is exactly K steps (ms_per_step is their mean);
a second leg of K steps with an event between consecutive steps gives the
median; the speedup comes from further alternating unfused / fused legs of K
steps each.

Prints ONE JSON line: metric = fused TFLOP/s (value), % of the fp16/bf16 dense
MFMA peak (roofline.frac), fused vs unfused speedup; roofline of the dominant
kernel with its average duration from HIP events on the launch stream; and the
CPU fp64 oracle timed on a bounded row sample of the same workload
(cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 MFMA (published)
PEAK_TFLOPS_FP8 = 5000.0  # MI355X dense fp8 MFMA (published)
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E (published)
DEFAULT_WORKLOAD = "gemm_relu_bias_fp16_65536x16384x16384"
# device code of the fused kernel and the config table that picks its instance
# the sources each kernel family is built from: a traffic record taken on a
# family's kernels stays valid until one of these files changes
KERNEL_SOURCES = {
    "gemm": ("egm_gemm.hpp", "egm_device.hpp", "egm_kernels.hip", "egm_launch.hpp", "egm_epilogue.hpp"),
    "layernorm": ("egm_layernorm.hpp", "egm_device.hpp", "egm_kernels.hip", "egm_launch.hpp"),
}


def kernel_family(workload: str) -> str:
    return "layernorm" if workload.startswith("layernorm") else "gemm"


def kernel_source_hash(workload: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_family(workload)]:
        with open(os.path.join(ROOT, "dense_gemm_epilogue_fp16_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """Measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled
    by a plain-copy calibration), if taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return t.get("bytes_per_launch")


def algorithmic_bytes(m, n, k, epilog, bias_layout, operand_bytes=2):
    """Fused path: read A, B, bias (+R) once, write D (+mask) once; the
    backward epilogues read the mask instead of a bias and (BGRAD) write the
    fp32 bias gradient.  operand_bytes: 2 (fp16/bf16) or 1 (fp8 A and B; the
    bias, residual and D stay 16-bit)."""
    b = operand_bytes * (m * k + k * n) + 2 * m * n
    if epilog in ("DRELU", "DRELU_BGRAD"):
        b += m * n // 8
        if epilog == "DRELU_BGRAD":
            b += 4 * (m if bias_layout == "row" else n)
        return b
    b += 2 * (m if bias_layout == "row" else n)
    if epilog == "BIAS_RESIDUAL":
        b += 2 * m * n
    if epilog == "RELU_AUX_BIAS":
        b += m * n // 8
    return b


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: about 2 s of work)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed warm-up steps (default: about 1.5 s of work)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (calibrates rocprofv3 byte counters)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this benchmark with "
                         "--copy-mib into profiles/traffic_<workload>.json, then exit")
    ap.add_argument("--cold", action="store_true",
                    help="also time single steps with the caches flushed (a 512 MiB write between steps, outside "
                         "the events), and the host-side latency of one launch plus synchronize")
    ap.add_argument("--torch-context", action="store_true",
                    help="also time torch.matmul (the vendor GEMM, no epilogue) and torch's eager "
                         "matmul + bias + activation on the same operands, with the same warm-up and step counts")
    ap.add_argument("--launch-amortisation", type=int, default=0, metavar="N",
                    help="also time N problems of the workload's shape (own A and D, shared B) as N separate "
                         "executes, as one replayed HIP graph of those executes, and as one strided-batch launch")
    ap.add_argument("--sustain", type=float, default=0.0,
                    help="instead of the bench line: run the fused step back to back for this many seconds and "
                         "print one JSON line per second with its throughput and the board power and clocks "
                         "that amd-smi reports meanwhile")
    ap.add_argument("--sustain-vendor", action="store_true",
                    help="with --sustain: then run the vendor GEMM alone (torch.matmul into the same outputs; "
                         "torch._scaled_mm for fp8) the same way, for the clock and power it sustains (context only)")
    ap.add_argument("--mfma-shape-probe", type=float, default=0.0, metavar="SECONDS",
                    help="instead of the bench line: run the MFMA-only probe (libegm_probe.so) with each 16-bit "
                         "MFMA shape (32x32x16, then 16x16x32, twice) back to back on every CU for this many "
                         "seconds each, printing one JSON line per second with its throughput and the board "
                         "power and clocks, then one summary line per shape")
    args = ap.parse_args()
    if args.mfma_shape_probe > 0:
        mfma_shape_probe(args.mfma_shape_probe)
        return
    if args.ingest_pmc:
        ingest_pmc(args.workload, *args.ingest_pmc, copy_mib=args.copy_mib or 1024)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the fused GEMM + epilogue needs no "
                          "collective, and every workload fits one MI355X; run with --gpus 1"}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import dense_gemm_epilogue_fp16_amd as egm
    import egm_workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}), flush=True)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def to_dev(bits, dtype, shape):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(torch.float16 if dtype == "fp16" else torch.bfloat16).reshape(shape).to(dev)

    t_setup = time.time()
    name = args.workload
    if name in W.LAYERNORM_WORKLOADS:
        bench_layernorm(args, name, dev)
        return
    wl = {**W.WORKLOADS, **W.BACKWARD_WORKLOADS, **W.FP8_WORKLOADS}[name]
    fp8 = name in W.FP8_WORKLOADS
    keep = []
    mm_kw = {}  # Matmul constructor arguments (fp8: scales and output dtype)
    if fp8:
        ops = W.fp8_workload_operands(name)
        f8t = torch.float8_e4m3fn if ops.a_fmt == "e4m3" else torch.float8_e5m2
        a = torch.from_numpy(ops.a).to(dev).view(f8t)
        b = torch.from_numpy(ops.b).to(dev).view(f8t)
        sa = torch.tensor([float(ops.scale_a)], dtype=torch.float32, device=dev)
        sb = torch.tensor([float(ops.scale_b)], dtype=torch.float32, device=dev)
        bias = to_dev(ops.bias, ops.out_dtype, (ops.m, 1) if ops.bias_layout == "row" else (1, ops.n))
        d = torch.empty((ops.m, ops.n), dtype=bias.dtype, device=dev)
        epilog = wl.epilogs[-1]
        out = dict(out=d)
        if epilog == "RELU_AUX_BIAS":
            out["aux"] = torch.empty((ops.m, ops.n // 8), dtype=torch.uint8, device=dev)
        specs = [((a, b), epilog, {"bias": bias}, out, (ops.m, ops.n, ops.k), ops.bias_layout)]
        mm_kw = dict(scale_a=sa, scale_b=sb, out_dtype=bias.dtype)
        keep += [a, b, bias, d, sa, sb]
        host_ops = ops
    elif name in W.BACKWARD_WORKLOADS:
        ops, mask = W.backward_operands(name)
        a = to_dev(ops.a, ops.dtype, (ops.m, ops.k))
        b = to_dev(ops.b, ops.dtype, (ops.k, ops.n))
        aux = torch.from_numpy(mask).to(dev)
        grad = torch.empty((1, ops.n) if wl.bias_layout == "col" else (ops.m, 1), dtype=torch.float32, device=dev)
        d = torch.empty((ops.m, ops.n), dtype=a.dtype, device=dev)
        specs = [((a, b), wl.epilogs[-1], {"bias_grad": grad}, dict(out=d, aux=aux), (ops.m, ops.n, ops.k),
                  wl.bias_layout)]
        keep += [a, b, d, aux, grad]
        host_ops = ops
        host_ops.meta["mask"] = mask
    elif name.startswith("ffn_"):
        f = W.ffn_operands()
        x = to_dev(f.x, "bf16", (f.tokens, f.hidden))
        w1 = to_dev(f.w1, "bf16", (f.hidden, f.ffn))
        w2 = to_dev(f.w2, "bf16", (f.ffn, f.hidden))
        b1 = to_dev(f.b1, "bf16", (1, f.ffn))
        b2 = to_dev(f.b2, "bf16", (1, f.hidden))
        h = torch.empty((f.tokens, f.ffn), dtype=torch.bfloat16, device=dev)
        d = torch.empty((f.tokens, f.hidden), dtype=torch.bfloat16, device=dev)
        specs = [((x, w1), "GELU_BIAS", {"bias": b1}, dict(out=h), (f.tokens, f.ffn, f.hidden), "col"),
                 ((h, w2), "BIAS_RESIDUAL", {"bias": b2, "residual": x}, dict(out=d), (f.tokens, f.hidden, f.ffn),
                  "col")]
        keep += [x, w1, w2, b1, b2, h, d]
        host_ops = None
    else:
        ops = W.workload_operands(name)
        a = to_dev(ops.a, ops.dtype, (ops.m, ops.k))
        b = to_dev(ops.b, ops.dtype, (ops.k, ops.n))
        bias = to_dev(ops.bias, ops.dtype, (ops.m, 1) if ops.bias_layout == "row" else (1, ops.n))
        d = torch.empty((ops.m, ops.n), dtype=a.dtype, device=dev)
        epilog = wl.epilogs[-1]
        out = dict(out=d)
        if epilog == "RELU_AUX_BIAS":
            out["aux"] = torch.empty((ops.m, ops.n // 8), dtype=torch.uint8, device=dev)
        specs = [((a, b), epilog, {"bias": bias}, out, (ops.m, ops.n, ops.k), ops.bias_layout)]
        keep += [a, b, bias, d]
        host_ops = ops
    if args.copy_mib:
        # counter calibration: an elementwise pass that reads and writes
        # exactly copy_mib MiB, under a kernel name nothing else here uses
        src = torch.zeros(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)
        del src, dst
    torch.cuda.synchronize(dev)
    setup_s = time.time() - t_setup

    def make(fused):
        res = []
        for (aa, bb), ep, ins, out, (m, n, k), layout in specs:
            mm = egm.Matmul(aa, bb, **mm_kw)
            mm.plan(ep, ins, fused=fused)
            res.append((mm, out, (m, n, k), ep, layout))
        return res

    fused_plans = make(True)
    unfused_plans = make(False)
    flops = sum(2 * m * n * k for _, _, (m, n, k), _, _ in fused_plans)

    def step(plans):
        for mm, out, _, _, _ in plans:
            mm.execute(**out)

    def timed(plans, steps, warmup):
        for _ in range(warmup):
            step(plans)
        torch.cuda.synchronize(dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            step(plans)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall

    # step counts: from one probe step unless given
    probe_ms, _ = timed(fused_plans, 1, 1)
    if args.sustain > 0:
        sustain(lambda: step(fused_plans), probe_ms, flops, args.sustain, dev, stream)
        if args.sustain_vendor:
            if fp8:
                print(json.dumps({"leg": "vendor fp8 GEMM alone (torch._scaled_mm, B column-major), context only"}),
                      flush=True)
                (aa, bb), _, _, _, _, _ = specs[0]
                bcm = bb.t().contiguous().t()  # the vendor call wants B column-major

                def vendor_step():
                    torch._scaled_mm(aa, bcm, scale_a=mm_kw["scale_a"], scale_b=mm_kw["scale_b"],
                                     out_dtype=mm_kw["out_dtype"])
            else:
                print(json.dumps({"leg": "vendor GEMM alone (torch.matmul), context only"}), flush=True)

                def vendor_step():
                    for (aa, bb), _, _, out, _, _ in specs:
                        torch.matmul(aa, bb, out=out["out"])

            vendor_step()
            torch.cuda.synchronize(dev)
            sustain(vendor_step, probe_ms, flops, args.sustain, dev, stream)
        for mm, *_ in fused_plans + unfused_plans:
            mm.free()
        return
    warmup = args.warmup if args.warmup is not None else max(3, int(1500.0 / max(probe_ms, 1e-3)))
    steps = args.steps if args.steps is not None else max(10, int(2000.0 / max(probe_ms, 1e-3)))
    args.warmup, args.steps = warmup, steps
    # Pre-heat, always (also when --warmup is given): the board needs about a
    # second of load to reach its steady power and clock, so a short timed
    # region that follows only a few warm-up steps would time the ramp.
    preheat_s = preheat(lambda: step(fused_plans), probe_ms, PREHEAT_SECONDS, dev)
    for _ in range(warmup):
        step(fused_plans)
    # the timed region: exactly `steps` fused steps
    fused_ms, fused_wall = timed(fused_plans, steps, 0)
    # per-step event times in a leg of the same length right after it (events
    # between the steps of the timed region itself would add host work to
    # every launch of the small workloads): their median and spread
    per_step = per_step_ms(lambda: step(fused_plans), steps, stream, dev)
    # fused-vs-unfused: alternating legs of the same length after it
    unfused_legs, fused_legs = [], [fused_ms]
    for _ in range(2):
        unfused_legs.append(timed(unfused_plans, steps, 1)[0])
        if len(fused_legs) < 2:
            fused_legs.append(timed(fused_plans, steps, 1)[0])
    unfused_ms = sum(unfused_legs) / len(unfused_legs)
    fused_cmp_ms = sum(fused_legs) / len(fused_legs)

    # per-launch roofline of the dominant kernel (the largest GEMM of the step)
    dom = max(fused_plans, key=lambda p: p[2][0] * p[2][1] * p[2][2])
    dm, dn, dk = dom[2]
    if len(fused_plans) > 1:
        only = [dom]
        dom_ms, _ = timed(only, args.steps, 1)
    else:
        dom_ms = fused_ms
    dom_flops = 2 * dm * dn * dk
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    tb = traffic_from_profile(name)

    value = flops / (fused_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS_FP8 if fp8 else PEAK_TFLOPS
    ob = 1 if fp8 else 2
    alg = sum(algorithmic_bytes(m, n, k, ep, lay, ob) for _, _, (m, n, k), ep, lay in fused_plans)
    # P written and read back (+ D read again for the two-kernel bias gradient)
    extra = sum((6 if ep == "DRELU_BGRAD" else 4) * m * n for _, _, (m, n, k), ep, _ in fused_plans)
    result = {
        "metric": ("fused GEMM+epilogue TFLOP/s (fp8 MFMA, fp32 accumulate)" if fp8 else
                   "fused GEMM+epilogue TFLOP/s (fp16/bf16 MFMA, fp32 accumulate)"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fused_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"fp8_{ops.a_fmt}" if fp8 else wl.dtype,
        "data": "synthetic (seeded normal operands, resident in HBM)",
        "config": {"workload": name, "m": wl.m, "n": wl.n, "k": wl.k, "epilog": "+".join(wl.epilogs),
                   "bias": "(m,1)" if wl.bias_layout == "row" else "(1,n)", "accumulate": "fp32",
                   **({"operands": f"{ops.a_fmt} x {ops.b_fmt}, per-tensor scales", "out": wl.dtype} if fp8 else {}),
                   "plan": fused_plans[0][0].describe()},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "unfused_ms_per_step": round(unfused_ms, 4),
        "speedup_vs_unfused": round(unfused_ms / fused_cmp_ms, 4),
        "bytes_fused_algorithmic": alg,
        "bytes_saved_by_fusion": extra,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": tb,
                     "kernel": f"gemm_epilogue_kernel {dm}x{dn}x{dk} {dom[3]}",
                     "avg_launch_ms": round(dom_ms, 4), "flops_per_launch": dom_flops,
                     "algorithmic_bytes_per_launch": algorithmic_bytes(dm, dn, dk, dom[3], dom[4], ob)},
        "median_ms_per_step": round(statistics.median(per_step), 4),
        "per_step_ms_min_max": [round(min(per_step), 4), round(max(per_step), 4)],
        "preheat_s": round(preheat_s, 2),
        "setup_s": round(setup_s, 1),
        "timed_wall_s": round(fused_wall, 3),
    }

    if args.torch_context:
        result["torch_context"] = (torch_context_fp8(specs, mm_kw, timed, steps, warmup, flops) if fp8 else
                                   torch_context(specs, timed, steps, warmup, flops))

    if args.launch_amortisation:
        result["launch_amortisation"] = launch_amortisation(specs, mm_kw, args.launch_amortisation, dev)

    if args.cold:
        result["cold_cache"] = cold_and_latency(lambda: step(fused_plans), lambda: step(unfused_plans),
                                                flops, alg, dev, stream)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(name, host_ops, keep, args.cpu_seconds)

    for mm, *_ in fused_plans + unfused_plans:
        mm.free()
    print(json.dumps(result), flush=True)


PREHEAT_SECONDS = 1.5


def preheat(run_step, probe_ms, seconds, dev):
    """Run steps back to back for at least ``seconds`` of wall time (in
    batches of about 50 ms of GPU work, synchronising between batches so the
    queue never runs far ahead); returns the seconds spent."""
    import torch
    batch = max(1, int(50.0 / max(probe_ms, 1e-3)))
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            run_step()
        torch.cuda.synchronize(dev)
    return time.perf_counter() - t0


def per_step_ms(run_step, steps, stream, dev):
    """Event time of each of ``steps`` back-to-back steps (one event between
    consecutive steps, recorded on the launch stream)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run_step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def host_description():
    """CPU model (with family / model numbers, since virtual machines may
    report a generic name) and numpy's BLAS library and thread count."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                key, _, val = ln.partition(":")
                key = key.strip()
                if key in ("model name", "cpu family", "model") and key not in info:
                    info[key] = val.strip()
                if len(info) == 3:
                    break
    except OSError:  # pragma: no cover
        pass
    cpu = info.get("model name")
    if cpu is not None and ("cpu family" in info or "model" in info):
        cpu = f"{cpu} (family {info.get('cpu family', '?')}, model {info.get('model', '?')})"
    blas = None
    try:
        import numpy  # noqa: F401  (loads its BLAS, which threadpoolctl then sees)
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = libs[0]
            blas = (f"{i.get('internal_api')} {i.get('version')} ({i.get('prefix')}, kernels for "
                    f"{i.get('architecture')}, {i.get('num_threads')} threads)")
    except Exception:  # pragma: no cover
        pass
    return cpu, blas


def torch_context(specs, timed, steps, warmup, flops):
    """torch.matmul alone, and torch's eager matmul + bias + activation (+ residual),
    timed like the fused step: context for the fused kernel, not a code path of
    the library."""
    import torch

    keep_cache = {}

    def eager(spec, with_epilogue):
        (aa, bb), ep, ins, out, _, _ = spec
        y = torch.matmul(aa, bb)
        if with_epilogue and ep in ("DRELU", "DRELU_BGRAD"):
            # eager backward: the mask as a bool tensor (unpacked once, outside
            # the timing), the product masked, then the bias gradient
            aux = out["aux"]
            if id(aux) not in keep_cache:
                bits = torch.arange(8, device=aux.device, dtype=torch.uint8)
                keep_cache[id(aux)] = ((aux.unsqueeze(-1) >> bits) & 1).bool().reshape(aa.shape[0], -1)
            dz = y * keep_cache[id(aux)]
            if ep == "DRELU_BGRAD":
                dz.sum(dim=0 if ins["bias_grad"].shape[0] == 1 else 1, dtype=torch.float32)
            return dz
        if with_epilogue:
            y = y + ins["bias"]
            if ep in ("RELU_BIAS", "RELU_AUX_BIAS"):
                y = torch.relu(y)
                if ep == "RELU_AUX_BIAS":
                    (y > 0)  # the predicate pass a backward mask needs (unpacked)
            elif ep == "GELU_BIAS":
                y = torch.nn.functional.gelu(y, approximate="tanh")
            elif ep == "BIAS_RESIDUAL":
                y = y + ins["residual"]
        return y

    res = {}
    for label, with_epi in (("matmul_ms", False), ("matmul_bias_act_ms", True)):
        runner = [lambda sp=spec, w=with_epi: eager(sp, w) for spec in specs]
        ms, _ = _timed_callables(runner, timed, steps, warmup)
        res[label] = round(ms, 5)
    res["matmul_tflops"] = round(flops / (res["matmul_ms"] * 1e-3) / 1e12, 2)
    res["note"] = "torch.matmul is the vendor GEMM (hipBLASLt); the second figure is the eager op sequence"
    return res


def torch_context_fp8(specs, mm_kw, timed, steps, warmup, flops):
    """torch._scaled_mm (the vendor fp8 GEMM, per-tensor scales, bf16 out) on
    the same operands, alone and with torch's eager bias + activation: context,
    not a code path of the library."""
    import torch
    (aa, bb), ep, ins, out, _, _ = specs[0]
    bt = bb.t().contiguous().t()  # the vendor call wants B column-major
    sa, sb = mm_kw["scale_a"], mm_kw["scale_b"]

    def run(with_epilogue):
        y = torch._scaled_mm(aa, bt, scale_a=sa, scale_b=sb, out_dtype=mm_kw["out_dtype"])
        if with_epilogue:
            y = y + ins["bias"]
            if ep in ("RELU_BIAS", "RELU_AUX_BIAS"):
                y = torch.relu(y)
                if ep == "RELU_AUX_BIAS":
                    (y > 0)
        return y

    res = {}
    try:
        for label, w in (("matmul_ms", False), ("matmul_bias_act_ms", True)):
            ms, _ = _timed_callables([lambda w=w: run(w)], timed, steps, warmup)
            res[label] = round(ms, 5)
        res["matmul_tflops"] = round(flops / (res["matmul_ms"] * 1e-3) / 1e12, 2)
        res["note"] = ("torch._scaled_mm is the vendor fp8 GEMM (hipBLASLt); the second figure adds torch's eager "
                       "bias and activation")
    except Exception as exc:  # the vendor call may be missing for this type on this build
        res = {"error": f"{type(exc).__name__}: {exc}"[:300]}
    return res


def bench_layernorm(args, name, dev):
    """The LayerNorm row kernel: one step = one launch over the whole
    [rows, cols] input, inputs resident in HBM.  Memory-bound: value and
    roofline in GB/s of algorithmic bytes (x read, y written, gamma and beta
    read once).  The comparison path is the page's own multi-kernel form
    (mean, centre, variance, rsqrt, scale and shift as separate torch ops)."""
    import numpy as np
    import torch

    import dense_gemm_epilogue_fp16_amd as egm
    import egm_workloads as W
    wl = W.LAYERNORM_WORKLOADS[name]
    t0 = time.time()
    o = W.layernorm_operands(wl.m, wl.n, wl.dtype, seed=0)

    def to_dev(bits, shape):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).reshape(shape).to(dev)

    x, g, b = to_dev(o.x, (wl.m, wl.n)), to_dev(o.gamma, (wl.n,)), to_dev(o.beta, (wl.n,))
    y = torch.empty_like(x)
    if args.copy_mib:  # counter calibration, as for the GEMM workloads
        src = torch.zeros(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        torch.bitwise_not(src, out=torch.empty_like(src))
        del src
    torch.cuda.synchronize(dev)
    setup_s = time.time() - t0
    stream = torch.cuda.current_stream(dev)

    def fused():
        egm.layer_norm(x, g, b, 1e-5, out=y)

    def multi_kernel():  # the eager op sequence: each line its own kernel(s) and HBM round trip
        mean = x.mean(dim=-1, keepdim=True)
        xc = x - mean
        var = (xc * xc).mean(dim=-1, keepdim=True)
        return xc * torch.rsqrt(var + 1e-5) * g + b

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / steps, time.perf_counter() - t

    probe, _ = timed(fused, 1, 1)
    warmup = args.warmup if args.warmup is not None else max(3, int(500.0 / max(probe, 1e-3)))
    steps = args.steps if args.steps is not None else max(10, int(1000.0 / max(probe, 1e-3)))
    for _ in range(warmup):
        fused()
    ms, wall = timed(fused, steps, 0)
    unf = [timed(multi_kernel, steps, 1)[0], timed(multi_kernel, steps, 1)[0]]
    fus = [ms, timed(fused, steps, 1)[0]]
    alg = 2 * 2 * wl.m * wl.n + 2 * 2 * wl.n
    gbs = alg / (ms * 1e-3) / 1e9
    tb = traffic_from_profile(name)
    result = {
        "metric": "LayerNorm row kernel GB/s (algorithmic bytes: x read, y written once)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded normal rows, resident in HBM)",
        "config": {"workload": name, "rows": wl.m, "cols": wl.n, "eps": 1e-5, "affine": True,
                   "statistics": "fp32, one pass (Welford merge)"},
        "unfused_ms_per_step": round(sum(unf) / 2, 5),
        "speedup_vs_unfused": round((sum(unf) / 2) / (sum(fus) / 2), 4),
        "unfused_note": "torch eager: mean, centre, variance, rsqrt, scale, shift as separate kernels",
        "bytes_fused_algorithmic": alg,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": tb,
                     "kernel": f"layernorm_kernel {wl.m}x{wl.n}", "avg_launch_ms": round(ms, 5),
                     "algorithmic_bytes_per_launch": alg},
        "setup_s": round(setup_s, 1), "timed_wall_s": round(wall, 3),
    }
    if args.torch_context:
        tl, _ = timed(lambda: torch.nn.functional.layer_norm(x, (wl.n,), g, b, 1e-5), steps, warmup)
        result["torch_context"] = {"layer_norm_ms": round(tl, 5), "layer_norm_gbs": round(alg / (tl * 1e-3) / 1e9, 1),
                                   "note": "torch.nn.functional.layer_norm (torch's own fused kernel)"}
    if not args.no_cpu_baseline:
        from oracle import egm_oracle as eo
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        except Exception:  # pragma: no cover
            cores = len(os.sched_getaffinity(0))
        count = min(wl.m, 2048)
        secs = 0.0
        while True:
            rows = W.sample_rows(wl.m, count, seed=2)
            t = time.perf_counter()
            yr, _, _ = eo.layer_norm_reference(o.x[rows], wl.dtype, o.gamma, o.beta, 1e-5)
            secs = time.perf_counter() - t
            if secs > 0.5 * args.cpu_seconds or count >= wl.m:
                break
            count = min(wl.m, int(count * max(2.0, 0.6 * args.cpu_seconds / max(secs, 1e-3))))
        sel = y.index_select(0, torch.from_numpy(rows).to(dev)).cpu()
        d = eo.widen(sel.view(torch.int16).numpy().view(np.uint16), wl.dtype)
        byts = 4.0 * len(rows) * wl.n
        result["cpu_baseline"] = {"value": round(byts / secs / 1e9, 3), "unit": "GB/s", "cores": int(cores),
                                  "kind": "oracle", "sample": f"{len(rows)} of {wl.m} rows x {wl.n}, fp64 numpy "
                                  f"oracle; {secs:.1f} s", "seconds": round(secs, 2),
                                  "parity_max_abs_err": float(np.abs(d - yr).max()),
                                  "parity_tol": eo.TOLERANCE[wl.dtype]}
    print(json.dumps(result), flush=True)


def launch_amortisation(specs, mm_kw, nprob, dev, target_ms=400.0):
    """Per-GEMM time of nprob problems of the workload's shape (own A and D,
    shared B and bias): nprob executes launched one by one, the same executes
    captured once in a HIP graph and replayed, and one strided-batch execute;
    plus the host time of one execute call."""
    import torch

    import dense_gemm_epilogue_fp16_amd as egm
    if len(specs) != 1 or specs[0][1] == "DRELU_BGRAD":
        return {"error": "one forward GEMM per step only"}
    (aa, bb), ep, ins, out, (m, n, k), _ = specs[0]
    mm = egm.Matmul(aa, bb, **mm_kw)
    mm.plan(ep, ins)
    a_b = aa.unsqueeze(0).expand(nprob, m, k).contiguous()
    d_b = torch.empty((nprob, m, n), dtype=mm.dtype, device=dev)
    aux_b = torch.empty((nprob, m, n // 8), dtype=torch.uint8, device=dev) if ep == "RELU_AUX_BIAS" else None

    def eager():
        for i in range(nprob):
            mm.execute(a=a_b[i], out=d_b[i], aux=aux_b[i] if aux_b is not None else None)

    def batched():
        mm.execute_batched(a_b, bb, out=d_b, aux=aux_b)

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        eager()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        eager()

    def time_it(fn):
        fn()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize(dev)
        once = max(e0.elapsed_time(e1), 1e-3)
        reps = max(3, int(target_ms / once))
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / reps * 1000.0 / nprob  # us per GEMM

    res = {"problems": nprob, "shape": [m, n, k], "epilog": ep,
           "eager_us_per_gemm": round(time_it(eager), 3),
           "graph_us_per_gemm": round(time_it(g.replay), 3),
           "strided_us_per_gemm": round(time_it(batched), 3)}
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    eager()
    res["host_us_per_execute_call"] = round((time.perf_counter() - t0) * 1e6 / nprob, 2)
    torch.cuda.synchronize(dev)
    res["flops_per_gemm"] = 2 * m * n * k
    res["note"] = ("eager = one launch per execute; graph = the same executes captured in one HIP graph; strided = "
                   "egm_execute_strided, one launch for all problems")
    mm.free()
    del g
    return res


def _timed_callables(runner, timed, steps, warmup):
    class _Plan:
        def __init__(self, fn):
            self.fn = fn

        def execute(self, **_):
            self.fn()
    return timed([(_Plan(fn), {}, None, None, None) for fn in runner], steps, warmup)


def cold_and_latency(run_fused, run_unfused, flops, alg_bytes, dev, stream, reps=30):
    """Median single-step GPU time (HIP events) with L2 and MALL flushed before
    every step by a 512 MiB write outside the events, for the fused and the
    unfused path; and the median host time of one fused launch followed by a
    synchronize (warm), which includes the launch overhead."""
    import statistics

    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def one(run, cold):
        if cold:
            flush.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1)

    out = {}
    for label, run in (("fused", run_fused), ("unfused", run_unfused)):
        one(run, True)
        ms = statistics.median(one(run, True) for _ in range(reps))
        out[f"{label}_ms"] = round(ms, 5)
    out["fused_tflops"] = round(flops / (out["fused_ms"] * 1e-3) / 1e12, 2)
    out["fused_algorithmic_gbs"] = round(alg_bytes / (out["fused_ms"] * 1e-3) / 1e9, 1)
    out["speedup_vs_unfused"] = round(out["unfused_ms"] / out["fused_ms"], 4)
    lat = []
    for _ in range(reps):
        t0 = time.perf_counter()
        run_fused()
        torch.cuda.synchronize(dev)
        lat.append(time.perf_counter() - t0)
    out["single_shot_fused_us"] = round(statistics.median(lat) * 1e6, 1)
    del flush
    return out


def _smi_sample():
    """Board power (W) and per-XCD graphics clocks (MHz) from amd-smi, or None."""
    import csv
    import io
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--csv"], capture_output=True, text=True, timeout=10)
        rows = list(csv.DictReader(io.StringIO(r.stdout)))
    except Exception:  # pragma: no cover - tool missing or failed
        return None
    if not rows:
        return None
    row = rows[0]
    clks = [int(v) for k, v in row.items() if k and re.fullmatch(r"gfx_\d+_clk", k) and v.isdigit()]
    power = row.get("socket_power")
    return {"power_w": int(power) if power and power.isdigit() else None, "gfx_clk_mhz": clks}


def mfma_shape_probe(seconds):
    """Sustained throughput of the two 16-bit MFMA shapes with no memory
    traffic (egm_mfma_probe.hip): 4 workgroups of 8 waves per CU, every wave a
    chain of independent MFMAs on operands that switch between MFMAs.  Each
    shape runs for `seconds` in windows of about one second, timed with HIP
    events on the launch stream while amd-smi is sampled in a side thread; the
    summary takes the windows after the first two (the board's ramp)."""
    import ctypes
    import threading

    import torch
    path = os.path.join(ROOT, "dense_gemm_epilogue_fp16_amd", "libegm_probe.so")
    if not os.path.exists(path):
        print(json.dumps({"error": "libegm_probe.so is not built: run __graft_entry__.build()"}), flush=True)
        sys.exit(1)
    lib = ctypes.CDLL(path)
    lib.egm_mfma_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.egm_mfma_probe.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    blocks = 4 * 256
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    per_iter = {32: 8 * 2 * 32 * 32 * 16, 16: 32 * 2 * 16 * 16 * 32}
    iters = {32: 4000, 16: 2000}  # the same flops per launch for both shapes
    summary = []
    for shape in (32, 16, 32, 16):
        flops = blocks * 8 * iters[shape] * per_iter[shape]
        samples = []
        stop = threading.Event()

        def sampler():
            while not stop.is_set():
                smp = _smi_sample()
                if smp is not None:
                    samples.append((time.perf_counter(), smp))
                stop.wait(0.5)

        th = threading.Thread(target=sampler, daemon=True)
        th.start()
        windows = []
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            w0 = time.perf_counter()
            e0.record(stream)
            n = 0
            while time.perf_counter() - w0 < 1.0:
                rc = lib.egm_mfma_probe(shape, iters[shape], blocks, ctypes.c_void_p(out.data_ptr()),
                                        ctypes.c_void_p(stream.cuda_stream))
                if rc != 0:
                    stop.set()
                    print(json.dumps({"error": f"egm_mfma_probe returned {rc}"}), flush=True)
                    sys.exit(1)
                n += 1
                if n % 8 == 0:
                    torch.cuda.synchronize(dev)
            e1.record(stream)
            torch.cuda.synchronize(dev)
            w1 = time.perf_counter()
            inwin = [smp for (ts, smp) in samples if w0 <= ts <= w1]
            pw = [smp["power_w"] for smp in inwin if smp["power_w"]]
            clk = [sum(smp["gfx_clk_mhz"]) / len(smp["gfx_clk_mhz"]) for smp in inwin if smp["gfx_clk_mhz"]]
            line = {"mfma": f"{shape}x{shape}x{16 if shape == 32 else 32}", "t_s": round(w1 - t0, 2),
                    "tflops": round(n * flops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1),
                    "power_w": round(sum(pw) / len(pw)) if pw else None,
                    "gfx_clk_mhz_mean": round(sum(clk) / len(clk)) if clk else None}
            windows.append(line)
            print(json.dumps(line), flush=True)
        stop.set()
        th.join()
        steady = windows[2:] or windows
        tf = sum(w["tflops"] for w in steady) / len(steady)
        clks = [w["gfx_clk_mhz_mean"] for w in steady if w["gfx_clk_mhz_mean"]]
        pws = [w["power_w"] for w in steady if w["power_w"]]
        summary.append({"mfma": windows[0]["mfma"], "steady_tflops": round(tf, 1),
                        "gfx_clk_mhz": round(sum(clks) / len(clks)) if clks else None,
                        "power_w": round(sum(pws) / len(pws)) if pws else None,
                        "frac_of_clock_limited_peak": round(tf / (2500.0 * sum(clks) / len(clks) / 2400.0), 3)
                        if clks else None})
    for s_ in summary:
        print(json.dumps({"summary": s_}), flush=True)


def sustain(run_step, probe_ms, flops, seconds, dev, stream):
    """Back-to-back fused steps for `seconds`, in windows of about one second,
    each timed with HIP events on the launch stream; amd-smi is sampled in a
    side thread.  Shows where the board's power limit settles the clock."""
    import threading

    import torch
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            smp = _smi_sample()
            if smp is not None:
                samples.append((time.perf_counter(), smp))
            stop.wait(0.5)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    per_window = max(1, int(1000.0 / max(probe_ms, 1e-3)))
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < seconds:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(per_window):
            run_step()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        w1 = time.perf_counter()
        ms = e0.elapsed_time(e1) / per_window
        inwin = [smp for (ts, smp) in samples if w0 <= ts <= w1]
        line = {"t_s": round(w1 - t_start, 2), "steps": per_window, "ms_per_step": round(ms, 4),
                "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        if inwin:
            pw = [smp["power_w"] for smp in inwin if smp["power_w"] is not None]
            clk = [c for smp in inwin for c in smp["gfx_clk_mhz"]]
            line["power_w"] = round(sum(pw) / len(pw)) if pw else None
            line["gfx_clk_mhz_mean"] = round(sum(clk) / len(clk)) if clk else None
            line["gfx_clk_mhz_range"] = [min(clk), max(clk)] if clk else None
        print(json.dumps(line), flush=True)
    stop.set()
    th.join(timeout=15)
    idle = _smi_sample()
    if idle is not None:
        print(json.dumps({"after_run": idle}), flush=True)


def _pmc_per_kernel(directory, counter):
    """Average counter value per dispatch, by kernel name, from rocprofv3 CSVs."""
    import csv
    import glob
    sums, counts = {}, {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                k = row.get("Kernel_Name", "?")
                sums[k] = sums.get(k, 0.0) + float(row["Counter_Value"])
                counts[k] = counts.get(k, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def ingest_pmc(workload, fetch_dir, write_dir, copy_mib):
    """HBM bytes per launch of the dominant kernel: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) scaled by what the same counters read for the
    calibration pass over copy_mib MiB (an elementwise bitwise-not, which
    reads and writes exactly that many bytes; host-to-device copies of the
    inputs use other kernels)."""
    import re

    import egm_workloads as W
    fetch = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_kernel(write_dir, "WRITE_SIZE")
    copy_k = [k for k in fetch if "bitwise_not" in k]
    if workload in W.LAYERNORM_WORKLOADS:
        gemm_k = [k for k in fetch if "layernorm_kernel" in k]
    else:
        # the dominant fused kernel bench.py reports: the workload's first GEMM
        # (the FFN's up-projection) with its last epilog, never the first
        # kernel of the two-kernel path (epilog id 0)
        wl = {**W.WORKLOADS, **W.BACKWARD_WORKLOADS, **W.FP8_WORKLOADS}[workload]
        ids = {"BIAS": 1, "RELU_BIAS": 2, "GELU_BIAS": 3, "RELU_AUX_BIAS": 4, "BIAS_RESIDUAL": 5, "DRELU": 6,
               "DRELU_BGRAD": 7}
        epi = ids[wl.epilogs[0] if workload.startswith("ffn_") else wl.epilogs[-1]]
        gemm_k = [k for k in fetch if re.search(rf"gemm_epilogue_kernel<\d+, {epi},", k)]
    if not copy_k or not gemm_k:
        raise SystemExit(f"kernels not found: {sorted(fetch)}")
    copy_bytes = float(copy_mib << 20)
    ck = max(copy_k, key=lambda k: fetch[k])
    f_scale = copy_bytes / (fetch[ck] * 1024.0)
    w_scale = copy_bytes / (write[ck] * 1024.0)
    gk = max(gemm_k, key=lambda k: fetch[k])  # one kernel name per workload in practice
    out = {"workload": workload, "kernel": gk, "kernel_source_hash": kernel_source_hash(workload),
           "fetch_kib_per_launch": fetch[gk], "write_kib_per_launch": write.get(gk),
           "copy_kernel": ck, "copy_bytes": copy_bytes, "copy_fetch_kib": fetch[ck], "copy_write_kib": write[ck],
           "fetch_scale": f_scale, "write_scale": w_scale,
           "bytes_per_launch": fetch[gk] * 1024.0 * f_scale + (write.get(gk) or 0.0) * 1024.0 * w_scale}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def _cpu_baseline_backward(name, ops, keep, target_s, cores):
    """The backward oracle (DRELU part) on a row sample; checks the GPU's D on
    those rows.  The bias gradient needs every row and is not sampled."""
    import numpy as np
    import torch

    import egm_workloads as W
    from oracle import egm_oracle as eo
    mask = ops.meta["mask"]
    times = {}
    for cnt in (64, 192):
        rows = W.sample_rows(ops.m, min(ops.m, cnt), seed=2)
        t0 = time.perf_counter()
        eo.backward_reference(ops.a[rows], ops.b, ops.dtype, "DRELU", mask[rows])
        times[cnt] = time.perf_counter() - t0
    per_row = max((times[192] - times[64]) / 128.0, 1e-6)
    fixed = max(times[64] - 64 * per_row, 0.0)
    count = int(min(ops.m, 32768, max(64, (target_s - fixed) / per_row)))
    rows = W.sample_rows(ops.m, count, seed=2)
    t0 = time.perf_counter()
    dz, _, _ = eo.backward_reference(ops.a[rows], ops.b, ops.dtype, "DRELU", mask[rows])
    secs = time.perf_counter() - t0
    gpu_d = keep[2]
    sel = gpu_d.index_select(0, torch.from_numpy(rows).to(gpu_d.device)).cpu()
    d = eo.widen(sel.view(torch.int16).numpy().view(np.uint16), ops.dtype)
    flops = 2.0 * len(rows) * ops.n * ops.k
    cpu_model, blas = host_description()
    return {"value": round(flops / secs / 1e12, 4), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu": cpu_model, "blas": blas,
            "sample": f"{len(rows)} of {ops.m} output rows x all {ops.n} columns (k={ops.k}), DRELU part of "
                      f"{W.BACKWARD_WORKLOADS[name].epilogs[-1]}, fp64 numpy oracle; {secs:.1f} s",
            "seconds": round(secs, 2), "parity_max_abs_err": float(np.abs(d - dz).max()),
            "parity_tol": eo.TOLERANCE[ops.dtype]}


def _cpu_baseline_fp8(name, ops, keep, target_s, cores):
    """The fp8 oracle on a row sample; checks the GPU's D on those rows."""
    import numpy as np
    import torch

    import egm_workloads as W
    from oracle import egm_oracle as eo
    epilog = W.FP8_WORKLOADS[name].epilogs[-1]

    def ref(rows):
        return eo.reference_fp8(ops.a, ops.b, ops.a_fmt, ops.b_fmt, ops.scale_a, ops.scale_b, ops.out_dtype, epilog,
                                ops.bias, ops.bias_layout, rows=rows)

    times = {}
    for cnt in (64, 192):
        rows = W.sample_rows(ops.m, min(ops.m, cnt), seed=2)
        t0 = time.perf_counter()
        ref(rows)
        times[cnt] = time.perf_counter() - t0
    per_row = max((times[192] - times[64]) / 128.0, 1e-6)
    fixed = max(times[64] - 64 * per_row, 0.0)
    count = int(min(ops.m, 32768, max(64, (target_s - fixed) / per_row)))
    rows = W.sample_rows(ops.m, count, seed=2)
    t0 = time.perf_counter()
    y, _, _ = ref(rows)
    secs = time.perf_counter() - t0
    gpu_d = keep[3]
    sel = gpu_d.index_select(0, torch.from_numpy(rows).to(gpu_d.device)).cpu()
    d = eo.widen(sel.view(torch.int16).numpy().view(np.uint16), ops.out_dtype)
    flops = 2.0 * len(rows) * ops.n * ops.k
    cpu_model, blas = host_description()
    return {"value": round(flops / secs / 1e12, 4), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu": cpu_model, "blas": blas,
            "sample": f"{len(rows)} of {ops.m} output rows x all {ops.n} columns (k={ops.k}), {epilog} on "
                      f"{ops.a_fmt} x {ops.b_fmt} operands, fp64 numpy oracle; {secs:.1f} s",
            "seconds": round(secs, 2), "parity_max_abs_err": float(np.abs(d - y).max()),
            "parity_tol": eo.TOLERANCE[ops.out_dtype]}


def cpu_baseline(name, ops, keep, target_s):
    """The CPU fp64 oracle on a row sample of the same workload; also checks
    the GPU's D on those rows (a bench-time parity spot check)."""
    import numpy as np
    import torch

    import egm_workloads as W
    from oracle import egm_oracle as eo

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    if ops is not None and "mask" in ops.meta:  # backward: the DRELU part on a row sample
        return _cpu_baseline_backward(name, ops, keep, target_s, cores)
    if name in W.FP8_WORKLOADS:
        return _cpu_baseline_fp8(name, ops, keep, target_s, cores)
    if ops is None:  # FFN chain: time the up-projection oracle on a row sample
        f = W.ffn_operands()
        a, b, bias, layout, epilog, dtype = f.x, f.w1, f.b1, "col", "GELU_BIAS", "bf16"
        m, n, k = f.tokens, f.ffn, f.hidden
        gpu_d = None
    else:
        a, b, bias, layout, epilog, dtype = ops.a, ops.b, ops.bias, ops.bias_layout, W.WORKLOADS[name].epilogs[-1], ops.dtype
        m, n, k = ops.m, ops.n, ops.k
        gpu_d = keep[3]
    # two short calibration runs give the per-row cost (the oracle also widens
    # all of B once per call, a fixed cost); then size the timed sample
    times = {}
    for cnt in (64, 192):
        rows = W.sample_rows(m, min(m, cnt), seed=2)
        t0 = time.perf_counter()
        eo.reference(a, b, dtype, epilog, bias, layout, rows=rows)
        times[cnt] = time.perf_counter() - t0
    per_row = max((times[192] - times[64]) / 128.0, 1e-6)
    fixed = max(times[64] - 64 * per_row, 0.0)
    count = int(min(m, 32768, max(64, (target_s - fixed) / per_row)))
    rows = W.sample_rows(m, count, seed=2)
    t0 = time.perf_counter()
    y, _, _ = eo.reference(a, b, dtype, epilog, bias, layout, rows=rows)
    secs = time.perf_counter() - t0
    flops = 2.0 * len(rows) * n * k
    cpu_model, blas = host_description()
    out = {"value": round(flops / secs / 1e12, 4), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "cpu": cpu_model, "blas": blas, "full_workload_seconds_extrapolated": round(secs * m / len(rows), 1),
           "sample": f"{len(rows)} of {m} output rows x all {n} columns (k={k}), {epilog}, fp64 numpy oracle; "
                     f"{secs:.1f} s",
           "seconds": round(secs, 2)}
    if gpu_d is not None:
        sel = gpu_d.index_select(0, torch.from_numpy(rows).to(gpu_d.device)).cpu()
        d = eo.widen(sel.view(torch.int16).numpy().view(np.uint16), dtype)
        out["parity_max_abs_err"] = float(np.abs(d - y).max())
        out["parity_tol"] = eo.TOLERANCE[dtype]
    return out


if __name__ == "__main__":
    main()
