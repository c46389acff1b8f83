"""Benchmark of the block-scaled FP8 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one fp8_block_linear call (fused dequant + GEMM, fp32 accumulation,
bf16 output) over one batch of the workload's synthetic input, with X, Q, S
already resident in HBM. The K timed steps are captured into one HIP graph
and replayed (``--eager`` times K separate calls instead). Weights are drawn fp32 from the seeded generator and
quantized on the GPU by fp8_block_quantize before timing. To keep the 256 MB
Infinity Cache from serving the weights, the timed steps rotate over enough
distinct (X, Q, S, Y) sets to exceed twice its size.

Prints ONE JSON line: throughput over the K timed steps, the roofline of the
dominant kernel (per-launch duration from HIP events recorded on the launch
stream), and the CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
HBM_PEAK_GBPS = 8000.0             # MI355X HBM3E
MALL_BYTES = 256 << 20

# workload name -> (generator name, linear index, bound)
WORKLOADS = {
    "attn_proj": ("attn_proj", 0, "mfma"),
    "mlp_gate": ("mlp_pair", 0, "mfma"),
    "mlp_down": ("mlp_pair", 2, "mfma"),
    "dit_qkv": ("dit_large_m", 0, "mfma"),
    "dit_mlp_up": ("dit_large_m", 1, "mfma"),
    "skinny_m16": ("skinny", 0, "hbm"),
    "skinny_m1": ("skinny", 1, "hbm"),
    "tiny": ("tiny", 0, "mfma"),
}

# The HBM-bound half of the metric, measured after the headline line.
SECONDARY = ("skinny_m16", "skinny_m1")

# --path values -> fp8bl_path
PATHS = {"auto": 0, "tiled": 1, "skinny": 2, "large": 3}


# What one timed launch (one library call per step) runs on the GPU; the
# rocprofv3 summaries list these kernels with their own averages, which add
# up to avg_launch_us.
LAUNCH_KERNELS = {
    "linear": "fp8_block_linear: gemm_large_kernel, gemm_tiled_kernel or gemm_skinny_kernel, "
              "+ reduce_partials_kernel when K is split",
    "dequant": "fp8_block_dequant: dequant_kernel",
    "quantize": "fp8_block_quantize: quantize_kernel<float>",
    "mlp": "fp8_block_mlp_gate_up: gemm_large_kernel<false, true> (the gated form), or on the tiled "
           "planner's pick gemm_gated_paired_kernel (below 2048 rows) or gemm_gated_kernel",
    "w8a8": "fp8_block_linear_w8a8_bf16: act_quantize_kernel + gemm_w8a8_large_kernel or "
            "gemm_w8a8_kernel, + reduce_partials_kernel when K is split",
    "w8a8_gemm": "fp8_block_linear_w8a8: gemm_w8a8_large_kernel or gemm_w8a8_kernel, "
                 "+ reduce_partials_kernel when K is split",
}


# Source files behind each kernel (besides the shared device/launch files):
# a traffic figure stays valid while the files of the kernels it was measured
# on are unchanged.
KERNEL_SOURCES = {
    "gemm_tiled_kernel": ("gemm_tiled.hip",),
    "gemm_gated_kernel": ("gemm_tiled.hip",),
    "gemm_gated_paired_kernel": ("gemm_tiled.hip",),
    "gemm_large_kernel": ("gemm_large.hip",),
    "gemm_skinny_kernel": ("gemm_skinny.hip",),
    "reduce_partials_kernel": ("gemm_skinny.hip",),
    "dequant_kernel": ("dequant.hip",),
    "quantize_kernel": ("quantize.hip",),
    "act_quantize_kernel": ("quantize.hip",),
    "gemm_w8a8_kernel": ("gemm_w8a8.hip",),
    "gemm_w8a8_large_kernel": ("gemm_w8a8_large.hip",),
    "stream_read_kernel": ("stream_read.hip",),
}
SHARED_SOURCES = ("fp8bl_api.hip", "fp8bl_device.h", "fp8bl_internal.h")


def code_only(src):
    """C++ source bytes without ``//`` and ``/* */`` comments, trailing blanks
    or empty lines; string and character literals are kept as written. An
    edit to comments alone therefore leaves the hash below unchanged."""
    s = src.decode("utf-8", "surrogateescape")
    out, i, n = [], 0, len(s)
    while i < n:
        c = s[i]
        if s.startswith("//", i):
            j = s.find("\n", i)
            i = n if j < 0 else j
        elif s.startswith("/*", i):
            j = s.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and s[j] != c:
                j += 2 if s[j] == "\\" else 1
            out.append(s[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line).encode("utf-8", "surrogateescape")


def kernel_source_sha(kernels=None, read=None):
    """Hash of the code (comments excluded, see ``code_only``) of the HIP
    sources of ``kernels`` (names as rocprofv3 prints them, template arguments
    allowed) plus the shared device and launch files; all of csrc when
    ``kernels`` is None. ``read(name) -> bytes`` supplies file contents
    (default: the working tree)."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "block_scaled_fp8_linear_amd", "csrc")
    if read is None:
        read = lambda name: open(os.path.join(csrc, name), "rb").read()
    if kernels is None:
        names = sorted(os.path.basename(f) for f in glob.glob(os.path.join(csrc, "*")))
    else:
        names = set(SHARED_SOURCES)
        for kname in kernels:
            base = kname.split("<")[0].strip()
            if base not in KERNEL_SOURCES:
                raise KeyError(f"no source files recorded for kernel {kname!r}")
            names.update(KERNEL_SOURCES[base])
        names = sorted(names)
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode())
        h.update(code_only(read(name)))
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), or None
    if there is none for this workload or its kernels' sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get("workloads", {}).get(workload)
    if not ent or not ent.get("kernels") or ent.get("source_sha") is None:
        return None
    try:
        if ent["source_sha"] != kernel_source_sha(ent["kernels"]):
            return None
    except (OSError, KeyError):
        return None
    return ent.get("hbm_bytes_per_launch")


def alg_bytes(m, n, k):
    gn, gk = -(-n // 128), -(-k // 128)
    return 2 * m * k + n * k + 4 * gn * gk + 2 * m * n


def cpu_baseline(lin, x_bits, budget_s=12.0):
    """The oracle as it stands (dequant + fp64 matmul + bound inputs) on a
    bounded sample of the workload, on this host's cores: a row sample of X
    doubled until one pass takes a fair share of the budget, and when the
    whole workload is that quick, whole passes repeated until about
    ``budget_s`` seconds of CPU work are done."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    q, s = O.quantize(lin.w)
    m_all = x_bits.shape[0]

    split = {"dequant_s": 0.0, "matmul_s": 0.0}

    def one_pass(rows):
        t0 = time.perf_counter()
        wd = O.dequant(q, s)
        t1 = time.perf_counter()
        O.linear_exact(x_bits[:rows], wd)
        t2 = time.perf_counter()
        split["dequant_s"] += t1 - t0
        split["matmul_s"] += t2 - t1
        return t2 - t0

    rows = 1
    while True:
        split["dequant_s"] = split["matmul_s"] = 0.0
        dt = one_pass(rows)
        if dt * 2.5 > budget_s or rows >= m_all:
            break
        rows = min(rows * 2, m_all)
    passes, total_t = 1, dt
    while rows >= m_all and total_t + dt < budget_s:
        total_t += one_pass(rows)
        passes += 1
    flops = 2.0 * rows * lin.n * lin.k * passes
    what = (f"{passes} passes over all {m_all} rows" if passes > 1 else f"{rows} of {m_all} rows")
    one_thread = None
    if lin.n * lin.k <= 5120 * 5120:
        # the fp64 matmul alone on one BLAS thread, a row sample of a few seconds
        try:
            from threadpoolctl import threadpool_limits
            wd = O.dequant(q, s)
            r1, t1 = 1, 0.0
            with threadpool_limits(limits=1):
                while True:
                    t0 = time.perf_counter()
                    O.linear_exact(x_bits[:r1], wd)
                    t1 = time.perf_counter() - t0
                    if t1 * 2.5 > 3.0 or r1 >= m_all:
                        break
                    r1 = min(r1 * 2, m_all)
            one_thread = {"tflops": 2.0 * r1 * lin.n * lin.k / t1 / 1e12, "rows": r1, "seconds": round(t1, 3)}
        except Exception:  # pragma: no cover
            one_thread = None
    return {
        "value": flops / total_t / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{what} of X against the full {lin.n}x{lin.k} weight (dequant + fp64 Y* and "
                  f"sum|x w|), {total_t:.2f} s",
        "cpu_model": cpu_model(),
        "dequant_s": round(split["dequant_s"], 3),
        "matmul_s": round(split["matmul_s"], 3),
        "matmul_1thread": one_thread,
        "seconds": total_t,
        "rows": rows,
        "passes": passes,
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stream_ceiling(nbytes=1 << 30, reps=10):
    """Practical HBM ceilings the HBM-bound kernels are compared with: the
    library's plain streaming read (fp8_block_stream_read) over 8 rotated
    copies of a buffer the size of the skinny workload's weight (524 MB in
    all, twice the MALL) and over one 1 GiB buffer, plus torch's sum (a
    read with a reduction) and copy over 1 GiB."""
    import torch
    import block_scaled_fp8_linear_amd as F
    dev = torch.device("cuda:0")
    out = {}
    blocks = 2048
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)

    def timed(fn, n):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n

    def read(buf):
        F.fp8_block_stream_read(buf, blocks, sink)

    wbytes = 8000 * 8192
    bufs = [torch.ones(wbytes, dtype=torch.uint8, device=dev) for _ in range(8)]
    t = timed(lambda i: read(bufs[i % 8]), 40)
    out["stream_read_66MB_GBps"] = round(wbytes / t / 1e9, 1)
    del bufs
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    xb = x.view(torch.uint8)
    t = timed(lambda i: read(xb), reps)
    out["stream_read_1GiB_GBps"] = round(nbytes / t / 1e9, 1)
    y = torch.empty_like(x)
    out["torch_sum_read_GBps"] = round(nbytes / timed(lambda i: x.sum(), reps) / 1e9, 1)
    out["torch_copy_GBps"] = round(2 * nbytes / timed(lambda i: y.copy_(x), reps) / 1e9, 1)
    return out


def measure(args, workload, op="linear", path="auto", steps=None, warmup=None):
    """Time `steps` launches of one library call on `workload` (inputs resident
    in HBM, rotated over enough buffer sets to defeat the MALL) and return the
    throughput and roofline fields of one result."""
    import torch

    import block_scaled_fp8_linear_amd as F
    from workloads import generate

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    gen_name, idx, bound = WORKLOADS[workload]
    wl = generate(gen_name)
    lin = wl.linears[idx]
    m, n, k = lin.m, lin.n, lin.k
    x_bits = lin.x
    if x_bits is None:                   # the MLP down input: any bf16 of that shape
        from workloads import draw_x
        x_bits = draw_x(np.random.default_rng(wl.seed + 100), m, k)

    dev = torch.device("cuda:0")
    if not F.device_supported(0):
        raise RuntimeError("cuda:0 is not a gfx950 device")
    set_bytes = 2 * m * k + n * k + 2 * m * n
    if op == "mlp":
        set_bytes += n * k
    rotate = args.rotate or int(min(64, max(1, -(-2 * MALL_BYTES // set_bytes))))

    w_dev = torch.from_numpy(lin.w).to(dev)
    x0 = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    sets = []
    for r in range(rotate):
        q, s = F.fp8_block_quantize(w_dev)
        x = x0.clone()
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        sets.append((x, q, s, y))
    del w_dev
    if op == "mlp":
        # the up weight of the pair, one copy per set like the gate weight
        wu_dev = torch.from_numpy(wl.linears[idx + 1].w).to(dev)
        ups = [F.fp8_block_quantize(wu_dev) for _ in range(rotate)]
        del wu_dev
    ws_bytes = F.workspace_size(m, n, k)
    if op in ("w8a8", "w8a8_gemm"):
        ws_bytes = F.w8a8_workspace_size(m, n, k)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    if op == "dequant":
        wouts = [torch.empty((n, k), dtype=torch.bfloat16, device=dev) for _ in range(rotate)]
    if op == "w8a8_gemm":
        xqs = [F.fp8_act_quantize(st[0]) for st in sets]
    if op == "quantize":
        w_srcs = [torch.from_numpy(lin.w).to(dev) for _ in range(min(rotate, 4))]
    path_id = PATHS[path]

    def step(i):
        x, q, s, y = sets[i % rotate]
        if op == "linear":
            F.fp8_block_linear(x, q, s, out=y, workspace=ws, path=path_id)
        elif op == "w8a8":
            F.fp8_block_linear_w8a8_bf16(x, q, s, out=y, workspace=ws)
        elif op == "w8a8_gemm":
            xq, xs = xqs[i % rotate]
            F.fp8_block_linear_w8a8(xq, xs, q, s, out=y, workspace=ws, path=path_id)
        elif op == "mlp":
            qu, su = ups[i % rotate]
            F.fp8_block_mlp_gate_up(x, q, s, qu, su, out=y, path=path_id)
        elif op == "dequant":
            F.fp8_block_dequant(q, s, out=wouts[i % rotate])
        else:
            F.fp8_block_quantize(w_srcs[i % len(w_srcs)], q, s)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if args.eager:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        # The K steps are captured once into a HIP graph and replayed, so the
        # host-side cost of K separate calls stays off the timed path.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                step(i)
        graph.replay()                    # untimed: first replay uploads the graph
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    gpu_s = e0.elapsed_time(e1) / 1e3
    # per-launch average over the timed region, from HIP events on the launch
    # stream (a launch = one library call; with split-K that is the GEMM
    # kernel plus the ordered reduce kernel)
    avg_launch_s = gpu_s / steps

    flops = 2.0 * m * n * k
    abytes = alg_bytes(m, n, k)
    gn, gk = -(-n // 128), -(-k // 128)
    if op == "dequant":          # 1 B code in, 2 B bf16 out, plus the scale grid
        bound, flops, abytes = "hbm", 0.0, 3 * n * k + 4 * gn * gk
    elif op == "quantize":       # 4 B fp32 in, 1 B code out, plus the scale grid
        bound, flops, abytes = "hbm", 0.0, 5 * n * k + 4 * gn * gk
    elif op == "mlp":            # two products over one X, one bf16 output
        flops = 4.0 * m * n * k
        abytes = 2 * m * k + 2 * (n * k + 4 * gn * gk) + 2 * m * n
    mfma_peak, dtype = MFMA_BF16_PEAK_TFLOPS, "bf16"
    if op in ("w8a8", "w8a8_gemm"):
        # E4M3 x E4M3 products on the fp8 matrix cores, fp32 accumulation
        mfma_peak, dtype = MFMA_FP8_PEAK_TFLOPS, "fp8_e4m3"
        abytes = (m * k + 4 * m * -(-k // 128) + n * k + 4 * gn * gk + 2 * m * n
                  + (3 * m * k if op == "w8a8" else 0))
    if bound == "hbm":
        unit, value = "GB/s", abytes * steps / wall / 1e9
        achieved, peak, r_unit = abytes / avg_launch_s / 1e9, HBM_PEAK_GBPS, "GB/s"
    else:
        unit, value = "TFLOP/s", flops * steps / wall / 1e12
        achieved, peak, r_unit = flops / avg_launch_s / 1e12, mfma_peak, "TFLOP/s"
    traffic_key = workload if op == "linear" else f"{op}:{workload}"
    if path != "auto":
        traffic_key += f"@{path}"
    roof = {
        "bound": bound,
        "achieved": round(achieved, 3),
        "peak": peak,
        "unit": r_unit,
        "frac": round(achieved / peak, 4),
        "traffic": measured_traffic(traffic_key),
        "avg_launch_us": round(avg_launch_s * 1e6, 3),
        "launch": LAUNCH_KERNELS[op],
        "alg_bytes": abytes,
        "flops": flops,
    }
    if op == "linear" and bound == "hbm":
        # the weight stream alone (codes + scale grid), the part that scales with N*K
        wbytes = n * k + 4 * gn * gk
        roof["weight_GBps"] = round(wbytes / avg_launch_s / 1e9, 1)
    del sets, ws
    torch.cuda.empty_cache()
    return {
        "value": value, "unit": unit, "wall": wall, "dtype": dtype, "roofline": roof,
        "m": m, "n": n, "k": k, "rotate": rotate, "lin": lin, "x_bits": x_bits, "bound": bound,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dit_mlp_up", choices=sorted(WORKLOADS),
                    help="the workload of the headline line (default: the M=16384 DiT MLP "
                         "up projection, 16384x12288x3072)")
    ap.add_argument("--path", default="auto", choices=sorted(PATHS),
                    help="kernel choice for --op linear, w8a8_gemm and mlp (auto: the library's "
                         "own; w8a8_gemm and mlp take tiled or large)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the skinny-M (M=16, M=1) HBM-bound lines")
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets (0 = auto)")
    ap.add_argument("--op", default="linear",
                    choices=["linear", "dequant", "quantize", "mlp", "w8a8", "w8a8_gemm"],
                    help="linear (default): the fused layer; dequant / quantize: the "
                         "standalone kernels on the workload's weight; mlp: the gate/up "
                         "pair with the SwiGLU epilogue in one launch (workload mlp_gate); "
                         "w8a8: per-token activation quantize + FP8 x FP8 GEMM from bf16 X; "
                         "w8a8_gemm: the FP8 GEMM alone on pre-quantized X")
    ap.add_argument("--eager", action="store_true",
                    help="time K separate calls instead of one replay of a captured graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only time plain streaming reads and a copy (practical HBM ceilings) and exit")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration, "launches": 5}))
        return

    if args.stream_ceiling:
        print(json.dumps({"stream_ceiling": stream_ceiling()}))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer would shard by rows of X, or by columns or rows of W with a "
              "gather or sum of the partial outputs across GPUs).",
              file=sys.stderr)
        sys.exit(2)

    if args.op == "mlp" and args.workload != "mlp_gate":
        print("--op mlp runs on the gate/up pair: use --workload mlp_gate", file=sys.stderr)
        sys.exit(2)

    r = measure(args, args.workload, args.op, args.path)
    m, n, k = r["m"], r["n"], r["k"]
    out = {
        "metric": "FP8-block linear TFLOP/s (% bf16 MFMA peak) and weight GB/s (% HBM) at M<=32",
        "value": round(r["value"], 3),
        "unit": r["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall"] / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "op": args.op, "path": args.path, "m": m, "n": n,
                   "k": k, "weight": "e4m3 + fp32 128x128 scale_inv",
                   "rotated_sets": r["rotate"],
                   "launch": "eager" if args.eager else "hip graph of K steps",
                   "parallelism": "none (1 GPU)"},
        "roofline": r["roofline"],
    }
    if args.op == "linear" and not args.no_secondary and args.workload not in SECONDARY:
        # The metric's other half: the HBM-bound skinny shapes (M <= 32), each
        # timed the same way (its own rotated buffer sets, graph replay).
        sec = []
        for wname in SECONDARY:
            rs = measure(args, wname, "linear", "auto", steps=max(args.steps, 200),
                         warmup=args.warmup)
            sec.append({"workload": wname, "m": rs["m"], "n": rs["n"], "k": rs["k"],
                        "value": round(rs["value"], 3), "unit": rs["unit"],
                        "rotated_sets": rs["rotate"], "roofline": rs["roofline"]})
        out["secondary"] = sec
    if not args.no_cpu_baseline and args.op == "linear":
        cb = cpu_baseline(r["lin"], r["x_bits"])
        rows, passes = cb.pop("rows"), cb.pop("passes")
        if r["bound"] == "hbm":
            # oracle throughput expressed in the metric's unit (bytes of the sample)
            cb["value"] = alg_bytes(rows, n, k) * passes / cb.pop("seconds") / 1e9
            cb["unit"] = "GB/s"
        else:
            cb.pop("seconds")
        cb["value"] = round(cb["value"], 6)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
