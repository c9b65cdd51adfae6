"""Benchmark of the PTPC-FP8 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 70b_down]

One step = every stage of the path over one batch of resident synthetic
input: per-channel weight quantization + prepack, per-token activation
quantization, the fused FP8 GEMM, and the two-step (unfused) GEMM.  Each
stage is bracketed by HIP events on the stream it runs on, so per-kernel
averages come from the timed region itself.

Every timing rotates over several copies of the inputs at distinct
addresses, more than 768 MiB in all, so that no stage finds its input in
the GPU's 256 MB memory-side cache from an earlier repetition: what the
HBM figures measure is HBM.

Prints one JSON line.  `value` is whole-step throughput: the FP8 contraction
work of the step (two GEMMs, 2*T*Ci*Co flops each) divided by the step time.
`roofline` is the fused GEMM against the dense FP8 MFMA peak; `quant_act`
carries the activation quantizer against HBM bandwidth; `comparison` holds
the other forms timed in interleaved rounds; `judged_shapes` the fused GEMM
and the activation quantizer on the other large layer shapes; `cpu_baseline`
is the CPU oracle on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ROTATE_BYTES = 768 << 20      # rotated input bytes: three times the 256 MB memory-side cache
MAX_SETS = 64

# HBM-traffic records (rocprofv3 FETCH_SIZE / WRITE_SIZE of one kernel on
# the default workload), valid only while the kernel's code is unchanged.
TRAFFIC = {
    "gemm_fused": {"file": "gemm_fused_70b_down_traffic.json",
                   "sources": ("gemm.hip", "device_common.h"),
                   "kernel": "gemm16_kernel<256, 256, 2, 2, true, false>"},
    "quant_act": {"file": "quant_act_70b_down_traffic.json",
                  "sources": ("quant.hip", "device_common.h"),
                  "kernel": "quant_act_kernel<256, 16>"},
}


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=30,
                   help="untimed steps first; the shader clock needs tens of ms to settle")
    p.add_argument("--workload", default="70b_down")
    p.add_argument("--layer", default=None, help="70b_sweep layer")
    p.add_argument("--T", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-judged", action="store_true",
                   help="skip the per-shape lines of the other large layer shapes")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--only", default=None,
                   help="comma list of stages to run (profiling); default all")
    p.add_argument("--judged-only", default=None,
                   help="profiling: run only the judged shapes whose names contain this text")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="run a plain device copy of this many MiB (3x) before timing, "
                        "as the reference kernel for HBM byte counters")
    p.add_argument("--scaled-mm-context", action="store_true",
                   help="context only: time torch._scaled_mm (hipBLASLt) in the pages' two forms "
                        "(row-wise scales; unit scales + two multiplies) and per-tensor, on the "
                        "same quantized data as ptpc_gemm (one JSON line)")
    p.add_argument("--model-load", action="store_true",
                   help="quantize + prepack every linear weight of the 80 Llama-3.1-70B "
                        "decoder layers and report the load-time cost (one JSON line)")
    p.add_argument("--sweep", action="store_true",
                   help="one JSON line per workload shape (every config, every 70B layer x T): "
                        "quant_act GB/s, fused / two-step GEMM TFLOP/s; not the bench line")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                        "--only <kernel> --copy-calibration-mb run into the traffic record of "
                        "--traffic-kernel and exit (no GPU needed)")
    p.add_argument("--traffic-kernel", default="gemm_fused", choices=sorted(TRAFFIC))
    p.add_argument("--shapes", default=None, metavar="T:Ci:Co,...",
                   help="ptpc_gemm and ptpc_gemm_ws on these shapes (inputs drawn on the GPU, "
                        "rotated, graph-timed in interleaved rounds); one JSON line per shape")
    p.add_argument("--timeline", action="store_true",
                   help="per-workgroup phases of the tiled GEMM (timeline debug build) on the "
                        "bench workload and the judged shapes; one JSON line per shape")
    return p.parse_args(argv)


# ---------------------------------------------------------------------------
# HBM traffic records
# ---------------------------------------------------------------------------
def source_hash(kind):
    """Hash of a kernel's code (its sources with comments and blank space
    removed), so that a traffic record stays valid across comment edits and
    is dropped on any code change."""
    import re
    text = ""
    for name in TRAFFIC[kind]["sources"]:
        with open(os.path.join(ROOT, "scaled_gemm_amd", "csrc", name)) as f:
            text += f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def traffic_file(kind):
    return os.path.join(ROOT, "profiles", TRAFFIC[kind]["file"])


def measured_traffic(workload, kind):
    """HBM bytes per launch of `kind` from rocprofv3 FETCH_SIZE/WRITE_SIZE,
    only if the counters were taken on this workload and the current code."""
    try:
        with open(traffic_file(kind)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("source_sha256_16") != source_hash(kind):
        return None
    return t.get("bytes_per_launch")


def traffic_record(fetch_csv, write_csv, workload, copy_mb, kind):
    """HBM bytes per launch: the FETCH_SIZE / WRITE_SIZE counters (KiB per
    dispatch) of the kernel, each scaled by the ratio of the known bytes of a
    plain device copy to what the same counter reads for it."""
    import csv

    match = TRAFFIC[kind]["kernel"]

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                key = "kernel" if match in name else "copy" if "copyBuffer" in name else None
                if key:
                    vals.setdefault(key, []).append(float(r["Counter_Value"]))
        # The input copies of the rotation are device copies too; the
        # calibration copies are the largest of the run (copy_mb, more than
        # any input copy): keep only those.
        big = max(vals["copy"])
        vals["copy"] = [v for v in vals["copy"] if v >= 0.95 * big]
        assert len(vals["copy"]) == 3, "expected the three calibration copies"
        return {k: sum(v) / len(v) for k, v in vals.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = float(copy_mb) * (1 << 20)
    f_factor = copy_bytes / (f["copy"] * 1024.0)
    w_factor = copy_bytes / (w["copy"] * 1024.0)
    fetch = f["kernel"] * 1024.0 * f_factor
    write = w["kernel"] * 1024.0 * w_factor
    prof = (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {{c}} --output-format csv "
            f"-d $OUT/prof_{{d}} -o p -- python -u $REPO/bench.py --steps 3 "
            f"--warmup 1 --no-cpu-baseline --no-judged --only {kind} "
            f"--copy-calibration-mb {copy_mb}")
    return {"workload": workload, "source_sha256_16": source_hash(kind),
            "kernel": f"{match} ({kind}, this workload's launch)",
            "fetch_kib_raw": f["kernel"], "write_kib_raw": w["kernel"],
            "copy_bytes": copy_bytes, "copy_fetch_kib_raw": f["copy"],
            "copy_write_kib_raw": w["copy"], "fetch_factor": f_factor,
            "write_factor": w_factor, "fetch_bytes": fetch, "write_bytes": write,
            "bytes_per_launch": fetch + write,
            "commands": [
                prof.format(c="FETCH_SIZE", d="fetch"), prof.format(c="WRITE_SIZE", d="write"),
                "python bench.py --traffic-from $OUT/prof_fetch/p_counter_collection.csv "
                f"$OUT/prof_write/p_counter_collection.csv --copy-calibration-mb "
                f"{copy_mb} --traffic-kernel {kind}"],
            "note": ("Counters in KiB per dispatch, averaged over the kernel's launches (inputs "
                     "rotating over copies larger than the memory-side cache); each scaled by "
                     "known copy bytes / counter reading for a device copy of "
                     f"{copy_mb} MiB (torch copy_) in the same run.")}


# ---------------------------------------------------------------------------
# CPU baseline
# ---------------------------------------------------------------------------
def cpu_baseline(x_bits, w_bits, target_s):
    """The CPU oracle (as it stands) on the first R token rows with the whole
    weight: quantize, contract exactly, scale.  The oracle spreads rows over
    its threads, so R is a multiple of the thread count, grown until about
    target_s seconds of CPU work."""
    import numpy as np
    import oracle
    Ci, Co = w_bits.shape
    nthr = oracle.num_threads()
    t0 = time.perf_counter()
    qw, dw = oracle.quant_weight(w_bits)
    t_w = time.perf_counter() - t0

    def rows(R):
        t0 = time.perf_counter()
        qx, dx = oracle.quant_act(np.ascontiguousarray(x_bits[:R]))
        oracle.apply_scales(oracle.gemm_exact(qx, qw), dx, dw)
        return time.perf_counter() - t0

    R = min(nthr, x_bits.shape[0])
    t_g = rows(R)
    reps = int((target_s - t_w - t_g) / max(t_g, 1e-6))
    if reps >= 1 and R < x_bits.shape[0]:
        R = min(x_bits.shape[0], R * (reps + 1))
        t_g = rows(R)
    total = t_w + t_g
    flops = 2.0 * R * Ci * Co
    nproc = os.cpu_count()
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": min(nthr, R),
            "kind": "oracle", "nproc": nproc, "cpus_available": affinity,
            "sample": (f"first {R} token rows of the workload with its whole weight: "
                       f"quant_weight [{Ci}x{Co}] + quant_act [{R}x{Ci}] + exact GEMM "
                       f"[{R}x{Ci}]x[{Ci}x{Co}] + scales; {total:.1f} s wall "
                       f"(weight quantization {t_w:.1f} s); {nthr} OpenMP threads, "
                       f"nproc {nproc}, {affinity} CPUs available to the process")}


def no_nan(v):
    """JSON has no NaN: stages that did not run (--only) report null."""
    if isinstance(v, float) and v != v:
        return None
    if isinstance(v, dict):
        return {k: no_nan(x) for k, x in v.items()}
    if isinstance(v, list):
        return [no_nan(x) for x in v]
    return v


def act_bytes(T, Ci):
    """Algorithmic bytes of the activation quantizer: 2 read + 1 written per
    element, 4 per row scale."""
    return 3.0 * T * Ci + 4.0 * T


def gemm_min_bytes(T, Ci, Co):
    return T * Ci + Ci * Co + 2.0 * T * Co + 4.0 * (T + Co)


def round_k(Ci):
    """K extent of the packed weight (whole 128-byte K tiles)."""
    return (Ci + 127) // 128 * 128


def n_sets(set_bytes):
    """Input copies to rotate over so that more than ROTATE_BYTES pass
    between two uses of one copy (at least 3)."""
    return int(min(MAX_SETS, max(3, math.ceil(ROTATE_BYTES / max(set_bytes, 1)) + 2)))


def batch_ms(launch, n, stream):
    """Per-launch time of n back-to-back launches between one HIP event pair
    on `stream`; launch(i) issues repetition i (on input copy i mod sets)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for i in range(n):
        launch(i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / n


def graph_ms(launch, n, stream, replays=5):
    """Per-launch time of n launches captured once in a HIP graph and
    replayed: the GPU time of short kernels without the host's per-call cost
    (launch(i) issues repetition i on input copy i mod sets; nothing the
    captured calls launch clears memory with a memset).  Median over replays,
    each between its own event pair on `stream`."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                launch(i)
    stream.wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    t = []
    for _ in range(replays):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        g.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        t.append(ev[0].elapsed_time(ev[1]) / n)
    del g
    return sorted(t)[len(t) // 2]


# ---------------------------------------------------------------------------
# model-scale load time, hipBLASLt context, sweep
# ---------------------------------------------------------------------------
def model_load(args):
    """Load-time weight quantization at model scale: each of the 80 decoder
    layers' four linear weights is drawn in bf16 on the GPU, quantized per
    output channel and prepacked (HIP events around each ptpc_quant_weight),
    and the bf16 copy is freed, as a loader that quantizes on the fly would;
    the packed weights of all layers stay resident."""
    import numpy as np
    import torch

    import scaled_gemm_amd as sg
    import workloads

    dev = torch.device("cuda:0")
    sg.lib()
    stream = torch.cuda.current_stream()
    packed, times, elems = [], [], 0
    t0 = time.perf_counter()
    for layer in range(workloads.LLAMA70B_LAYERS):
        for index, (name, (Ci, Co)) in enumerate(workloads.SWEEP_LAYERS.items()):
            w = workloads.device_weight(layer, index, Ci, Co, 0.01, dev)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pw = sg.quant_weight(w)
            e1.record(stream)
            packed.append(pw)
            times.append((e0, e1))
            elems += Ci * Co
            del w
        if layer % 10 == 9:
            torch.cuda.synchronize()
            print(f"# layers done: {layer + 1}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in times]
    total_ms = float(np.sum(ms))
    resident = sum(p.data.numel() + 4 * p.dw.numel() for p in packed)
    print(json.dumps({
        "what": "load-time per-channel quantization + prepack of every linear weight of "
                "Llama-3.1-70B (80 layers x qkv/o/gate_up/down), bf16 drawn on the GPU",
        "layers": workloads.LLAMA70B_LAYERS, "weights": len(packed),
        "bf16_bytes": 2 * elems, "packed_bytes_resident": resident,
        "quant_weight_ms_total": round(total_ms, 2),
        "quant_weight_gbs": round(3.0 * elems / (total_ms * 1e-3) / 1e9, 1),
        "per_layer_ms": round(total_ms / workloads.LLAMA70B_LAYERS, 3),
        "max_memory_allocated_gb": round(torch.cuda.max_memory_allocated() / 1e9, 1),
        "wall_s_including_generation": round(wall, 1),
    }), flush=True)


def scaled_mm_context(args):
    """torch._scaled_mm (hipBLASLt) on the same quantized operands as
    ptpc_gemm, in the two forms the pages show -- the fused call with
    row-wise token / channel scales, and the naive one (unit scales, then a
    multiply by each scale vector) -- and with per-tensor scales.  Context
    only: nothing in the library calls it."""
    import numpy as np
    import torch

    import scaled_gemm_amd as sg
    import workloads

    dev = torch.device("cuda:0")
    sg.lib()
    if args.workload == "70b_sweep":
        shape, xb, wb = workloads.make("70b_sweep", T=args.T or 8192, layer=args.layer or "gate_up")
    else:
        shape, xb, wb = workloads.make(args.workload, T=args.T)
    T, Ci, Co = shape.T, shape.Ci, shape.Co
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(dev)
    del xb, wb
    qx, dx = sg.quant_act(x)
    pw = sg.quant_weight(w)
    a8 = qx.view(torch.float8_e4m3fn)
    b8 = sg.unpack_weight(pw).t().contiguous().view(torch.float8_e4m3fn).t()  # column-major
    sa, sb = dx.view(T, 1).contiguous(), pw.dw.view(1, Co).contiguous()
    one = torch.ones((), dtype=torch.float32, device=dev)
    out = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((max(1, sg.gemm_workspace_bytes(T, Ci, Co)),), dtype=torch.uint8, device=dev)
    calls = {
        "ptpc_gemm": lambda: sg.gemm(qx, dx, pw, out=out),
        "ptpc_gemm_ws": lambda: sg.gemm_ws(qx, dx, pw, out=out, workspace=ws),
        "scaled_mm_rowwise": lambda: torch._scaled_mm(a8, b8, scale_a=sa, scale_b=sb,
                                                      out_dtype=torch.bfloat16),
        "scaled_mm_naive": lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one,
                                                    out_dtype=torch.bfloat16) * sa * sb,
        "scaled_mm_per_tensor": lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one,
                                                         out_dtype=torch.bfloat16),
    }
    # Every form warmed up, then three interleaved rounds of `steps` calls
    # each; the best round counts (the clock drifts while a box warms up, and
    # whichever form ran first would otherwise pay for it).
    ms = {}
    for k, fn in list(calls.items()):
        try:
            for _ in range(max(3, args.warmup)):
                fn()
        except RuntimeError as e:                      # a form hipBLASLt does not support
            ms[k] = None
            del calls[k]
            print(f"# {k}: {e}", file=sys.stderr)
    torch.cuda.synchronize()
    for _ in range(3):
        for k, fn in calls.items():
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            for _ in range(args.steps):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            t = ev[0].elapsed_time(ev[1]) / args.steps
            ms[k] = t if ms.get(k) is None else min(ms[k], t)
    flops = 2.0 * T * Ci * Co
    print(json.dumps({
        "what": "context only: torch._scaled_mm (hipBLASLt) on the same quantized data",
        "workload": shape.name, "T": T, "Ci": Ci, "Co": Co,
        "ms": {k: (round(v, 4) if v else None) for k, v in ms.items()},
        "tflops": {k: (round(flops / v / 1e9, 1) if v else None) for k, v in ms.items()},
    }), flush=True)


def sweep(args):
    """Per-shape kernel rates over every workload shape.  After a warm-up,
    three interleaved rounds over the stages; each round captures a run of
    launches rotating over copies of the inputs (more than 768 MiB between
    two uses of a copy) in a HIP graph and times its replays (median of 3,
    each between one HIP event pair), so that the host's per-call cost does
    not enter the few-microsecond shapes; the best round per stage."""
    import numpy as np
    import torch

    import scaled_gemm_amd as sg
    import workloads

    dev = torch.device("cuda:0")
    sg.lib()
    shapes = [("tiny", None, None), ("8b_qkv_decode", None, None), ("8b_gate_up", None, None),
              ("70b_down", None, None)]
    shapes += [("70b_sweep", T, layer) for layer in workloads.SWEEP_LAYERS
               for T in workloads.SWEEP_T]
    stream = torch.cuda.current_stream()
    for name, T_, layer in shapes:
        if name == "70b_sweep":
            shape, x_bits, w_bits = workloads.make(name, T=T_, layer=layer)
        else:
            shape, x_bits, w_bits = workloads.make(name)
        T, Ci, Co = shape.T, shape.Ci, shape.Co
        x0 = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        w0 = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        del x_bits, w_bits
        pw0 = sg.quant_weight(w0)
        qx0, dx0 = sg.quant_act(x0)
        n = n_sets(T * Ci + pw0.data.numel())
        nx = n_sets(2 * T * Ci)
        xs = [x0] + [x0.clone() for _ in range(nx - 1)]
        qxs = [qx0] + [qx0.clone() for _ in range(max(n, nx) - 1)]
        dxs = [dx0] + [dx0.clone() for _ in range(max(n, nx) - 1)]
        pws = [pw0] + [sg.PackedWeight(pw0.data.clone(), pw0.dw.clone(), Ci, Co)
                       for _ in range(n - 1)]
        ws_ = [w0] + [w0.clone() for _ in range(2)]
        sx_t = sg.tensor_scale(x0)
        pw_t = sg.quant_weight_static(w0, sg.tensor_scale(w0))
        pwts = [pw_t] + [sg.PackedWeight(pw_t.data.clone(), pw_t.dw, Ci, Co, per_tensor=True)
                         for _ in range(n - 1)]
        out = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((T, Co), dtype=torch.float32, device=dev)
        ws16 = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
        gws = torch.empty((max(1, sg.gemm_workspace_bytes(T, Ci, Co)),), dtype=torch.uint8,
                          device=dev)
        calls = {
            "quant_weight": lambda i: sg.quant_weight(ws_[i % 3], out=pws[i % n]),
            "quant_act": lambda i: sg.quant_act(xs[i % nx], qx=qxs[i % nx], dx=dxs[i % nx]),
            "gemm_fused": lambda i: sg.gemm(qxs[i % n], dxs[i % n], pws[i % n], out=out),
            "gemm_unfused": lambda i: sg.gemm_unfused(qxs[i % n], dxs[i % n], pws[i % n],
                                                      out=out, workspace=ws),
            "gemm_unfused_bf16": lambda i: sg.gemm_unfused_bf16(qxs[i % n], dxs[i % n],
                                                                pws[i % n], out=out,
                                                                workspace=ws16),
            "gemm_tensor": lambda i: sg.gemm_tensor(qxs[i % n], sx_t, pwts[i % n], out=out),
            "gemm_ws": lambda i: sg.gemm_ws(qxs[i % n], dxs[i % n], pws[i % n], out=out,
                                            workspace=gws),
        }
        for fn in calls.values():
            for i in range(max(3, args.warmup)):
                fn(i)
        rounds = {k: [] for k in calls}
        reps = max(args.steps, 2 * max(n, nx))
        for _ in range(3):
            for k, fn in calls.items():
                rounds[k].append(graph_ms(fn, reps, stream, replays=3))
        ms = {k: min(v) for k, v in rounds.items()}
        flops = 2.0 * T * Ci * Co
        ab = act_bytes(T, Ci)
        print(json.dumps({
            "workload": shape.name, "T": T, "Ci": Ci, "Co": Co,
            "gemm_kernel": sg.gemm_kernel(T, Ci, Co), "input_copies": n,
            "ms": {k: round(v, 4) for k, v in ms.items()},
            "gemm_fused_tflops": round(flops / ms["gemm_fused"] / 1e9, 1),
            "gemm_fused_frac_fp8_peak": round(flops / ms["gemm_fused"] / 1e9 / PEAK_FP8_TFLOPS, 4),
            "gemm_fused_gbs_min_bytes": round(gemm_min_bytes(T, Ci, Co) / ms["gemm_fused"] / 1e6, 1),
            "gemm_unfused_tflops": round(flops / ms["gemm_unfused"] / 1e9, 1),
            "fused_over_unfused": round(ms["gemm_unfused"] / ms["gemm_fused"], 3),
            "fused_over_unfused_bf16": round(ms["gemm_unfused_bf16"] / ms["gemm_fused"], 3),
            "ptpc_over_per_tensor_gemm": round(ms["gemm_fused"] / ms["gemm_tensor"], 3),
            "gemm_ws_speedup": round(ms["gemm_fused"] / ms["gemm_ws"], 3),
            "gemm_ws_gbs_min_bytes": round(gemm_min_bytes(T, Ci, Co) / ms["gemm_ws"] / 1e6, 1),
            "quant_act_gbs": round(ab / ms["quant_act"] / 1e6, 1),
            "quant_act_frac_hbm": round(ab / ms["quant_act"] / 1e6 / PEAK_HBM_GBS, 4),
            "quant_weight_gbs": round((3.0 * Ci * Co + 4.0 * Co) / ms["quant_weight"] / 1e6, 1),
        }), flush=True)
        del x0, w0, xs, qxs, dxs, pws, ws_, pwts, pw_t, sx_t, out, ws, ws16, gws, calls
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# the other large layer shapes the performance targets are quoted on
# ---------------------------------------------------------------------------
def judged_shapes(stream, only=None):
    """The fused GEMM and the activation quantizer on the 70B layers at 1024
    and 8192 tokens and the 8B gate_up layer, inputs drawn on the GPU with
    the workloads' value structure.  Each figure: after a warm-up, five rounds
    of launches between one HIP event pair, rotating over input copies (more
    than 768 MiB between two uses of a copy); the median round.  The GEMM's
    rounds are back-to-back launches; the activation quantizer's (3-130 us
    kernels, shorter than the host's per-call cost at the smaller shapes)
    replay the launches captured in a HIP graph.  Where the workspace form
    splits K (ptpc_gemm_ws; the 70B down projection at 1024 tokens), it is
    timed the same way, partial sums and their reduction included."""
    import torch

    import scaled_gemm_amd as sg
    import workloads

    dev = torch.device("cuda:0")
    shapes = [("8b_gate_up", 2048, 4096, 28672, "outlier_normal", 0.02)]
    shapes += [(f"70b_{layer}", T, Ci, Co, "student_lognormal", 0.01)
               for layer, (Ci, Co) in workloads.SWEEP_LAYERS.items() for T in (1024, 8192)]
    res = []
    for k, (name, T, Ci, Co, kind, sigma) in enumerate(shapes):
        if only and only not in f"{name}_T{T}":
            continue
        x = workloads.device_activation(kind, T, Ci, 7000 + k, dev)
        w = workloads.device_weight(100, k, Ci, Co, sigma, dev)
        pw = sg.quant_weight(w)
        del w
        qx, dx = sg.quant_act(x)
        n = n_sets(T * Ci + pw.data.numel())
        nx = n_sets(2 * T * Ci)
        pws = [pw] + [sg.PackedWeight(pw.data.clone(), pw.dw.clone(), Ci, Co) for _ in range(n - 1)]
        qxs = [qx] + [qx.clone() for _ in range(max(n, nx) - 1)]
        dxs = [dx] + [dx.clone() for _ in range(max(n, nx) - 1)]
        xs = [x] + [x.clone() for _ in range(nx - 1)]
        out = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)

        def gemm(i):
            sg.gemm(qxs[i % n], dxs[i % n], pws[i % n], out=out)

        def act(i):
            sg.quant_act(xs[i % nx], qx=qxs[i % nx], dx=dxs[i % nx])

        for i in range(3 * n):
            gemm(i)
        for i in range(2 * nx):
            act(i)
        reps_g = max(2 * n, 10)
        reps_a = max(2 * nx, 20)
        g_eager = sorted(batch_ms(gemm, reps_g, stream) for _ in range(5))[2]
        g_ms = graph_ms(gemm, reps_g, stream)
        a_ms = graph_ms(act, reps_a, stream)
        flops = 2.0 * T * Ci * Co
        ws_rec = {}
        ws_bytes = sg.gemm_workspace_bytes(T, Ci, Co)
        if ws_bytes:
            wsb = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)

            def gemm_ws(i):
                sg.gemm_ws(qxs[i % n], dxs[i % n], pws[i % n], out=out, workspace=wsb)

            for i in range(2 * n):
                gemm_ws(i)
            w_ms = graph_ms(gemm_ws, reps_g, stream)
            ws_rec = {"gemm_ws_ms": round(w_ms, 4),
                      "gemm_ws_splits": sg.gemm_ws_splits(T, Ci, Co),
                      "gemm_ws_frac_fp8_peak": round(flops / w_ms / 1e9 / PEAK_FP8_TFLOPS, 4)}
            del wsb
        res.append({
            "shape": f"{name}_T{T}", "T": T, "Ci": Ci, "Co": Co,
            "gemm_kernel": sg.gemm_kernel(T, Ci, Co),
            "gemm_ms": round(g_ms, 4), "gemm_eager_batch_ms": round(g_eager, 4),
            "gemm_tflops": round(flops / g_ms / 1e9, 1),
            "gemm_frac_fp8_peak": round(flops / g_ms / 1e9 / PEAK_FP8_TFLOPS, 4),
            "quant_act_ms": round(a_ms, 4),
            "quant_act_gbs": round(act_bytes(T, Ci) / a_ms / 1e6, 1),
            "quant_act_frac_hbm": round(act_bytes(T, Ci) / a_ms / 1e6 / PEAK_HBM_GBS, 4),
            **ws_rec,
            "input_copies": {"gemm": n, "quant_act": nx},
        })
        print(f"# judged {name} T={T}: gemm {res[-1]['gemm_frac_fp8_peak']:.3f} of FP8 peak, "
              f"quant_act {res[-1]['quant_act_frac_hbm']:.3f} of HBM", file=sys.stderr, flush=True)
        del x, pw, qx, dx, pws, qxs, dxs, xs, out
        torch.cuda.empty_cache()
    return res


def shapes_mode(args):
    """ptpc_gemm and ptpc_gemm_ws on the given (T, Ci, Co): the 70B layers'
    activation structure (Student-t x log-normal rows) and normal weights,
    drawn on the GPU, rotated over copies (more than 768 MiB between two uses
    of one); after a warm-up, three interleaved rounds of graph replays of
    each form, the best round.  The workspace form's time includes its
    partial sums and their reduction where it splits K."""
    import torch

    import scaled_gemm_amd as sg
    import workloads

    stream = torch.cuda.current_stream()
    dev = torch.device("cuda:0")
    for k, spec in enumerate(args.shapes.split(",")):
        T, Ci, Co = (int(v) for v in spec.split(":"))
        x = workloads.device_activation("student_lognormal", T, Ci, 9000 + k, dev)
        w = workloads.device_weight(200, k, Ci, Co, 0.01, dev)
        pw = sg.quant_weight(w)
        del w
        qx, dx = sg.quant_act(x)
        del x
        n = n_sets(T * Ci + pw.data.numel())
        pws = [pw] + [sg.PackedWeight(pw.data.clone(), pw.dw.clone(), Ci, Co) for _ in range(n - 1)]
        qxs = [qx] + [qx.clone() for _ in range(n - 1)]
        dxs = [dx] + [dx.clone() for _ in range(n - 1)]
        out = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
        ws_bytes = sg.gemm_workspace_bytes(T, Ci, Co)
        wsb = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)

        def gemm(i):
            sg.gemm(qxs[i % n], dxs[i % n], pws[i % n], out=out)

        def gemm_ws(i):
            sg.gemm_ws(qxs[i % n], dxs[i % n], pws[i % n], out=out, workspace=wsb)

        reps = max(2 * n, 10)
        for i in range(2 * n):
            gemm(i)
            gemm_ws(i)
        t = {"gemm": [], "gemm_ws": []}
        for _ in range(3):
            t["gemm"].append(graph_ms(gemm, reps, stream))
            t["gemm_ws"].append(graph_ms(gemm_ws, reps, stream))
        g, w_ = min(t["gemm"]), min(t["gemm_ws"])
        flops = 2.0 * T * Ci * Co
        print(json.dumps({
            "shape": f"T{T}_Ci{Ci}_Co{Co}", "T": T, "Ci": Ci, "Co": Co,
            "gemm_kernel": sg.gemm_kernel(T, Ci, Co),
            "gemm_us": round(g * 1e3, 1),
            "gemm_frac_fp8_peak": round(flops / g / 1e9 / PEAK_FP8_TFLOPS, 4),
            "gemm_ws_splits": sg.gemm_ws_splits(T, Ci, Co),
            "gemm_ws_us": round(w_ * 1e3, 1),
            "gemm_ws_frac_fp8_peak": round(flops / w_ / 1e9 / PEAK_FP8_TFLOPS, 4),
            "ws_speedup": round(g / w_, 3),
            "input_copies": n,
        }), flush=True)
        del qx, dx, pw, pws, qxs, dxs, out, wsb
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# timeline of the tiled GEMM (debug build)
# ---------------------------------------------------------------------------
def timeline(args):
    """Where the fused GEMM's time goes, per workgroup: the timeline debug
    build of the library (libptpc_timeline.so) records, for every workgroup
    of the tiled kernel, its start, the moment its K loop begins (first
    operands landed), the end of its K loop and the completion of its last
    output store.  Inputs are drawn on the GPU (the 70B layers' Student-t x
    log-normal structure, the 8B layers' outlier channels) and rotate over
    copies as in every other timing; after
    a warm-up of back-to-back launches, three launches are recorded, each
    between its own HIP event pair; the median one is reported.  Workgroups
    are grouped into rounds of 256 (one per CU) by start time."""
    import ctypes

    import numpy as np
    import torch

    import scaled_gemm_amd as sg
    import workloads
    from scaled_gemm_amd import build

    dev = torch.device("cuda:0")
    sg.lib()
    stream = torch.cuda.current_stream()
    L = ctypes.CDLL(build.TIMELINE_LIB)
    P, I = ctypes.c_void_p, ctypes.c_int64
    L.ptpc_gemm.restype = ctypes.c_int
    L.ptpc_gemm.argtypes = [P, I, P, P, P, I, I, I, P, I, P]
    L.ptpc_debug_set_timeline.restype = ctypes.c_int
    L.ptpc_debug_set_timeline.argtypes = [P]
    shapes = [("70b_down", 4096, 28672, 8192, "student_lognormal", 0.01),
              ("8b_gate_up", 2048, 4096, 28672, "outlier_normal", 0.02)]
    shapes += [(f"70b_{layer}", T, Ci, Co, "student_lognormal", 0.01)
               for layer, (Ci, Co) in workloads.SWEEP_LAYERS.items() for T in (1024, 8192)]
    for k, (name, T, Ci, Co, kind, sigma) in enumerate(shapes):
        kname = sg.gemm_kernel(T, Ci, Co)
        if not kname.startswith("gemm16_kernel<"):
            continue
        bm, bn = (int(v) for v in kname[len("gemm16_kernel<"):].split(",")[:2])
        x = workloads.device_activation(kind, T, Ci, 9000 + k, dev)
        w = workloads.device_weight(200, k, Ci, Co, sigma, dev)
        pw = sg.quant_weight(w)
        del w
        qx, dx = sg.quant_act(x)
        del x
        n = n_sets(T * Ci + pw.data.numel())
        pws = [pw] + [sg.PackedWeight(pw.data.clone(), pw.dw.clone(), Ci, Co) for _ in range(n - 1)]
        qxs = [qx] + [qx.clone() for _ in range(n - 1)]
        out = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
        ref = sg.gemm(qx, dx, pw)
        wgs = ((T + bm - 1) // bm) * ((Co + bn - 1) // bn)
        buf = torch.zeros((wgs, 4), dtype=torch.int64, device=dev)

        def run(i):
            assert L.ptpc_gemm(P(qxs[i % n].data_ptr()), Ci, P(dx.data_ptr()),
                               P(pws[i % n].data.data_ptr()), P(pws[i % n].dw.data_ptr()), T, Ci,
                               Co, P(out.data_ptr()), Co, P(stream.cuda_stream)) == 0

        assert L.ptpc_debug_set_timeline(None) == 0
        for i in range(2 * n):
            run(i)
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.int16), ref.view(torch.int16))
        recs = []
        for rep in range(3):
            buf.zero_()
            torch.cuda.synchronize()
            assert L.ptpc_debug_set_timeline(P(buf.data_ptr())) == 0
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(rep + 1)
            e1.record(stream)
            torch.cuda.synchronize()
            assert L.ptpc_debug_set_timeline(None) == 0
            t = buf.cpu().numpy().astype(np.float64) * 0.01          # 100 MHz ticks -> us
            assert np.all(t[:, 0] > 0), "a workgroup did not record"
            t -= t[:, 0].min()
            recs.append((e0.elapsed_time(e1) * 1e3, t))
        recs.sort(key=lambda r: r[0])
        ev_us, t = recs[1]
        pro, kl, epi = t[:, 1] - t[:, 0], t[:, 2] - t[:, 1], t[:, 3] - t[:, 2]
        order = np.argsort(t[:, 0])
        rounds = []
        for r0 in range(0, wgs, 256):
            idx = order[r0:r0 + 256]
            rounds.append({"workgroups": int(idx.size),
                           "start_us": [round(float(t[idx, 0].min()), 2),
                                        round(float(t[idx, 0].max()), 2)],
                           "end_us": [round(float(t[idx, 3].min()), 2),
                                      round(float(t[idx, 3].max()), 2)],
                           "prologue_us_median": round(float(np.median(pro[idx])), 2),
                           "k_loop_us_median": round(float(np.median(kl[idx])), 2),
                           "epilogue_us_median": round(float(np.median(epi[idx])), 2)})
        tile_flops = 2.0 * bm * bn * round_k(Ci)
        kl_rate = tile_flops / (np.median(kl) * 1e-6) * 256 / 1e12
        flops = 2.0 * T * Ci * Co
        print(json.dumps({
            "shape": f"{name}_T{T}", "T": T, "Ci": Ci, "Co": Co, "kernel": kname,
            "workgroups": wgs, "output_equals_release": same,
            "event_us": round(ev_us, 2), "span_us": round(float(t[:, 3].max()), 2),
            "frac_fp8_peak_event": round(flops / (ev_us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "prologue_us": [round(float(v), 2) for v in np.percentile(pro, [10, 50, 90])],
            "k_loop_us": [round(float(v), 2) for v in np.percentile(kl, [10, 50, 90])],
            "epilogue_us": [round(float(v), 2) for v in np.percentile(epi, [10, 50, 90])],
            "k_loop_tflops_if_256_cus": round(float(kl_rate), 1),
            "k_loop_frac_fp8_peak": round(float(kl_rate) / PEAK_FP8_TFLOPS, 4),
            "rounds": rounds,
        }), flush=True)
        del pws, qxs, out, ref, buf, pw, qx, dx
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# the bench line
# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "libptpc runs on one GPU (no multi-GPU sharding); "
                                   "--gpus must be 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    if args.model_load:
        model_load(args)
        return
    if args.scaled_mm_context:
        scaled_mm_context(args)
        return
    if args.timeline:
        timeline(args)
        return
    if args.shapes:
        shapes_mode(args)
        return
    if args.traffic_from:
        rec = traffic_record(args.traffic_from[0], args.traffic_from[1], args.workload,
                             args.copy_calibration_mb or 1024, args.traffic_kernel)
        with open(traffic_file(args.traffic_kernel), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec, indent=1))
        return

    import numpy as np
    import torch

    import scaled_gemm_amd as sg
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sg.lib()
    stream = torch.cuda.current_stream()

    if args.judged_only:
        print(json.dumps(judged_shapes(stream, args.judged_only)), flush=True)
        return

    if args.workload == "70b_sweep":
        shape, x_bits, w_bits = workloads.make("70b_sweep", T=args.T or 8192,
                                               layer=args.layer or "gate_up")
    else:
        shape, x_bits, w_bits = workloads.make(args.workload, T=args.T)
    T, Ci, Co = shape.T, shape.Ci, shape.Co
    x0 = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    w0 = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)

    # Input copies at distinct addresses: step k works on activation copy
    # k mod nx and weight copy k mod nw, each count sized so that more than
    # 768 MiB of other copies pass between two uses of one (so every stage
    # reads inputs from HBM, not from the memory-side cache).  Outputs are
    # written, not read, and are shared.
    nx = n_sets(2 * T * Ci)
    nw = n_sets(Co * round_k(Ci))
    n = max(nx, nw)
    xs = [x0] + [x0.clone() for _ in range(nx - 1)]
    wts = [w0] + [w0.clone() for _ in range(nw - 1)]
    qxs = [torch.empty((T, Ci), dtype=torch.uint8, device=dev) for _ in range(nx)]
    dxs = [torch.empty((T,), dtype=torch.float32, device=dev) for _ in range(nx)]
    pws = [sg.PackedWeight(torch.empty((sg.packed_bytes(Ci, Co),), dtype=torch.uint8, device=dev),
                           torch.empty((Co,), dtype=torch.float32, device=dev), Ci, Co)
           for _ in range(nw)]
    out = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
    out2 = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((T, Co), dtype=torch.float32, device=dev)

    stages = ["quant_weight", "quant_act", "gemm_fused", "gemm_unfused"]
    run = set(args.only.split(",")) if args.only else set(stages)
    unknown = run - set(stages)
    if unknown:
        raise SystemExit(f"unknown stages {sorted(unknown)}")

    def step(k, ev=None):
        a, b = k % nx, k % nw

        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        if "quant_weight" in run:
            sg.quant_weight(wts[b], out=pws[b])
        mark(1)
        if "quant_act" in run:
            sg.quant_act(xs[a], qx=qxs[a], dx=dxs[a])
        mark(2)
        if "gemm_fused" in run:
            sg.gemm(qxs[a], dxs[a], pws[b], out=out)
        mark(3)
        if "gemm_unfused" in run:
            sg.gemm_unfused(qxs[a], dxs[a], pws[b], out=out2, workspace=ws)
        mark(4)

    # inputs of the GEMMs exist even when their producers are not timed
    for b in range(nw):
        sg.quant_weight(wts[b], out=pws[b])
    for a in range(nx):
        sg.quant_act(xs[a], qx=qxs[a], dx=dxs[a])
    if args.copy_calibration_mb:
        nb = args.copy_calibration_mb << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k, events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    per_stage = {s: [] for s in stages}
    for ev in events:
        for i, s in enumerate(stages):
            per_stage[s].append(ev[i].elapsed_time(ev[i + 1]))
    avg = {s: float(np.mean(v)) for s, v in per_stage.items()}
    med = {s: float(np.median(v)) for s, v in per_stage.items()}

    # The activation quantizer as a stream: back-to-back launches between one
    # event pair, rotating over the input copies (the per-launch pairs inside
    # the step also span each launch's own gap).
    act_ms = act_ms_eager = float("nan")
    act_reps = max(20, 2 * nx)
    if "quant_act" in run:
        def act(i):
            sg.quant_act(xs[i % nx], qx=qxs[i % nx], dx=dxs[i % nx])
        act_ms_eager = sorted(batch_ms(act, act_reps, stream) for _ in range(5))[2]
        act_ms = graph_ms(act, act_reps, stream)

    # Comparison forms on the same inputs, in interleaved rounds: each round
    # runs every form once, on the next input copy, each between its own
    # event pair, so that all forms see the same clock; ratios are the median
    # of the per-round ratios.
    cmp = None
    copy_gbs = cast_gbs = float("nan")
    if not args.only:
        pwts = [sg.quant_weight_static(wts[b], sg.tensor_scale(wts[b])) for b in range(nw)]
        sxs = [sg.tensor_scale(xs[a]) for a in range(nx)]
        qx_t = torch.empty_like(qxs[0])
        sx_t = torch.empty((1,), dtype=torch.float32, device=dev)
        ws16 = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
        forms = {
            "gemm_fused": lambda r: sg.gemm(qxs[r % nx], dxs[r % nx], pws[r % nw], out=out),
            "gemm_unfused": lambda r: sg.gemm_unfused(qxs[r % nx], dxs[r % nx], pws[r % nw],
                                                      out=out2, workspace=ws),
            "gemm_unfused_bf16": lambda r: sg.gemm_unfused_bf16(qxs[r % nx], dxs[r % nx],
                                                                pws[r % nw], out=out2,
                                                                workspace=ws16),
            "gemm_tensor": lambda r: sg.gemm_tensor(qxs[r % nx], sxs[r % nx], pwts[r % nw],
                                                    out=out2),
            "quant_act": lambda r: sg.quant_act(xs[r % nx], qx=qxs[r % nx], dx=dxs[r % nx]),
            "act_per_tensor": lambda r: (sg.tensor_scale(xs[r % nx], d=sx_t),
                                         sg.quant_act_static(xs[r % nx], sx_t, qx=qx_t)),
        }
        for r in range(3):
            for fn in forms.values():
                fn(r)
        torch.cuda.synchronize()
        rounds = max(args.steps, 2 * n)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(forms))]
               for _ in range(rounds)]
        for r in range(rounds):
            for i, fn in enumerate(forms.values()):
                evs[r][2 * i].record(stream)
                fn(r)
                evs[r][2 * i + 1].record(stream)
        torch.cuda.synchronize()
        t = {k: np.array([e[2 * i].elapsed_time(e[2 * i + 1]) for e in evs])
             for i, k in enumerate(forms)}

        def ratio(a, b):
            return round(float(np.median(t[a] / t[b])), 4)

        cmp = {
            "timing": (f"{rounds} interleaved rounds, every form once per round on the next "
                       f"input copies ({nx} of X, {nw} of W), each between its own HIP event "
                       "pair; medians"),
            "ms_median": {k: round(float(np.median(v)), 4) for k, v in t.items()},
            "fused_gemm_tflops": round(2.0 * T * Ci * Co / np.median(t["gemm_fused"]) / 1e9, 1),
            "two_step_fp32_over_fused": ratio("gemm_unfused", "gemm_fused"),
            "two_step_bf16_over_fused": ratio("gemm_unfused_bf16", "gemm_fused"),
            "ptpc_over_per_tensor_gemm": ratio("gemm_fused", "gemm_tensor"),
            "ptpc_over_per_tensor_act_quant": ratio("quant_act", "act_per_tensor"),
        }
        del pwts, sxs, qx_t, ws16

        # HBM references: a plain device copy (512 MiB read + 512 MiB written
        # per launch, larger than the cache on its own) and torch's unscaled
        # bf16 -> float8 cast of the same X copies (quant_act's traffic).
        cp_src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        cp_dst = torch.empty_like(cp_src)
        cp_dst.copy_(cp_src)
        copy_gbs = 2.0 * cp_src.numel() / (batch_ms(lambda i: cp_dst.copy_(cp_src), 5, stream)
                                           * 1e-3) / 1e9
        del cp_src, cp_dst
        cast_dst = torch.empty((T, Ci), dtype=torch.float8_e4m3fn, device=dev)
        cast_dst.copy_(xs[0])
        cast_gbs = 3.0 * T * Ci / (batch_ms(lambda i: cast_dst.copy_(xs[i % nx]),
                                            max(10, 2 * nx), stream) * 1e-3) / 1e9
        del cast_dst

    judged = None
    if not args.only and not args.no_judged:
        del xs, wts, qxs, dxs, pws, out, out2, ws
        torch.cuda.empty_cache()
        try:
            judged = judged_shapes(stream)
        except Exception as e:      # the step's own line is still printed
            print(f"judged_shapes failed: {e!r}", file=sys.stderr, flush=True)
            judged = {"error": repr(e)}

    gemm_flops = 2.0 * T * Ci * Co
    w_bytes = 3.0 * Ci * Co + 4.0 * Co
    ms_per_step = elapsed * 1e3 / args.steps
    n_gemms = ("gemm_fused" in run) + ("gemm_unfused" in run)
    value = n_gemms * gemm_flops / (ms_per_step * 1e-3) / 1e12

    def rate(work, stage, scale):
        return work / (avg[stage] * 1e-3) / scale if stage in run else float("nan")

    fused_tflops = rate(gemm_flops, "gemm_fused", 1e12)
    unfused_tflops = rate(gemm_flops, "gemm_unfused", 1e12)
    act_gbs = act_bytes(T, Ci) / (act_ms * 1e-3) / 1e9 if "quant_act" in run else float("nan")
    w_gbs = rate(w_bytes, "quant_weight", 1e9)

    result = {
        "metric": "ptpc_gemm TFLOP/s (% FP8 MFMA peak); quant_act GB/s (% HBM) on 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded, Llama-3.1-70B/8B-shaped linear layers with outlier channels)",
        "config": {
            "workload": shape.name, "T": T, "Ci": Ci, "Co": Co,
            "x": f"bf16 [{T}x{Ci}]", "w": f"bf16 [{Ci}x{Co}]", "out": f"bf16 [{T}x{Co}]",
            "step": " + ".join(s for s in stages if s in run),
            "value_work": f"{n_gemms} GEMMs x 2*T*Ci*Co flops per step",
            "input_copies": {"x": nx, "w": nw},
            "rotation": (f"step k uses copy k mod {nx} of X (and its codes) and copy k mod {nw} "
                         "of W (and its packed form), at distinct addresses: more than 768 MiB "
                         "of other copies pass between two uses of one, three times the 256 MB "
                         "memory-side cache"),
        },
        "roofline": {
            "kernel": "ptpc_gemm (fused): " + str(sg.gemm_kernel(T, Ci, Co)),
            "bound": "mfma",
            "achieved": round(fused_tflops, 1),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fused_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": measured_traffic(shape.name, "gemm_fused"),
            "algorithmic_min_bytes": gemm_min_bytes(T, Ci, Co),
            "avg_launch_ms": round(avg["gemm_fused"], 4),
        },
        "quant_act": {
            "kernel": sg.quant_act_kernel(T, Ci),
            "bound": "hbm", "achieved": round(act_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(act_gbs / PEAK_HBM_GBS, 4), "avg_launch_ms": round(act_ms, 4),
            "timing": (f"{act_reps} launches rotating over {nx} copies of X, captured in a HIP "
                       "graph, median of 5 replays between one HIP event pair each"),
            "eager_batch_ms": round(act_ms_eager, 4),
            "in_step_avg_launch_ms": round(avg["quant_act"], 4),
            "bytes_per_launch": act_bytes(T, Ci),
            "traffic": measured_traffic(shape.name, "quant_act"),
            "device_copy_gbs": round(copy_gbs, 1),
            "torch_cast_gbs": round(cast_gbs, 1),
            "frac_of_torch_cast": round(act_gbs / cast_gbs, 4),
        },
        "stages_ms_avg": {k: round(v, 4) for k, v in avg.items()},
        "stages_ms_median": {k: round(v, 4) for k, v in med.items()},
        "quant_weight_gbs": round(w_gbs, 1),
        "gemm_unfused_tflops": round(unfused_tflops, 1),
        "comparison": cmp,
        "judged_shapes": judged,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        try:
            result["cpu_baseline"] = cpu_baseline(x_bits, w_bits, args.cpu_seconds)
        except Exception as e:      # the step's own line is still printed
            print(f"cpu_baseline failed: {e!r}", file=sys.stderr, flush=True)
            result["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(no_nan(result)), flush=True)


if __name__ == "__main__":
    main()
