"""Benchmark of the PTPC-FP8 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 70b_down]

One step = every stage of the path over one batch of resident synthetic
input: per-channel weight quantization + prepack, per-token activation
quantization, the fused FP8 GEMM, and the two-step (unfused) GEMM.  Each
stage is bracketed by HIP events on the stream it runs on, so per-kernel
averages come from the timed region itself.

Prints one JSON line.  `value` is whole-step throughput: the FP8 contraction
work of the step (two GEMMs, 2*T*Ci*Co flops each) divided by the step time.
`roofline` is the fused GEMM against the dense FP8 MFMA peak; `quant_act`
carries the activation quantizer against HBM bandwidth; `cpu_baseline` is
the CPU oracle on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_fused_70b_down_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=30,
                   help="untimed steps first; the shader clock needs tens of ms to settle")
    p.add_argument("--workload", default="70b_down")
    p.add_argument("--layer", default=None, help="70b_sweep layer")
    p.add_argument("--T", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--only", default=None,
                   help="comma list of stages to run (profiling); default all")
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
                        "--only gemm_fused --copy-calibration-mb run into the traffic record "
                        "and exit (no GPU needed)")
    return p.parse_args()


def gemm_source_hash():
    """Hash of the GEMM's code: gemm.hip and the device header it includes,
    with comments and blank space removed, so that the traffic record stays
    valid across comment edits and is dropped on any code change."""
    import re
    text = ""
    for name in ("gemm.hip", "device_common.h"):
        with open(os.path.join(ROOT, "scaled_gemm_amd", "csrc", name)) as f:
            text += f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per fused-GEMM launch from rocprofv3 FETCH_SIZE/WRITE_SIZE,
    only if the counters were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return t.get("bytes_per_launch")


def traffic_record(fetch_csv, write_csv, workload, copy_mb):
    """HBM bytes per fused-GEMM launch: the FETCH_SIZE / WRITE_SIZE counters
    (KiB per dispatch) of the GEMM, each scaled by the ratio of the known
    bytes of a plain device copy to what the same counter reads for it."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                key = ("gemm" if "gemm16_kernel<256, 256, 2, 2, true>" in name
                       else "copy" if "copyBuffer" in name else None)
                if key:
                    vals.setdefault(key, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in vals.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = float(copy_mb) * (1 << 20)
    f_factor = copy_bytes / (f["copy"] * 1024.0)
    w_factor = copy_bytes / (w["copy"] * 1024.0)
    fetch = f["gemm"] * 1024.0 * f_factor
    write = w["gemm"] * 1024.0 * w_factor
    return {"workload": workload, "gemm_source_sha256_16": gemm_source_hash(),
            "kernel": "gemm16_kernel<256, 256, 2, 2, true> (fused, this workload's tiles)",
            "fetch_kib_raw": f["gemm"], "write_kib_raw": w["gemm"],
            "copy_bytes": copy_bytes, "copy_fetch_kib_raw": f["copy"],
            "copy_write_kib_raw": w["copy"], "fetch_factor": f_factor,
            "write_factor": w_factor, "fetch_bytes": fetch, "write_bytes": write,
            "bytes_per_launch": fetch + write,
            "commands": [
                "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv "
                "-d $REPO/gpurun_out/prof_fetch -o p -- python -u $REPO/bench.py --steps 3 "
                f"--warmup 1 --no-cpu-baseline --only gemm_fused --copy-calibration-mb {copy_mb}",
                "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv "
                "-d $REPO/gpurun_out/prof_write -o p -- python -u $REPO/bench.py --steps 3 "
                f"--warmup 1 --no-cpu-baseline --only gemm_fused --copy-calibration-mb {copy_mb}",
                "python bench.py --traffic-from $REPO/gpurun_out/prof_fetch/p_counter_collection.csv "
                f"$REPO/gpurun_out/prof_write/p_counter_collection.csv --copy-calibration-mb {copy_mb}"],
            "note": ("Counters in KiB per dispatch, averaged over the fused-GEMM launches; each "
                     "scaled by known copy bytes / counter reading for a device copy of "
                     f"{copy_mb} MiB (torch copy_) in the same run. On MI355X FETCH_SIZE reads "
                     "about half of the copy's bytes, WRITE_SIZE all of them.")}


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
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": min(nthr, R),
            "kind": "oracle",
            "sample": (f"first {R} token rows of the workload with its whole weight: "
                       f"quant_weight [{Ci}x{Co}] + quant_act [{R}x{Ci}] + exact GEMM "
                       f"[{R}x{Ci}]x[{Ci}x{Co}] + scales; {total:.1f} s wall "
                       f"(weight quantization {t_w:.1f} s); {nthr} OpenMP threads")}


def no_nan(v):
    """JSON has no NaN: stages that did not run (--only) report null."""
    if isinstance(v, float) and v != v:
        return None
    if isinstance(v, dict):
        return {k: no_nan(x) for k, x in v.items()}
    if isinstance(v, list):
        return [no_nan(x) for x in v]
    return v


def act_bytes_ref(T, Ci):
    """Bytes a bf16 -> 1-byte cast of a [T x Ci] matrix moves."""
    return 3.0 * T * Ci


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
    """Per-shape kernel rates over every workload shape (after a warm-up, three
    interleaved rounds over the stages, each round one HIP event pair on the
    launch stream around `steps` back-to-back launches; the best round per
    stage)."""
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
        x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        w = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        del x_bits, w_bits
        pw = sg.quant_weight(w)
        qx, dx = sg.quant_act(x)
        out = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
        out2 = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((T, Co), dtype=torch.float32, device=dev)
        ws16 = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
        gws = torch.empty((max(1, sg.gemm_workspace_bytes(T, Ci, Co)),), dtype=torch.uint8,
                          device=dev)
        sx_t = sg.tensor_scale(x)
        pw_t = sg.quant_weight_static(w, sg.tensor_scale(w))
        calls = {
            "quant_weight": lambda: sg.quant_weight(w, out=pw),
            "quant_act": lambda: sg.quant_act(x, qx=qx, dx=dx),
            "gemm_fused": lambda: sg.gemm(qx, dx, pw, out=out),
            "gemm_unfused": lambda: sg.gemm_unfused(qx, dx, pw, out=out2, workspace=ws),
            "gemm_unfused_bf16": lambda: sg.gemm_unfused_bf16(qx, dx, pw, out=out2,
                                                              workspace=ws16),
            "gemm_tensor": lambda: sg.gemm_tensor(qx, sx_t, pw_t, out=out2),
            "gemm_ws": lambda: sg.gemm_ws(qx, dx, pw, out=out2, workspace=gws),
        }
        # Three interleaved rounds over the stages, each stage's best round
        # reported: a stage timed in one block right after another reads the
        # clock's settling (short launches by up to 20%).
        for fn in calls.values():
            for _ in range(max(3, args.warmup)):
                fn()
        rounds = {k: [] for k in calls}
        for _ in range(3):
            for k, fn in calls.items():
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                ev[0].record(stream)
                for i in range(args.steps):
                    fn()
                ev[1].record(stream)
                torch.cuda.synchronize()
                rounds[k].append(ev[0].elapsed_time(ev[1]) / args.steps)
        ms = {k: min(v) for k, v in rounds.items()}
        flops = 2.0 * T * Ci * Co
        act_b = 3.0 * T * Ci + 4.0 * T
        print(json.dumps({
            "workload": shape.name, "T": T, "Ci": Ci, "Co": Co,
            "ms": {k: round(v, 4) for k, v in ms.items()},
            "gemm_fused_tflops": round(flops / ms["gemm_fused"] / 1e9, 1),
            "gemm_fused_frac_fp8_peak": round(flops / ms["gemm_fused"] / 1e9 / PEAK_FP8_TFLOPS, 4),
            "gemm_fused_gbs_min_bytes": round((T * Ci + Ci * Co + 2.0 * T * Co + 4.0 * (T + Co))
                                              / ms["gemm_fused"] / 1e6, 1),
            "gemm_unfused_tflops": round(flops / ms["gemm_unfused"] / 1e9, 1),
            "fused_over_unfused": round(ms["gemm_unfused"] / ms["gemm_fused"], 3),
            "fused_over_unfused_bf16": round(ms["gemm_unfused_bf16"] / ms["gemm_fused"], 3),
            "ptpc_over_per_tensor_gemm": round(ms["gemm_fused"] / ms["gemm_tensor"], 3),
            "gemm_ws_speedup": round(ms["gemm_fused"] / ms["gemm_ws"], 3),
            "gemm_ws_gbs_min_bytes": round((T * Ci + Ci * Co + 2.0 * T * Co + 4.0 * (T + Co))
                                           / ms["gemm_ws"] / 1e6, 1),
            "quant_act_gbs": round(act_b / ms["quant_act"] / 1e6, 1),
            "quant_act_frac_hbm": round(act_b / ms["quant_act"] / 1e6 / PEAK_HBM_GBS, 4),
            "quant_weight_gbs": round((3.0 * Ci * Co + 4.0 * Co) / ms["quant_weight"] / 1e6, 1),
        }), flush=True)
        del x, w, pw, qx, dx, out, out2, ws, ws16, sx_t, pw_t, gws
        torch.cuda.empty_cache()


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
    if args.traffic_from:
        rec = traffic_record(args.traffic_from[0], args.traffic_from[1], args.workload,
                             args.copy_calibration_mb or 1024)
        with open(TRAFFIC_FILE, "w") as f:
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

    if args.workload == "70b_sweep":
        shape, x_bits, w_bits = workloads.make("70b_sweep", T=args.T or 8192,
                                               layer=args.layer or "gate_up")
    else:
        shape, x_bits, w_bits = workloads.make(args.workload, T=args.T)
    T, Ci, Co = shape.T, shape.Ci, shape.Co
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)

    # outputs allocated once, outside the timed region
    qx = torch.empty((T, Ci), dtype=torch.uint8, device=dev)
    dx = torch.empty((T,), dtype=torch.float32, device=dev)
    pw = sg.PackedWeight(torch.empty((sg.packed_bytes(Ci, Co),), dtype=torch.uint8, device=dev),
                         torch.empty((Co,), dtype=torch.float32, device=dev), Ci, Co)
    out = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
    out2 = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((T, Co), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    stages = ["quant_weight", "quant_act", "gemm_fused", "gemm_unfused"]
    run = set(args.only.split(",")) if args.only else set(stages)
    unknown = run - set(stages)
    if unknown:
        raise SystemExit(f"unknown stages {sorted(unknown)}")

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        if "quant_weight" in run:
            sg.quant_weight(w, out=pw)
        mark(1)
        if "quant_act" in run:
            sg.quant_act(x, qx=qx, dx=dx)
        mark(2)
        if "gemm_fused" in run:
            sg.gemm(qx, dx, pw, out=out)
        mark(3)
        if "gemm_unfused" in run:
            sg.gemm_unfused(qx, dx, pw, out=out2, workspace=ws)
        mark(4)

    # inputs of the GEMMs exist even when their producers are not timed
    sg.quant_weight(w, out=pw)
    sg.quant_act(x, qx=qx, dx=dx)
    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # The per-tensor comparator on the same inputs (not part of the step):
    # dynamic per-tensor activation scale + static cast, and the GEMM with
    # scalar scales; the weight is quantized per tensor once, outside.
    pt = None
    if not args.only:
        sw_t = sg.tensor_scale(w)
        pw_t = sg.quant_weight_static(w, sw_t)
        sx_t = torch.empty((1,), dtype=torch.float32, device=dev)
        qx_t = torch.empty_like(qx)
        out_t = torch.empty_like(out)
        ws16 = torch.empty((T, Co), dtype=torch.bfloat16, device=dev)
        pt_calls = [("tensor_scale", lambda: sg.tensor_scale(x, d=sx_t)),
                    ("quant_act_static", lambda: sg.quant_act_static(x, sx_t, qx=qx_t)),
                    ("gemm_tensor", lambda: sg.gemm_tensor(qx_t, sx_t, pw_t, out=out_t)),
                    ("gemm_unfused_bf16", lambda: sg.gemm_unfused_bf16(qx, dx, pw, out=out_t,
                                                                       workspace=ws16))]
        for _ in range(3):
            for _, fn in pt_calls:
                fn()
        pt_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(pt_calls) + 1)]
                 for _ in range(args.steps)]
        for k in range(args.steps):
            for i, (_, fn) in enumerate(pt_calls):
                pt_ev[k][i].record(stream)
                fn()
            pt_ev[k][len(pt_calls)].record(stream)
        torch.cuda.synchronize()
        pt = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in pt_ev]))
              for i, (name, _) in enumerate(pt_calls)}
        del sw_t, pw_t, sx_t, qx_t, out_t, ws16

    # References for the activation quantizer's HBM rate next to the 8 TB/s
    # peak: a plain device copy (torch copy_, 512 MiB read + 512 MiB written)
    # and torch's own unscaled bf16 -> float8_e4m3fn cast of the same X, which
    # has exactly quant_act's traffic (2 bytes read, 1 written per element).
    def timed(fn, n=5):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(n):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e-3 / n
    copy_gbs = cast_gbs = float("nan")
    # quant_act timed the same way as those references: back-to-back
    # launches between one event pair (the per-launch pairs inside the step
    # also span each launch's own gap, several us against a 58 us kernel).
    act_batch_ms = float("nan")
    if "quant_act" in run:
        act_batch_ms = timed(lambda: sg.quant_act(x, qx=qx, dx=dx), n=20) * 1e3
    if not args.only:
        cp_src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        cp_dst = torch.empty_like(cp_src)
        copy_gbs = 2.0 * cp_src.numel() / timed(lambda: cp_dst.copy_(cp_src)) / 1e9
        del cp_src, cp_dst
        cast_dst = torch.empty((T, Ci), dtype=torch.float8_e4m3fn, device=dev)
        cast_gbs = act_bytes_ref(T, Ci) / timed(lambda: cast_dst.copy_(x)) / 1e9
        del cast_dst

    per_stage = {s: [] for s in stages}
    for ev in events:
        for i, s in enumerate(stages):
            per_stage[s].append(ev[i].elapsed_time(ev[i + 1]))
    avg = {s: float(np.mean(v)) for s, v in per_stage.items()}
    med = {s: float(np.median(v)) for s, v in per_stage.items()}

    gemm_flops = 2.0 * T * Ci * Co
    act_bytes = 3.0 * T * Ci + 4.0 * T
    w_bytes = 3.0 * Ci * Co + 4.0 * Co
    fused_min_bytes = T * Ci + Ci * Co + 2.0 * T * Co + 4.0 * (T + Co)
    ms_per_step = elapsed * 1e3 / args.steps
    n_gemms = ("gemm_fused" in run) + ("gemm_unfused" in run)
    value = n_gemms * gemm_flops / (ms_per_step * 1e-3) / 1e12

    def rate(work, stage, scale):
        return work / (avg[stage] * 1e-3) / scale if stage in run else float("nan")

    fused_tflops = rate(gemm_flops, "gemm_fused", 1e12)
    unfused_tflops = rate(gemm_flops, "gemm_unfused", 1e12)
    act_gbs = act_bytes / (act_batch_ms * 1e-3) / 1e9 if "quant_act" in run else float("nan")
    w_gbs = rate(w_bytes, "quant_weight", 1e9)
    traffic = measured_traffic(shape.name)

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
        },
        "roofline": {
            "kernel": "ptpc_gemm (fused)",
            "bound": "mfma",
            "achieved": round(fused_tflops, 1),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fused_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_min_bytes": fused_min_bytes,
            "avg_launch_ms": round(avg["gemm_fused"], 4),
        },
        "quant_act": {
            "bound": "hbm", "achieved": round(act_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(act_gbs / PEAK_HBM_GBS, 4), "avg_launch_ms": round(act_batch_ms, 4),
            "timing": "20 back-to-back launches between one HIP event pair on the launch stream",
            "in_step_avg_launch_ms": round(avg["quant_act"], 4),
            "bytes_per_launch": act_bytes,
            "device_copy_gbs": round(copy_gbs, 1),
            "torch_cast_gbs": round(cast_gbs, 1),
            "frac_of_torch_cast": round(act_gbs / cast_gbs, 4),
        },
        "stages_ms_avg": {k: round(v, 4) for k, v in avg.items()},
        "stages_ms_median": {k: round(v, 4) for k, v in med.items()},
        "quant_weight_gbs": round(w_gbs, 1),
        "gemm_unfused_tflops": round(unfused_tflops, 1),
        "fused_over_unfused": (round(avg["gemm_unfused"] / avg["gemm_fused"], 3)
                               if {"gemm_fused", "gemm_unfused"} <= run else None),
        "cpu_baseline": None,
    }
    if pt is not None:
        result["two_step_bf16"] = {
            "what": "two-step form with a bf16 intermediate (GEMM -> bf16, then scale)",
            "ms_avg": round(pt.pop("gemm_unfused_bf16"), 4),
        }
        result["two_step_bf16"]["fused_speedup"] = round(
            result["two_step_bf16"]["ms_avg"] / avg["gemm_fused"], 4)
        result["per_tensor"] = {
            "what": "per-tensor FP8 comparator on the same inputs: tensor_scale(X) + "
                    "quant_act_static + gemm_tensor (weight quantized per tensor once)",
            "ms_avg": {k: round(v, 4) for k, v in pt.items()},
            "gemm_tensor_tflops": round(gemm_flops / (pt["gemm_tensor"] * 1e-3) / 1e12, 1),
            "ptpc_over_per_tensor_gemm_time": round(avg["gemm_fused"] / pt["gemm_tensor"], 4),
            "ptpc_over_per_tensor_act_quant_time": round(
                avg["quant_act"] / (pt["tensor_scale"] + pt["quant_act_static"]), 4),
        }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x_bits, w_bits, args.cpu_seconds)
    print(json.dumps(no_nan(result)), flush=True)


if __name__ == "__main__":
    main()
