"""Benchmark of the NVFP4 W4A4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload serving] [--format nvfp4]

A step is one pass of the whole hot path (activation quantize -> block-scaled
GEMM -> alpha/bias/bf16 epilogue, i.e. one linear call) over every case of the
workload. The default workload, `serving`, spans M = 1..8192:
  * decode: Llama-3.1-8B qkv (K=4096, N=6144), gate_up (4096, 28672) and down
    (14336, 4096) at M in {1, 8, 32, 128}, with bias (12 calls);
  * prefill: the same shapes at M in {2048, 8192}, 1% outlier channels (6 calls);
  * hadamard: Qwen3-32B gate_up (5120, 51200) and down (25600, 5120) at M in
    {1, 256, 4096} with the block-diagonal Hadamard rotation, b in
    {16, 32, 64, 128} (24 calls).
Inputs are seeded synthetic tensors (the `synthetic` module); weights are
quantized and packed on the GPU before timing and rotated through enough
copies that every call reads its weight from HBM, not from the 256 MB
last-level cache. Each step is one HIP graph replay.

Prints one JSON line. `value` is whole-step TFLOP/s (2*M*N*K summed over the
step / step time). `per_case` gives every call's time with its GB/s and HBM
fraction (algorithmic bytes: 0.5625 B per weight element + 2 B per activation
and output element + bias) and its TFLOP/s against the dense float16 MFMA
peak (the exact NVFP4 path multiplies dequantized float16 operands) and the
FP4 peak. `roofline` describes the kernel carrying the most time per step,
timed alone with HIP events on its launch stream. `calibration` holds what a
plain streaming read and MFMA loops reach on this GPU. `cpu_baseline` times
the CPU oracle on a bounded sample of the same workload, on all host cores and
on one thread.

`--format mxfp4|mxfp8|fp8|fp8_block` runs one of the sibling layers (scaled
FP4/FP8 MFMA) instead; their natural workload is `siblings` (K=4096,
N=14336, M=1 and 4096). Algorithmic weight bytes per element: MXFP4 0.53125,
MXFP8 1.03125, per-tensor FP8 1, block FP8 1 + 4/128^2.
"""

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFLOPS = 10100.0
FP8_PEAK_TFLOPS = 5000.0
F16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 512 << 20

SINGLE_WORKLOADS = ("decode", "prefill", "hadamard", "tiny", "siblings", "transform")
COMPOSITE_WORKLOADS = {"serving": ("decode", "prefill", "hadamard")}
WORKLOAD_KEYS = tuple(COMPOSITE_WORKLOADS) + SINGLE_WORKLOADS
FORMAT_KEYS = ("nvfp4", "mxfp4", "mxfp8", "fp8", "fp8_block")
# algorithmic weight bytes per element: code + scale bytes per element
WEIGHT_BYTES = {"nvfp4": 0.5 + 1.0 / 16, "mxfp4": 0.5 + 1.0 / 32, "mxfp8": 1.0 + 1.0 / 32,
                "fp8": 1.0, "fp8_block": 1.0 + 4.0 / (128 * 128)}
# dense MFMA peak the format runs on (TFLOP/s): NVFP4 multiplies exactly
# dequantized float16 operands; the others run on the scaled FP4 / FP8 MFMA
MFMA_PEAK = {"nvfp4": F16_PEAK_TFLOPS, "mxfp4": FP4_PEAK_TFLOPS, "mxfp8": FP8_PEAK_TFLOPS,
             "fp8": FP8_PEAK_TFLOPS, "fp8_block": FP8_PEAK_TFLOPS}
FORMAT_DTYPE = {
    "nvfp4": "nvfp4 (e2m1 x e4m3/16) -> f16 MFMA, f32 accumulate, bf16 out",
    "mxfp4": "mxfp4 (e2m1 x e8m0/32) -> scaled fp4 MFMA, f32 accumulate, bf16 out",
    "mxfp8": "mxfp8 (e4m3 x e8m0/32) -> scaled fp8 MFMA, f32 accumulate, bf16 out",
    "fp8": "fp8 e4m3, per-tensor scales -> fp8 MFMA, f32 accumulate, bf16 out",
    "fp8_block": "fp8 e4m3, 1x128 / 128x128 f32 scales -> fp8 MFMA + f32 promotion, bf16 out",
}
WORKLOAD_NAMES = {
    "serving": "serving: Llama-3.1-8B qkv/gate_up/down decode M=1,8,32,128 (bias) + prefill "
               "M=2048,8192 (1% outlier channels) + Qwen3-32B gate_up/down M=1,256,4096 with "
               "block-diagonal Hadamard b=16,32,64,128 (M=1..8192, 42 calls)",
    "decode": "decode: Llama-3.1-8B qkv/gate_up/down at M=1,8,32,128, bias",
    "prefill": "prefill: Llama-3.1-8B qkv/gate_up/down at M=2048,8192, 1% outlier channels",
    "hadamard": "hadamard: Qwen3-32B gate_up/down at M=1,256,4096, block-diagonal Hadamard",
    "tiny": "tiny: M=16, K=256, N=512",
    "siblings": "siblings: K=4096, N=14336 at M=1,4096",
    "transform": "transform: Qwen3-32B gate_up/down at M=1,256,4096, general b x b transform "
                 "(random orthogonal bf16, b=16..128)",
}


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_SUMMARIES = [os.path.join(ROOT, "profiles", "serving_hbm_traffic.md")]


def source_digest():
    """sha256 over the sources of the NVFP4 GEMM translation unit (gemm_nvfp4.hip and
    the headers it includes: names and bytes, in this order)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "fp8_quantized_linear_amd", "csrc")
    for f in ("gemm_nvfp4.hip", "fql_device.h", "fql_gemm.h", "fql_internal.h", "fql_quant.h"):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from a committed counter summary.

    A summary records FETCH_SIZE + WRITE_SIZE per launch (scaled by the
    plain-copy calibration) with the digest of the kernel sources it was taken
    on; once the sources differ, the figure no longer describes the kernel and
    None is returned.
    """
    digest = None
    for path in TRAFFIC_SUMMARIES:
        try:
            text = open(path).read()
        except OSError:
            continue
        for line in text.splitlines():
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
                if rec.get("kernel") != kernel:
                    continue
                digest = digest or source_digest()
                if rec.get("source_sha256") == digest:
                    return rec["bytes_per_launch"]
    return None


def _alg_bytes(M, N, K, with_bias, fmt="nvfp4"):
    return (WEIGHT_BYTES[fmt] * N * K + 2.0 * M * K + 2.0 * M * N
            + (2.0 * N if with_bias else 0.0))


def _case_name(wl, name, M, hb):
    tag = "b" if wl == "transform" else "hb"
    return f"{wl}/{name}/M={M}" + (f"/{tag}={hb}" if hb else "")


def _cases(workload, hb_override=None, only=None):
    """(wl, M, name, K, N, hb, with_bias) of the workload's calls, optionally restricted
    to one block size and to the case names in `only` (e.g. {"prefill/gate_up/M=8192"})."""
    import synthetic

    out = []
    for wl in COMPOSITE_WORKLOADS.get(workload, (workload,)):
        for M, name, K, N, hb, with_bias in synthetic.cases(wl):
            if hb_override is not None and hb != hb_override:
                continue
            if only and _case_name(wl, name, M, hb) not in only:
                continue
            out.append((wl, M, name, K, N, hb, with_bias))
    if only and not out:
        raise SystemExit(f"no case of the {workload} workload is named in {sorted(only)}")
    return out


def _kernel_of(M, N, K, fmt="nvfp4", general=False, dynamic=False, hb=0):
    """The GEMM kernel of one linear call of this shape (the library's own plan; the
    transform and dynamic-scale paths plan as unaligned calls)."""
    import fp8_quantized_linear_amd as fql

    if fmt != "nvfp4":
        return fql.linear_sc_plan(fmt, M, N, K).split(" grid=")[0].split(" + ")[-1]
    plan = fql.linear_plan(M, N, K, aligned=not (general or dynamic), transform=general,
                           hadamard_block=hb)
    return plan.split(" grid=")[0].split(" + ")[-1]


def _has_quant_pass(M, N, K):
    import fp8_quantized_linear_amd as fql

    return " + " in fql.linear_plan(M, N, K, aligned=True)


def gpu_bench(workload, steps, warmup, hb, per_case_reps=11, fmt="nvfp4", dynamic=False, only=None):
    import torch

    import fp8_quantized_linear_amd as fql
    import synthetic

    tmats = {}

    def tmat(b):
        if b not in tmats:
            tmats[b] = torch.from_numpy(synthetic.transform_matrix(b).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return tmats[b]

    ok, why = fql.is_supported(0)
    if not ok:
        raise SystemExit(f"GPU path not supported here: {why}")
    dev = torch.device("cuda:0")
    cases = _cases(workload, hb, only)
    setups = []
    weights = {}
    xs = {}
    for (wl, M, name, K, N, hbk, with_bias) in cases:
        general = wl == "transform"  # the block size is a general transform's, not a rotation's
        key = (wl, name, K, N, hbk)
        if key not in weights:
            W = torch.from_numpy(synthetic.weight(N, K, config=wl)).to(dev)
            if fmt == "nvfp4" and general:
                w0 = fql.NVFP4Weight.from_float(W, input_global_scale=1.0, transform=tmat(hbk))
            elif fmt == "nvfp4":
                w0 = fql.NVFP4Weight.from_float(W, input_global_scale=1.0, hadamard_block=hbk)
            elif fmt == "fp8":
                w0 = fql.FP8Weight.from_float(W, input_scale=1.0)
            else:
                w0 = {"mxfp4": fql.MXFP4Weight, "mxfp8": fql.MXFP8Weight,
                      "fp8_block": fql.FP8BlockWeight}[fmt].from_float(W)
            del W
            nbytes = w0.packed.numel()
            ncopies = max(1, -(-ROTATE_BYTES // nbytes))
            copies = [w0.packed] + [w0.packed.clone() for _ in range(ncopies - 1)]
            weights[key] = (w0, copies)
        w0, copies = weights[key]
        xkey = (wl, M, K)
        if xkey not in xs:
            xb = synthetic.activations(synthetic.WORKLOADS[wl]["x"], M, K, config=wl)
            xs[xkey] = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        x = xs[xkey]
        if fmt == "nvfp4":
            T = tmat(hbk) if general else None
            if general:  # calibration on the transformed activation (the library's amax kernel)
                gx = fql.global_scale_from_amax(fql.quant_nvfp4_dynamic(x, T=T)[2][0].item())
            else:
                gx = fql.global_scale_from_amax(fql.amax(x, hbk).item())
            objs = [fql.NVFP4Weight(p, N, K, gx, w0.weight_global_scale, 0 if general else hbk,
                                    transform=T, dynamic_input_scale=dynamic) for p in copies]
        elif fmt == "fp8":
            sx = fql.fp8_scale_from_amax(fql.amax(x).item())
            objs = [fql.FP8Weight(p, N, K, w0.weight_scale, sx) for p in copies]
        else:
            objs = [type(w0)(p, N, K) for p in copies]
        bias = None
        if with_bias:
            bias = torch.from_numpy(synthetic.bias(N, config=wl).view(np.int16)).view(
                torch.bfloat16).to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsb = (fql.linear_workspace_bytes(M, N, K) if fmt == "nvfp4"
               else fql.linear_sc_workspace_bytes(fmt, M, N, K))
        ws = fql.new_workspace(wsb, dev)
        split = (fmt == "nvfp4" and not general and not dynamic and _has_quant_pass(M, N, K))
        setups.append(dict(M=M, N=N, K=K, name=_case_name(wl, name, M, hbk), x=x, objs=objs,
                           bias=bias, y=y, ws=ws, flops=2.0 * M * N * K,
                           bytes=_alg_bytes(M, N, K, with_bias, fmt), split=split,
                           kernel=_kernel_of(M, N, K, fmt, general=general, dynamic=dynamic,
                                             hb=0 if general else (hbk or 0))))
    torch.cuda.synchronize()
    n = len(setups)

    linear = {"nvfp4": fql.linear_nvfp4, "mxfp4": fql.linear_mxfp4, "mxfp8": fql.linear_mxfp8,
              "fp8": fql.linear_fp8, "fp8_block": fql.linear_fp8_block}[fmt]

    def call(s, copy_index):
        w = s["objs"][copy_index % len(s["objs"])]
        linear(s["x"], w, bias=s["bias"], out=s["y"], workspace=s["ws"])

    # One HIP graph per step position: call j of step i uses weight copy i*n + j, so
    # consecutive calls on one weight shape never reuse a copy (cold last-level cache).
    period = max(len(s["objs"]) for s in setups)
    stream = torch.cuda.Stream(device=dev)
    graphs = []
    with torch.cuda.stream(stream):
        for j, s in enumerate(setups):  # eager warm-up of every call shape
            call(s, 0)
        stream.synchronize()
        for i in range(period):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for j, s in enumerate(setups):
                    call(s, i * n + j)
            graphs.append(g)
    torch.cuda.synchronize()

    # timed region: `steps` whole steps, graph replays on one stream
    with torch.cuda.stream(stream):
        for i in range(warmup):
            graphs[i % period].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            graphs[(warmup + i) % period].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = e0.elapsed_time(e1) / steps
    wall_ms_per_step = (t1 - t0) * 1e3 / steps
    del graphs

    # per-call duration of each case: a graph of R back-to-back calls of that case
    # (rotating weight copies), each replay timed with HIP events on the replay
    # stream; the median replay gives the per-call time, p10 and p90 its spread
    with torch.cuda.stream(stream):
        for s in setups:
            R = max(8, len(s["objs"]))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for r in range(R):
                    call(s, r)
            g.replay()
            stream.synchronize()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(per_case_reps + 1)]
            evs[0].record(stream)
            for i in range(per_case_reps):
                g.replay()
                evs[i + 1].record(stream)
            evs[-1].synchronize()
            per = sorted(evs[i].elapsed_time(evs[i + 1]) / R for i in range(per_case_reps))
            s["call_ms"] = per[len(per) // 2]
            s["call_ms_p10"] = per[int(0.1 * (len(per) - 1))]
            s["call_ms_p90"] = per[int(round(0.9 * (len(per) - 1)))]
            del g
    # GEMM kernel alone: calls with a quantizer pass run as their two halves, and
    # HIP events on the launch stream bracket each GEMM launch (rotating copies)
    with torch.cuda.stream(stream):
        for s in setups:
            if not s["split"]:
                s["kernel_ms"] = s["call_ms"]
                continue
            R = max(8, len(s["objs"]))
            evs = []
            for r in range(R + 1):
                w = s["objs"][r % len(s["objs"])]
                fql.linear_nvfp4_quantize(s["x"], w, s["ws"])
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fql.linear_nvfp4_gemm(s["M"], w, s["ws"], w.alpha, bias=s["bias"], out=s["y"])
                b.record(stream)
                if r > 0:  # the first round warms up
                    evs.append((a, b))
            stream.synchronize()
            s["kernel_ms"] = statistics.mean(a.elapsed_time(b) for a, b in evs)

    per_case = []
    for s in setups:
        ms = s["call_ms"]
        tf = s["flops"] / (ms * 1e-3) / 1e12
        gbs = s["bytes"] / (ms * 1e-3) / 1e9
        d = dict(case=s["name"], kernel=s["kernel"], us=round(ms * 1e3, 2),
                 us_p10=round(s["call_ms_p10"] * 1e3, 2), us_p90=round(s["call_ms_p90"] * 1e3, 2),
                 gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 3), tflops=round(tf, 1),
                 mfma_frac=round(tf / MFMA_PEAK[fmt], 3))
        if fmt == "nvfp4":
            d["fp4_frac"] = round(tf / FP4_PEAK_TFLOPS, 4)
        if s["split"]:
            d["gemm_us"] = round(s["kernel_ms"] * 1e3, 2)
        per_case.append(d)
    # dominant kernel: the GEMM kernel carrying the most time per step
    by_kernel = {}
    for s in setups:
        k = by_kernel.setdefault(s["kernel"], dict(ms=0.0, bytes=0.0, flops=0.0, launches=0,
                                                   cases=[]))
        k["ms"] += s["kernel_ms"]
        k["bytes"] += s["bytes"]
        k["flops"] += s["flops"]
        k["launches"] += 1
        k["cases"].append(s["name"])
    dom_name, dom = max(by_kernel.items(), key=lambda kv: kv[1]["ms"])
    flops = sum(s["flops"] for s in setups)
    alg_bytes = sum(s["bytes"] for s in setups)
    return dict(ms_per_step=ms_per_step, wall_ms_per_step=wall_ms_per_step, flops=flops,
                alg_bytes=alg_bytes, per_case=per_case, dominant=(dom_name, dom))


# ---------------------------------------------------------------------------
# calibration: what a plain streaming read and MFMA loops reach on this GPU
# ---------------------------------------------------------------------------

def calibration(stream_sizes_mb=(14.2, 33.1, 66.1, 147.5, 512.0), mfma_reps=3):
    """Streaming-read GB/s per buffer size (cold: rotated over >= 512 MB, graph of
    back-to-back reads, HIP events), MFMA-loop TFLOP/s (f16 32x32x16 and the
    scaled FP8 / FP4 16x16x128, one and two waves per SIMD) and the vendor
    library's float16 GEMM on the large layer shapes."""
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "fp8_quantized_linear_amd", "libfql_calib.so"))
    lib.fql_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.fql_calib_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    sst = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    out = {"stream_read_gbs": {}, "mfma_tflops": {}}
    pool = torch.ones(1024 << 20, dtype=torch.uint8, device=dev)
    for mb in stream_sizes_mb:
        nb = int(mb * 1e6) // 4096 * 4096
        bufs = max(2, (1024 << 20) // nb)
        grid = int(min(1 << 16, max(1, nb // (16 * 1024))))
        R = max(8, bufs)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for r in range(R):
                    p = pool.data_ptr() + (r % bufs) * nb
                    rc = lib.fql_calib_stream_read(ctypes.c_void_p(p), nb, grid,
                                                   ctypes.c_void_p(sink.data_ptr()),
                                                   ctypes.c_void_p(stream.cuda_stream))
                    if rc != 0:
                        raise RuntimeError(f"stream read calibration failed ({rc})")
            g.replay()
            stream.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(3):
                g.replay()
            b.record(stream)
            b.synchronize()
        ms = a.elapsed_time(b) / (3 * R)
        out["stream_read_gbs"][f"{mb:g}MB"] = round(nb / (ms * 1e-3) / 1e9, 1)
        del g
    del pool
    iters = 8000  # about a millisecond per launch, like the large GEMMs
    for kind, name, flop in ((0, "f16_32x32x16", 32768), (1, "fp8_16x16x128", 65536),
                             (2, "fp4_16x16x128", 65536), (4, "fp8_32x32x64", 131072),
                             (3, "fp4_32x32x64", 131072)):
        for wps in (1, 2):
            grid = 256 * wps
            with torch.cuda.stream(stream):
                lib.fql_calib_mfma_loop(kind, grid, iters, ctypes.c_void_p(sink.data_ptr()), sst)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(mfma_reps):
                    lib.fql_calib_mfma_loop(kind, grid, iters, ctypes.c_void_p(sink.data_ptr()), sst)
                b.record(stream)
                b.synchronize()
            ms = a.elapsed_time(b) / mfma_reps
            total = grid * 4 * iters * 8 * flop
            out["mfma_tflops"][f"{name}_waves_per_simd={wps}"] = round(total / (ms * 1e-3) / 1e12, 1)
    # the vendor library's dense float16 GEMM (torch.matmul -> hipBLASLt) on the
    # layer shapes of the largest calls, as a practical reference for an f16-MFMA GEMM
    out["library_f16_gemm_tflops"] = {}
    for (M, N, K) in ((8192, 28672, 4096), (8192, 4096, 14336), (4096, 51200, 5120),
                      (4096, 5120, 25600), (2048, 6144, 4096)):
        a = torch.randn(M, K, device=dev, dtype=torch.float16)
        b = torch.randn(N, K, device=dev, dtype=torch.float16)
        with torch.cuda.stream(stream):
            for _ in range(2):
                c = a @ b.T
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                c = a @ b.T
            e1.record(stream)
            e1.synchronize()
        ms = e0.elapsed_time(e1) / 5
        out["library_f16_gemm_tflops"][f"M={M},N={N},K={K}"] = round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)
        del a, b, c
    return out


def environment():
    """GPU, ROCm/HIP version and the GPU's clock limits (amd-smi), as far as available."""
    import torch

    env = {"hip": getattr(torch.version, "hip", None), "torch": torch.__version__}
    try:
        props = torch.cuda.get_device_properties(0)
        env.update(device=props.name, gcn_arch=getattr(props, "gcnArchName", None),
                   compute_units=props.multi_processor_count,
                   hbm_gib=round(props.total_memory / 2 ** 30, 1))
    except Exception:
        pass
    try:
        env["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    try:
        txt = subprocess.run(["amd-smi", "metric", "-c", "-p"], capture_output=True, text=True,
                             timeout=20).stdout
        for line in txt.splitlines():
            t = line.strip()
            if t.startswith("MAX_CLK:") and "gfx_max_clk_mhz" not in env:
                env["gfx_max_clk_mhz"] = t.split(":", 1)[1].strip()
            elif t.startswith("SOCKET_POWER:"):
                env["socket_power_idle"] = t.split(":", 1)[1].strip()
    except Exception:
        pass
    env["host_cpus"] = os.cpu_count()
    return env


# ---------------------------------------------------------------------------
# the oracle on the host (bounded sample)
# ---------------------------------------------------------------------------

def _threads():
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def _oracle_runner(workload, fmt, n_rows, m_rows):
    """A function running every case of the workload once through the oracle on a
    bounded sample (first `n_rows` weight rows, at most `m_rows` activation rows;
    weights quantized once, untimed); returns (seconds of oracle time, flops)."""
    import oracle.fp8 as P
    import oracle.mx as X
    import oracle.nvfp4 as Q
    import oracle.transform as TR
    import synthetic
    from oracle.formats import bf16_bits_to_f64
    from oracle.hadamard import fwht_fp32

    cases = _cases(workload)
    wcache, xcache = {}, {}

    def weight(wl, name, K, N, hb):
        key = (wl, name, hb)
        if key not in wcache:
            W = synthetic.weight(N, K, config=wl, rows=n_rows)
            if fmt != "nvfp4":
                if fmt == "mxfp4":
                    wcache[key] = X.quant_mxfp4(W)
                elif fmt == "mxfp8":
                    wcache[key] = P.quant_mxfp8(W)
                elif fmt == "fp8_block":
                    wcache[key] = P.quant_fp8_block_weight(W)
                else:
                    s = P.scale_from_amax(np.abs(W).max())
                    wcache[key] = (P.quant_fp8_tensor(W, s), s)
            else:
                Wr = fwht_fp32(W, hb) if hb and wl != "transform" else W
                gw = Q.global_scale_from_amax(Q.amax_for_calibration(Wr))
                wcache[key] = (gw,) + Q.quant_nvfp4(Wr, gw)
        return wcache[key]

    def act(wl, M, K):
        key = (wl, min(M, m_rows), K)
        if key not in xcache:
            xb = synthetic.activations(synthetic.WORKLOADS[wl]["x"], min(M, m_rows), K, config=wl)
            xcache[key] = synthetic.bf16_bits_to_f32(xb)
        return xcache[key]

    def quantize(wl, x, hb, wq):
        """the activation side: (operands for the GEMM step)"""
        if fmt == "mxfp4":
            return X.quant_mxfp4(x)
        if fmt == "mxfp8":
            return P.quant_mxfp8(x)
        if fmt == "fp8_block":
            return P.quant_fp8_block_act(x)
        if fmt == "fp8":
            sx = P.scale_from_amax(np.abs(x).max())
            return P.quant_fp8_tensor(x, sx), sx
        if wl == "transform":
            T64 = bf16_bits_to_f64(synthetic.transform_matrix(hb))
            gx = Q.global_scale_from_amax(TR.tensor_amax(TR.block_transform(x, T64)))
            return TR.quant_nvfp4_transform(x, T64, gx) + (gx,)
        gx = Q.global_scale_from_amax(Q.amax_for_calibration(x, hb))
        return Q.quant_nvfp4(x, gx, hb) + (gx,)

    def gemm(xq, wq):
        """the float64 GEMM and the epilogue"""
        if fmt == "mxfp4":
            return X.linear_mxfp4(*xq, *wq)
        if fmt == "mxfp8":
            return P.linear_mxfp8(*xq, *wq)
        if fmt == "fp8_block":
            return P.linear_fp8_block(*xq, *wq)
        if fmt == "fp8":
            return P.linear_fp8_tensor(xq[0], wq[0], P.output_scale(xq[1], wq[1]))
        gw, wc, wsc = wq
        xc, xs, gx = xq
        return Q.linear_nvfp4(xc, xs, wc, wsc, TR.dynamic_alpha(gx, gw))

    def run_once():
        """one pass: (seconds, flops, seconds in the activation quantizer)"""
        t_total = t_quant = flops = 0.0
        for (wl, M, name, K, N, hb, with_bias) in cases:
            wq = weight(wl, name, K, N, hb)
            x = act(wl, M, K)
            t0 = time.perf_counter()
            xq = quantize(wl, x, hb, wq)
            t1 = time.perf_counter()
            gemm(xq, wq)
            t2 = time.perf_counter()
            t_total += t2 - t0
            t_quant += t1 - t0
            flops += 2.0 * x.shape[0] * min(N, n_rows) * K
        return t_total, flops, t_quant

    return run_once, len(cases)


def cpu_baseline(workload, fmt="nvfp4", n_rows=384, m_rows=96, runs=3):
    """The oracle, as it stands, on a bounded sample of the workload: every case with
    the first `n_rows` weight rows and at most `m_rows` activation rows (the
    activation quantizer, the float64 GEMM and the epilogue are timed). Median of
    `runs` passes on all host cores, and median of `runs` passes on one thread."""
    run_once, ncases = _oracle_runner(workload, fmt, n_rows, m_rows)
    run_once()  # quantizes the weights (untimed) and warms up
    legs = {}
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    for leg in ("all", "one"):
        res = []
        for _ in range(runs):
            if leg == "one" and threadpool_limits is not None:
                with threadpool_limits(limits=1):
                    res.append(run_once())
            else:
                res.append(run_once())
        res.sort(key=lambda r: r[1] / r[0])
        t, f, tq = res[len(res) // 2]  # the median pass
        legs[leg] = dict(value=round(f / t / 1e12, 6), seconds=round(sum(r[0] for r in res), 1),
                         quant_s=round(tq, 3), gemm_s=round(t - tq, 3))
    sample = (f"median of {runs} passes over the {ncases} {workload} cases, each with the first "
              f"{n_rows} weight rows and at most {m_rows} activation rows (activation quantize + "
              f"float64 GEMM + epilogue); {legs['all']['seconds']} s of oracle time on all cores, "
              f"{legs['one']['seconds']} s on one thread")
    return dict(value=legs["all"]["value"], unit="TFLOP/s", cores=int(_threads()), kind="oracle",
                sample=sample,
                pass_seconds=dict(quantize=legs["all"]["quant_s"], gemm=legs["all"]["gemm_s"]),
                one_thread=dict(value=legs["one"]["value"], unit="TFLOP/s", cores=1,
                                pass_seconds=dict(quantize=legs["one"]["quant_s"],
                                                  gemm=legs["one"]["gemm_s"])))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="serving", choices=WORKLOAD_KEYS)
    ap.add_argument("--format", default="nvfp4", choices=FORMAT_KEYS)
    ap.add_argument("--hadamard-block", type=int, default=None,
                    help="restrict the hadamard/transform workloads to one block size")
    ap.add_argument("--dynamic-scale", action="store_true",
                    help="NVFP4: compute the activation global scale per call on the device")
    ap.add_argument("--cases", default=None,
                    help="comma-separated case names to run (e.g. prefill/gate_up/M=8192)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--detail", action="store_true", help="print per-case timings to stderr")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run 5 plain device-to-device copies of MB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer would shard by columns/rows across GPUs, not measured here)",
              file=sys.stderr)
        raise SystemExit(2)

    if args.copy_calibration:
        import torch

        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return
    if args.format != "nvfp4" and (args.dynamic_scale or args.workload == "transform"):
        raise SystemExit("--dynamic-scale and the transform workload are NVFP4 options")
    only = set(args.cases.split(",")) if args.cases else None
    print(f"[bench] {args.workload} {args.format}: setting up", file=sys.stderr, flush=True)
    r = gpu_bench(args.workload, args.steps, args.warmup, args.hadamard_block, fmt=args.format,
                  dynamic=args.dynamic_scale, only=only)
    print(f"[bench] timed {args.steps} steps: {r['ms_per_step']:.4f} ms/step", file=sys.stderr,
          flush=True)
    value = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
    dom_name, dom = r["dominant"]
    # binding bound of the dominant kernel: HBM bytes vs MFMA flops (the exact NVFP4
    # path multiplies dequantized float16 operands), whichever needs more time
    mfma_peak = MFMA_PEAK[args.format]
    t_hbm = dom["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = dom["flops"] / (mfma_peak * 1e12)
    if t_hbm >= t_mfma:
        ach = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(ach / mfma_peak, 4)}
        if args.format == "nvfp4":
            roof["frac_of_fp4_peak"] = round(ach / FP4_PEAK_TFLOPS, 4)
    roof.update({"traffic": measured_traffic(dom_name) if args.format == "nvfp4" else None,
                 "kernel": dom_name, "launches_per_step": dom["launches"],
                 "avg_launch_us": round(dom["ms"] * 1e3 / dom["launches"], 2),
                 "timing": "kernel alone, HIP events around each launch on its stream",
                 "alg_flops_per_launch": round(dom["flops"] / dom["launches"]),
                 "alg_bytes_per_launch": round(dom["bytes"] / dom["launches"]),
                 "cases": dom["cases"]})
    out = {
        "metric": "NVFP4 W4A4 linear TFLOP/s (quant+GEMM), M=1..8192; % of HBM/FP4-MFMA roofline",
        "format": args.format,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": FORMAT_DTYPE[args.format],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload]
                   + (", dynamic activation global scale" if args.dynamic_scale else ""),
                   "cases": len(r["per_case"]),
                   "timing": "HIP graph replay per step, weights rotated over >= 512 MB"},
        "roofline": roof,
        "per_case": r["per_case"],
    }
    if not args.no_calibration:
        print("[bench] calibration", file=sys.stderr, flush=True)
        out["calibration"] = calibration()
    out["env"] = environment()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args.workload, args.format)
    if args.detail:
        for d in r["per_case"]:
            print(json.dumps(d), file=sys.stderr)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
