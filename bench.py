"""Benchmark of the NVFP4 W4A4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode] [--format nvfp4]

A step is one pass of the whole hot path (activation quantize -> block-scaled
GEMM -> alpha/bias/bf16 epilogue, i.e. one linear call) over every case of the
workload. The default workload is the decode-shaped Llama-3.1-8B set: M in
{1, 8, 32, 128} for qkv (K=4096, N=6144), gate_up (4096, 28672) and down
(14336, 4096), with bias: 12 linear calls per step. Inputs are seeded
synthetic tensors (the `synthetic` module); weights are quantized and packed
on the GPU before timing and rotated through enough copies that every call
reads its weight from HBM, not from the 256 MB last-level cache.

Prints one JSON line. `value` is whole-step TFLOP/s (2*M*N*K summed over the
step / step time). `roofline` describes the GEMM calls against HBM bandwidth
(algorithmic bytes: 0.5625 B per weight element + 2 B per activation and
output element + bias), timed per call with HIP events on the launch stream.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

`--format mxfp4|mxfp8|fp8|fp8_block` runs one of the sibling layers (scaled
FP4/FP8 MFMA) instead; their natural workload is `siblings` (K=4096,
N=14336, M=1 and 4096). Algorithmic weight bytes per element: MXFP4 0.53125,
MXFP8 1.03125, per-tensor FP8 1, block FP8 1 + 4/128^2.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFLOPS = 10100.0
F16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 512 << 20

WORKLOAD_KEYS = ("decode", "prefill", "hadamard", "tiny", "siblings", "transform")
FORMAT_KEYS = ("nvfp4", "mxfp4", "mxfp8", "fp8", "fp8_block")
# algorithmic weight bytes per element: code + scale bytes per element
WEIGHT_BYTES = {"nvfp4": 0.5 + 1.0 / 16, "mxfp4": 0.5 + 1.0 / 32, "mxfp8": 1.0 + 1.0 / 32,
                "fp8": 1.0, "fp8_block": 1.0 + 4.0 / (128 * 128)}
# dense MFMA peak the format runs on (TFLOP/s): NVFP4 multiplies exactly
# dequantized float16 operands; the others run on the scaled FP4 / FP8 MFMA
MFMA_PEAK = {"nvfp4": 2500.0, "mxfp4": 10100.0, "mxfp8": 5000.0, "fp8": 5000.0, "fp8_block": 5000.0}
FORMAT_DTYPE = {
    "nvfp4": "nvfp4 (e2m1 x e4m3/16) -> f16 MFMA, f32 accumulate, bf16 out",
    "mxfp4": "mxfp4 (e2m1 x e8m0/32) -> scaled fp4 MFMA, f32 accumulate, bf16 out",
    "mxfp8": "mxfp8 (e4m3 x e8m0/32) -> scaled fp8 MFMA, f32 accumulate, bf16 out",
    "fp8": "fp8 e4m3, per-tensor scales -> fp8 MFMA, f32 accumulate, bf16 out",
    "fp8_block": "fp8 e4m3, 1x128 / 128x128 f32 scales -> fp8 MFMA + f32 promotion, bf16 out",
}
WORKLOAD_NAMES = {
    "decode": "decode: Llama-3.1-8B qkv/gate_up/down at M=1,8,32,128, bias",
    "prefill": "prefill: Llama-3.1-8B qkv/gate_up/down at M=2048,8192, 1% outlier channels",
    "hadamard": "hadamard: Qwen3-32B gate_up/down at M=1,256,4096, block-diagonal Hadamard",
    "tiny": "tiny: M=16, K=256, N=512",
    "siblings": "siblings: K=4096, N=14336 at M=1,4096",
    "transform": "transform: Qwen3-32B gate_up/down at M=1,256,4096, general b x b transform "
                 "(random orthogonal bf16, b=16..128)",
}


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_llama8b_hbm_traffic.md")


def source_digest():
    """sha256 over the library's kernel sources (names and bytes, sorted)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "fp8_quantized_linear_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary.

    The summary records FETCH_SIZE + WRITE_SIZE per launch (scaled by the
    plain-copy calibration) together with the digest of the kernel sources it
    was taken on; once the sources differ, the figure no longer describes the
    kernel and None is returned.
    """
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    for line in text.splitlines():
        if line.startswith("traffic-record: "):
            rec = json.loads(line[len("traffic-record: "):])
            if (rec.get("workload") == workload and rec.get("kernel") == kernel
                    and rec.get("source_sha256") == source_digest()):
                return rec["bytes_per_launch"]
    return None


def _alg_bytes(M, N, K, with_bias, fmt="nvfp4"):
    return (WEIGHT_BYTES[fmt] * N * K + 2.0 * M * K + 2.0 * M * N
            + (2.0 * N if with_bias else 0.0))


def _cases(workload, hb_override=None):
    import synthetic

    out = []
    for M, name, K, N, hb, with_bias in synthetic.cases(workload):
        if hb_override is not None and hb != hb_override:
            continue
        out.append((M, name, K, N, hb, with_bias))
    return out


def _kernel_of(M, N, K, fmt="nvfp4", general=False, dynamic=False):
    """The kernel that carries one linear call of this shape (the library's own plan;
    the transform and dynamic-scale paths plan as unaligned calls, the transform's
    with the x_hat operand)."""
    import fp8_quantized_linear_amd as fql

    if fmt != "nvfp4":
        return fql.linear_sc_plan(fmt, M, N, K).split(" grid=")[0].split(" + ")[-1]
    plan = fql.linear_plan(M, N, K, aligned=not (general or dynamic), transform=general)
    return plan.split(" grid=")[0].split(" + ")[-1]


def gpu_bench(workload, steps, warmup, hb, per_case_reps=3, fmt="nvfp4", dynamic=False):
    import torch

    import fp8_quantized_linear_amd as fql
    import synthetic

    general = workload == "transform"  # the block size is a general transform's, not a rotation's
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
    cases = _cases(workload, hb)
    setups = []
    weights = {}
    for (M, name, K, N, hbk, with_bias) in cases:
        key = (name, K, N, hbk)
        if key not in weights:
            W = torch.from_numpy(synthetic.weight(N, K, config=workload)).to(dev)
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
        xb = synthetic.activations(synthetic.WORKLOADS[workload]["x"], M, K, config=workload)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
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
            bias = torch.from_numpy(synthetic.bias(N, config=workload).view(np.int16)).view(
                torch.bfloat16).to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsb = (fql.linear_workspace_bytes(M, N, K) if fmt == "nvfp4"
               else fql.linear_sc_workspace_bytes(fmt, M, N, K))
        ws = fql.new_workspace(wsb, dev)
        setups.append(dict(M=M, N=N, K=K, name=name, hb=hbk, x=x, objs=objs, bias=bias, y=y,
                           ws=ws, flops=2.0 * M * N * K, bytes=_alg_bytes(M, N, K, with_bias, fmt),
                           kernel=_kernel_of(M, N, K, fmt, general=general, dynamic=dynamic)))
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

    # per-launch duration of each case: a graph of R back-to-back calls of that case
    # (rotating weight copies), timed with HIP events on the replay stream
    detail = []
    per_case_ms = []
    with torch.cuda.stream(stream):
        for s in setups:
            R = max(8, len(s["objs"]))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for r in range(R):
                    call(s, r)
            g.replay()
            stream.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(per_case_reps):
                g.replay()
            b.record(stream)
            b.synchronize()
            ms = a.elapsed_time(b) / (per_case_reps * R)
            per_case_ms.append(ms)
            tag = "b" if general else "hb"
            detail.append(dict(case=f"{s['name']}/M={s['M']}" + (f"/{tag}={s['hb']}" if s["hb"] else ""),
                               kernel=s["kernel"], us=round(ms * 1e3, 2),
                               tflops=round(s["flops"] / (ms * 1e-3) / 1e12, 2),
                               gbs=round(s["bytes"] / (ms * 1e-3) / 1e9, 1),
                               hbm_frac=round(s["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)))
            del g
    # dominant kernel: the one carrying the most time per step
    by_kernel = {}
    for s, ms in zip(setups, per_case_ms):
        k = by_kernel.setdefault(s["kernel"], dict(ms=0.0, bytes=0.0, flops=0.0, launches=0))
        k["ms"] += ms
        k["bytes"] += s["bytes"]
        k["flops"] += s["flops"]
        k["launches"] += 1
    dom_name, dom = max(by_kernel.items(), key=lambda kv: kv[1]["ms"])
    flops = sum(s["flops"] for s in setups)
    alg_bytes = sum(s["bytes"] for s in setups)
    return dict(ms_per_step=ms_per_step, wall_ms_per_step=wall_ms_per_step, flops=flops,
                alg_bytes=alg_bytes, detail=detail, dominant=(dom_name, dom))


def cpu_baseline_sc(workload, fmt, budget_s=12.0, n_rows=2048):
    """The sibling format's oracle on a bounded sample of the workload (as cpu_baseline)."""
    import oracle.fp8 as P
    import oracle.mx as X
    import synthetic

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1

    def quant_w(W):
        if fmt == "mxfp4":
            return X.quant_mxfp4(W)
        if fmt == "mxfp8":
            return P.quant_mxfp8(W)
        if fmt == "fp8_block":
            return P.quant_fp8_block_weight(W)
        s = P.scale_from_amax(np.abs(W).max())
        return P.quant_fp8_tensor(W, s), s

    def layer(x, wq):
        if fmt == "mxfp4":
            return X.linear_mxfp4(*X.quant_mxfp4(x), *wq)
        if fmt == "mxfp8":
            return P.linear_mxfp8(*P.quant_mxfp8(x), *wq)
        if fmt == "fp8_block":
            return P.linear_fp8_block(*P.quant_fp8_block_act(x), *wq)
        sx = P.scale_from_amax(np.abs(x).max())
        return P.linear_fp8_tensor(P.quant_fp8_tensor(x, sx), wq[0], P.output_scale(sx, wq[1]))

    cases = _cases(workload)
    wcache = {}
    flops = t_total = 0.0
    passes = 0
    while t_total < budget_s and passes < 20:
        for (M, name, K, N, hb, with_bias) in cases:
            ns = min(N, n_rows)
            if name not in wcache:
                wcache[name] = quant_w(synthetic.weight(N, K, config=workload)[:ns])
            Mr = min(M, 512)
            xb = synthetic.activations(synthetic.WORKLOADS[workload]["x"], Mr, K, config=workload)
            x = synthetic.bf16_bits_to_f32(xb)
            t0 = time.perf_counter()
            layer(x, wcache[name])
            t_total += time.perf_counter() - t0
            flops += 2.0 * Mr * ns * K
        passes += 1
    return dict(value=round(flops / t_total / 1e12, 6), unit="TFLOP/s", cores=int(threads),
                kind="oracle",
                sample=f"{passes} pass(es) over the {len(cases)} {workload} cases with the first "
                       f"{n_rows} weight rows and at most 512 activation rows each "
                       f"(x quantize + float64 GEMM + epilogue), {t_total:.1f} s of oracle time")


def cpu_baseline(workload, budget_s=12.0, n_rows=2048):
    """The oracle, as it stands, on a bounded sample of the workload.

    Every case runs with the first `n_rows` weight rows (weights quantized
    once per shape, untimed); the timed part is the activation quantizer plus
    the float64 GEMM and epilogue. Passes over the cases repeat until
    `budget_s` seconds of oracle time have accumulated.
    """
    import oracle.nvfp4 as Q
    import oracle.transform as TR
    import synthetic
    from oracle.formats import bf16_bits_to_f64
    from oracle.hadamard import fwht_fp32

    general = workload == "transform"

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cases = _cases(workload)
    wcache = {}
    flops = 0.0
    t_total = 0.0
    calls = 0
    passes = 0
    while t_total < budget_s and passes < 20:
        for (M, name, K, N, hb, with_bias) in cases:
            ns = min(N, n_rows)
            if (name, hb) not in wcache:
                W = synthetic.weight(N, K, config=workload)[:ns]
                Wr = fwht_fp32(W, hb) if hb and not general else W
                gw = Q.global_scale_from_amax(Q.amax_for_calibration(Wr))
                wcache[(name, hb)] = (gw,) + Q.quant_nvfp4(Wr, gw)
            gw, wc, wsc = wcache[(name, hb)]
            Mr = min(M, 512)  # rows of x in the sample
            xb = synthetic.activations(synthetic.WORKLOADS[workload]["x"], Mr, K, config=workload)
            x = synthetic.bf16_bits_to_f32(xb)
            if general:
                T64 = bf16_bits_to_f64(synthetic.transform_matrix(hb))
                gx = Q.global_scale_from_amax(TR.tensor_amax(TR.block_transform(x, T64)))
            else:
                gx = Q.global_scale_from_amax(Q.amax_for_calibration(x, hb))
            t0 = time.perf_counter()
            if general:
                xc, xs = TR.quant_nvfp4_transform(x, T64, gx)
            else:
                xc, xs = Q.quant_nvfp4(x, gx, hb)
            Q.linear_nvfp4(xc, xs, wc, wsc, np.float32(1.0 / (float(gx) * float(gw))))
            t_total += time.perf_counter() - t0
            flops += 2.0 * Mr * ns * K
            calls += 1
        passes += 1
    return dict(value=round(flops / t_total / 1e12, 6), unit="TFLOP/s", cores=int(threads),
                kind="oracle",
                sample=f"{passes} pass(es) over the {len(cases)} {workload} cases with the first "
                       f"{n_rows} weight rows and at most 512 activation rows each "
                       f"(x quantize + float64 GEMM + epilogue), {t_total:.1f} s of oracle time")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=WORKLOAD_KEYS)
    ap.add_argument("--format", default="nvfp4", choices=FORMAT_KEYS)
    ap.add_argument("--hadamard-block", type=int, default=None,
                    help="restrict the hadamard/transform workloads to one block size")
    ap.add_argument("--dynamic-scale", action="store_true",
                    help="NVFP4: compute the activation global scale per call on the device")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    r = gpu_bench(args.workload, args.steps, args.warmup, args.hadamard_block, fmt=args.format,
                  dynamic=args.dynamic_scale)
    value = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
    dom_name, dom = r["dominant"]
    # binding bound of the dominant kernel: HBM bytes vs f16-MFMA flops (the exact
    # NVFP4 path multiplies dequantized float16 operands), whichever needs more time
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
                "unit": "TFLOP/s", "frac": round(ach / mfma_peak, 4),
                "frac_of_fp4_peak": round(ach / FP4_PEAK_TFLOPS, 4)}
    roof.update({"kernel": dom_name, "launches_per_step": dom["launches"],
                 "alg_bytes_per_step": dom["bytes"], "flops_per_step": dom["flops"],
                 "avg_launch_us": round(dom["ms"] * 1e3 / dom["launches"], 2),
                 "alg_bytes_per_launch": round(dom["bytes"] / dom["launches"]),
                 "traffic": measured_traffic(args.workload, dom_name)
                 if args.format == "nvfp4" else None})
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
                   "cases": len(r["detail"]),
                   "timing": "HIP graph replay per step, weights rotated over >= 512 MB"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline(args.workload) if args.format == "nvfp4"
                               else cpu_baseline_sc(args.workload, args.format))
    if args.detail:
        for d in r["detail"]:
            print(json.dumps(d), file=sys.stderr)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
