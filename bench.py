"""Benchmark of the NVFP4 W4A4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

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
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFLOPS = 10100.0
F16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 512 << 20

WORKLOAD_KEYS = ("decode", "prefill", "hadamard", "tiny")


def _alg_bytes(M, N, K, with_bias):
    return 0.5625 * N * K + 2.0 * M * K + 2.0 * M * N + (2.0 * N if with_bias else 0.0)


def _cases(workload, hb_override=None):
    import synthetic

    out = []
    for M, name, K, N, hb, with_bias in synthetic.cases(workload):
        if hb_override is not None and hb != hb_override:
            continue
        out.append((M, name, K, N, hb, with_bias))
    return out


def gpu_bench(workload, steps, warmup, hb):
    import torch

    import fp8_quantized_linear_amd as fql
    import synthetic

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
            w0 = fql.NVFP4Weight.from_float(W, input_global_scale=1.0, hadamard_block=hbk)
            del W
            nbytes = w0.packed.numel()
            ncopies = max(1, -(-ROTATE_BYTES // nbytes))
            copies = [w0.packed] + [w0.packed.clone() for _ in range(ncopies - 1)]
            weights[key] = (w0, copies)
        w0, copies = weights[key]
        xb = synthetic.activations(synthetic.WORKLOADS[workload]["x"], M, K, config=workload)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        gx = fql.global_scale_from_amax(fql.amax(x, hbk).item())
        objs = [fql.NVFP4Weight(p, N, K, gx, w0.weight_global_scale, hbk) for p in copies]
        bias = None
        if with_bias:
            bias = torch.from_numpy(synthetic.bias(N, config=workload).view(np.int16)).view(
                torch.bfloat16).to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.zeros(fql.linear_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
        setups.append(dict(M=M, N=N, K=K, name=name, hb=hbk, x=x, objs=objs, bias=bias, y=y,
                           ws=ws, flops=2.0 * M * N * K, bytes=_alg_bytes(M, N, K, with_bias)))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def step(i, evs=None):
        for j, s in enumerate(setups):
            # a different weight copy on every call, so no call finds its weight in cache
            w = s["objs"][(i * len(setups) + j) % len(s["objs"])]
            if evs is not None:
                evs[j][0].record(stream)
            fql.linear_nvfp4(s["x"], w, bias=s["bias"], out=s["y"], workspace=s["ws"])
            if evs is not None:
                evs[j][1].record(stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in setups] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per_case_ms = np.zeros(len(setups))
    for i in range(steps):
        for j in range(len(setups)):
            per_case_ms[j] += events[i][j][0].elapsed_time(events[i][j][1])
    per_case_ms /= steps
    ms_per_step = (t1 - t0) * 1e3 / steps
    flops = sum(s["flops"] for s in setups)
    alg_bytes = sum(s["bytes"] for s in setups)
    detail = []
    for s, ms in zip(setups, per_case_ms):
        detail.append(dict(case=f"{s['name']}/M={s['M']}" + (f"/hb={s['hb']}" if s["hb"] else ""),
                           us=round(ms * 1e3, 2),
                           tflops=round(s["flops"] / (ms * 1e-3) / 1e12, 2),
                           gbs=round(s["bytes"] / (ms * 1e-3) / 1e9, 1),
                           hbm_frac=round(s["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)))
    sum_ms = float(per_case_ms.sum())
    return dict(ms_per_step=ms_per_step, flops=flops, alg_bytes=alg_bytes, sum_call_ms=sum_ms,
                detail=detail)


def cpu_baseline(workload, budget_s=15.0):
    """The oracle on a bounded sample: every case with a column slice of the weight."""
    import oracle.nvfp4 as Q
    import synthetic
    from oracle.hadamard import fwht_fp32

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cases = _cases(workload)
    n_cols = 512
    flops = 0.0
    t_total = 0.0
    done = 0
    for (M, name, K, N, hb, with_bias) in cases:
        ns = min(N, n_cols)
        W = synthetic.weight(N, K, config=workload)[:ns]
        Wr = fwht_fp32(W, hb) if hb else W
        gw = Q.global_scale_from_amax(Q.amax_for_calibration(Wr))
        wc, wsc = Q.quant_nvfp4(Wr, gw)
        xb = synthetic.activations(synthetic.WORKLOADS[workload]["x"], M, K, config=workload)
        x = synthetic.bf16_bits_to_f32(xb)
        gx = Q.global_scale_from_amax(Q.amax_for_calibration(x, hb))
        t0 = time.perf_counter()
        xc, xs = Q.quant_nvfp4(x, gx, hb)
        Q.linear_nvfp4(xc, xs, wc, wsc, np.float32(1.0 / (gx * gw)))
        t_total += time.perf_counter() - t0
        flops += 2.0 * M * ns * K
        done += 1
        if t_total > budget_s:
            break
    return dict(value=round(flops / t_total / 1e12, 6), unit="TFLOP/s", cores=int(threads),
                kind="oracle",
                sample=f"{done} of {len(cases)} {workload} cases, first {n_cols} weight rows each "
                       f"(x quantize + float64 GEMM), {t_total:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=WORKLOAD_KEYS)
    ap.add_argument("--hadamard-block", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--detail", action="store_true", help="print per-case timings to stderr")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer would shard by columns/rows across GPUs, not measured here)",
              file=sys.stderr)
        raise SystemExit(2)

    r = gpu_bench(args.workload, args.steps, args.warmup, args.hadamard_block)
    value = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
    gbs = r["alg_bytes"] / (r["sum_call_ms"] * 1e-3) / 1e9
    out = {
        "metric": "NVFP4 W4A4 linear TFLOP/s (quant+GEMM), M=1..8192; % of HBM/FP4-MFMA roofline",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 x e4m3/16) -> f16 MFMA, f32 accumulate, bf16 out",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: Llama-3.1-8B layer shapes" if args.workload in
                   ("decode", "prefill") else args.workload,
                   "cases": len(r["detail"])},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload)
    if args.detail:
        for d in r["detail"]:
            print(json.dumps(d), file=sys.stderr)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
