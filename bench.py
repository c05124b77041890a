"""Benchmark of the DF-SSM scaffold projection hot path on one MI355X.

Default workload: the Mamba-2 1.3B-shaped out_proj decode step (M=1 token, K=4096,
N=2048, rank-16 int8 LoRA), cold cache: `--copies` independent weight sets
(512 x 1.16 MB = 596 MB, above the 256 MB Infinity Cache) are rotated so every
step streams its packed weights from HBM.  One step = the whole hot path over all
copies: per-token absmax int8 quantization + LoRA down (one launch for all copies),
then the bit-unpack scaffold GEMV with the fused scale/LoRA-up epilogue (one
launch for all copies).  Inputs are resident in HBM before the timed region.

Prints ONE JSON line.  `value` is whole-job HBM GB/s (algorithmic bytes of the
step / time); `roofline` rates the dominant kernel (the GEMV launch, timed live
with HIP events on its stream) against the 8 TB/s HBM peak; `cpu_baseline` is the
plain C oracle on a bounded sample of the same workload on the host cores.
Extra keys report the per-call hipGraph latency and the prefill (M=2048) int8
MFMA throughput.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (5.0 POPS)
METRIC = "µs & HBM GB/s per scaffold+LoRA GEMV at M=1 (cold); int8 TOPS at M=2048"
RANK = 16


def gemm_call_bytes(M, N, K):
    """Algorithmic bytes of one scaffold GEMM call given x_q, s_x and t."""
    return (N * K // 8 + 4 * N + 16 * N + 4 * N + 4 * RANK   # packed signs, s_w, W_A, s_A, s_B
            + M * K + 4 * M + 4 * M * RANK                   # x_q, s_x, t
            + 4 * M * N)                                     # y


def step_bytes(M, N, K):
    """Algorithmic bytes of the whole hot path for one problem: reads x and every
    weight once, writes x_q, s_x, t and y once."""
    return (4 * M * K + N * K // 8 + 4 * N + 16 * N + 4 * N + 16 * K + 4 * RANK
            + M * K + 4 * M + 4 * M * RANK + 4 * M * N)


def gemm_ops(M, N, K):
    return 2 * M * N * K + 2 * M * RANK * (K + N)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the per-call graph and prefill legs")
    ap.add_argument("--prefill-iters", type=int, default=10)
    return ap.parse_args()


def time_events(torch, fn, iters, stream):
    """Average ms of fn() over iters, bracketed by events on `stream`."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(iters):
        fn()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) / iters


def cpu_baseline(probs, seconds):
    """The oracle (as it stands) on host cores over rotated copies for ~`seconds`."""
    import oracle
    cores = min(len(os.sched_getaffinity(0)), 16)
    res = {}
    for label, nthreads, budget in (("single", 1, seconds * 0.3), ("multi", cores, seconds * 0.7)):
        n, t0 = 0, time.perf_counter()
        while True:
            p = probs[n % len(probs)]
            x_q, s_x = oracle.quantize_act(p.x)
            oracle.scaffold_lora_gemm(x_q, s_x, p.P, p.s_w, p.W_A, p.s_A, p.W_B, p.s_B, nthreads=nthreads)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                break
        res[label] = (n, el, nthreads)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the projection is not sharded "
              "across GPUs in this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth_inputs as si
    from bit_scaffold_int8_amd.runner import DeviceProjections

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    M, N, K = 1, 2048, 4096
    R = args.copies

    t0 = time.perf_counter()
    probs = si.make_copies(M, N, K, 2, seed=1, copies=R)
    dp = DeviceProjections.from_problems(probs, device=dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    weight_bytes = R * (N * K // 8 + 4 * N + 16 * N + 4 * N + 16 * K + 4 * RANK)

    def step():
        dp.quantize_lora_down(stream)
        dp.gemm(stream, debug=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # the dominant kernel (the scaffold GEMV launch over all copies), timed live on its
    # stream: K back-to-back launches between two events, so the average is the
    # kernel's duration plus only the dispatch gap between consecutive launches
    gemv_ms = time_events(torch, lambda: dp.gemm(stream, debug=False), args.steps, stream)

    value = R * step_bytes(M, N, K) / (ms_per_step * 1e-3) / 1e9
    achieved = R * gemm_call_bytes(M, N, K) / (gemv_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "out_proj_decode_m1_k4096_n2048",
            "M": M, "K": K, "N": N, "rank": RANK,
            "copies_rotated": R, "rotated_weight_bytes": weight_bytes,
            "launch": "strided-batched: 2 launches per step (quantize+LoRA-down, scaffold GEMV) over all copies",
        },
        "us_per_gemv_step": round(ms_per_step * 1e3 / R, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_kernel (dfssm_scaffold_lora_gemm_strided_batched, M=1)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_launch_us": round(gemv_ms * 1e3, 3),
            "timing": "HIP events around back-to-back launches on the kernel's stream",
            "algorithmic_bytes_per_launch": R * gemm_call_bytes(M, N, K),
        },
    }

    if not args.no_extras:
        # per-call latency: every copy's two launches captured in one hipGraph
        single = [DeviceProjections(
            x=dp.x[b:b + 1], w_bits=dp.w_bits[b:b + 1], s_w=dp.s_w[b:b + 1], w_a=dp.w_a[b:b + 1],
            s_a=dp.s_a[b:b + 1], w_b=dp.w_b[b:b + 1], s_b=dp.s_b[b:b + 1], x_q=dp.x_q[b:b + 1],
            s_x=dp.s_x[b:b + 1], t=dp.t[b:b + 1], y=dp.y[b:b + 1], acc_dbg=None) for b in range(R)]
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        with torch.cuda.stream(cs):
            for p in single[:4]:
                p.forward(cs, debug=False)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cs):
            for p in single:
                p.forward(torch.cuda.current_stream(), debug=False)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        reps = 5
        graph_ms = time_events(torch, g.replay, reps, torch.cuda.current_stream())
        us_call = graph_ms * 1e3 / R
        out["per_call_graph"] = {
            "us_per_call": round(us_call, 3),
            "GBps": round(step_bytes(M, N, K) / (us_call * 1e-6) / 1e9, 2),
            "launches_per_call": 2,
            "note": "R rotated single-problem calls (2 kernels each) captured in one hipGraph",
        }

        # prefill: M=2048 tokens on the int8 MFMA path
        pre = {}
        for name, (pM, pN, pK, po) in zip(("in_proj", "out_proj"), si.CONFIGS["prefill_m2048"]["shapes"]):
            pp = DeviceProjections.from_problems([si.make_problem(pM, pN, pK, po, seed=4)], device=dev)
            pp.forward(debug=False)
            torch.cuda.synchronize()
            q_ms = time_events(torch, lambda: pp.quantize_lora_down(stream), args.prefill_iters, stream)
            g_ms = time_events(torch, lambda: pp.gemm(stream, debug=False), args.prefill_iters, stream)
            tops = gemm_ops(pM, pN, pK) / (g_ms * 1e-3) / 1e12
            pre[name] = {"M": pM, "K": pK, "N": pN, "gemm_us": round(g_ms * 1e3, 2),
                         "quantize_lora_down_us": round(q_ms * 1e3, 2), "TOPS": round(tops, 1),
                         "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
            del pp
        out["prefill_m2048"] = pre

    if not args.no_cpu_baseline:
        res = cpu_baseline(probs, args.cpu_seconds)
        n, el, cores = res["multi"]
        out["cpu_baseline"] = {
            "value": round(n * step_bytes(M, N, K) / el / 1e9, 4),
            "unit": "GB/s",
            "cores": cores,
            "kind": "oracle",
            "sample": f"{n} rotated out_proj decode problems (M=1 K=4096 N=2048), quantize + scaffold/LoRA "
                      f"projection, {el:.1f} s wall on {cores} threads; single-thread: "
                      f"{res['single'][0]} problems in {res['single'][1]:.1f} s",
            "us_per_call": round(el / n * 1e6, 1),
            "single_thread_us_per_call": round(res["single"][1] / res["single"][0] * 1e6, 1),
        }
    out["setup_s"] = round(setup_s, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
