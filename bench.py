"""Throughput of the dropless top-k MoE layer forward on one MI355X.

A step is one pass of the whole forward path over one batch of synthetic
tokens: route -> permute -> grouped gated FFN (+ shared expert) -> combine,
all through the libmoe C ABI on the current stream. Inputs and weights are
resident in HBM before timing starts.

Prints one JSON line (tokens/s, per-kernel times, the dominant kernel's
roofline fraction and the CPU oracle's throughput on a bounded sample).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks.
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0


def flops(p):
    """Algorithmic FLOPs of one forward, per kernel (multiply-add = 2)."""
    T, E, k, d, h, hs = p.tokens, p.experts, p.top_k, p.d_model, p.d_hidden, p.d_shared
    S = T * k
    f = {
        "route": 2 * T * d * E,
        "gemm_gate_up": 2 * S * d * 2 * h,
        "gemm_down": 2 * S * h * d,
    }
    if hs:
        f["shared_gate_up"] = 2 * T * d * 2 * hs
        f["shared_down"] = 2 * T * hs * d
    return f


def cpu_baseline(p, sample_tokens):
    """The CPU oracle (as it stands) on the first `sample_tokens` tokens of
    the same workload: routing, permutation and every output row."""
    import dataclasses

    from dropless_grouped_gemm_router_amd.inputs import make_inputs
    from oracle import oracle

    q = dataclasses.replace(p, tokens=sample_tokens)
    inp = make_inputs(q, seed=0)
    v = {n: t.value for n, t in inp.items()}
    nthreads = oracle.max_threads()
    t0 = time.perf_counter()
    _, idx, w = oracle.route(v["x"], v["w_router"], q.top_k, nthreads)
    oracle.permute(idx, q.experts, q.block_m)
    oracle.forward_rows(v["x"], v["w_gate"], v["w_up"], v["w_down"], idx, w, v.get("ws_gate"),
                        v.get("ws_up"), v.get("ws_down"), nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of the same workload (seed 0), full forward "
                      f"in double, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, help="index into inputs.WORKLOADS")
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--cpu-sample", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (--gpus {args.gpus} "
              "requested); see the sharding paragraph of the design notes.", file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import torch

    from dropless_grouped_gemm_router_amd import binding as B
    from dropless_grouped_gemm_router_amd.inputs import WORKLOADS, make_inputs

    name, p, _ = WORKLOADS[args.workload]
    if args.block_m:
        p = dataclasses.replace(p, block_m=args.block_m)
    torch.cuda.set_device(0)
    print(f"bench: {name} bm={p.block_m}: generating inputs", file=sys.stderr, flush=True)
    dev = B.device_inputs(make_inputs(p, seed=0), "cuda:0")
    buf = B.allocate(p, "cuda:0")
    x = dev.pop("x")
    w = dev
    torch.cuda.synchronize()

    def step():
        B.forward(p, x, w, buf)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    B.moe_trace_enable(True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    kern = B.moe_trace_summary()
    B.moe_trace_enable(False)

    f = flops(p)
    per = {k: {"ms": v["ms"] / max(1, v["count"]) * (v["count"] / args.steps),
               "launches_per_step": v["count"] / args.steps} for k, v in kern.items()}
    gemms = [k for k in f if k != "route" and k in per]
    dom = max(gemms, key=lambda k: per[k]["ms"])
    dom_avg_ms = kern[dom]["ms"] / kern[dom]["count"]
    achieved = f[dom] / (dom_avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[p.dtype]
    routed_ms = sum(per[k]["ms"] for k in ("gemm_gate_up", "gemm_down"))
    routed_fl = f["gemm_gate_up"] + f["gemm_down"]
    total_fl = sum(f.values())
    line = {
        "metric": "dropless MoE fwd tokens/s + grouped-GEMM % MFMA peak (E=64 top-8, 131k tok)",
        "value": p.tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded Gaussian tokens, N(0,1/fan_in) weights)",
        "config": {"workload": name, "tokens": p.tokens, "experts": p.experts, "top_k": p.top_k,
                   "d_model": p.d_model, "d_hidden": p.d_hidden, "d_shared": p.d_shared,
                   "block_m": p.block_m},
        "tflops": total_fl / (ms * 1e-3) / 1e12,
        "grouped_gemm_pct_mfma_peak": 100.0 * routed_fl / (routed_ms * 1e-3) / 1e12 / peak,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None},
        "kernels_ms_per_step": {k: round(v["ms"], 5) for k, v in sorted(per.items())},
    }
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(p, min(args.cpu_sample, p.tokens))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
