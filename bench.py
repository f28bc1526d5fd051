"""Throughput of the dropless top-k MoE layer forward on one MI355X.

A step is one pass of the whole forward path over one batch of synthetic
tokens: route -> permute -> grouped gated FFN (+ shared expert) -> combine,
all through the libmoe C ABI on the current stream. Inputs and weights are
resident in HBM before timing starts.

Prints one JSON line: tokens/s, per-kernel times from HIP events over the
timed steps, the dominant kernel's roofline fraction, the train step
(forward + backward) on the 16384-token workload, and the CPU oracle's
throughput on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks (no sparsity).
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0
# fp32 vector FMA peak without packed math: 256 CUs x 64 lanes x 2 flop x 2.4 GHz.
PEAK_VALU_TFLOPS = 78.6

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TRAFFIC_TRAIN_FILE = os.path.join(ROOT, "profiles", "traffic_train.json")
KERNEL_SOURCES = ["gemm_core.h", "gemm_wide.h", "gemm_launch.h", "gemm_dgrad.h", "gemm_wgrad.h",
                  "ffn.hip", "route.hip", "permute.hip", "combine.hip", "bwd.hip", "common.h",
                  "sort_rows.h"]


def strip_comments(src):
    """C++ source without its comments and blank lines (string and character
    literals kept), so that a comment edit does not mark the counters of an
    unchanged kernel as stale."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = [ln.rstrip() for ln in "".join(out).split("\n")]
    return "\n".join(ln for ln in lines if ln.strip())


def kernel_source_hash():
    """Hash of the kernel sources (comments stripped) that the stored
    FETCH/WRITE counters were taken with."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dropless_grouped_gemm_router_amd", "csrc", f)) as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def work(p, dispatch="gather"):
    """Algorithmic work of each forward kernel per launch: (flops, bytes).
    FLOPs count a multiply-add as 2; bytes are the minimum each kernel must
    move through HBM (each input read once, each output written once)."""
    T, E, k, d, h, hs = p.tokens, p.experts, p.top_k, p.d_model, p.d_hidden, p.d_shared
    S = T * k
    es = 2 if p.dtype == "bf16" else 4
    # the gate/up GEMM reads each token once, or (sorted) the expert-ordered copy
    a_rows = S if dispatch == "sorted" else T
    w = {
        # x and the router read, indices and weights written
        "route": (2 * T * d * E, T * d * es + d * E * 4 + S * 8),
        # tokens, packed gate|up weights, H written
        "gemm_gate_up": (2 * S * d * 2 * h, a_rows * d * es + E * 2 * h * d * es + S * h * es),
        # H read, down weights, y_sorted written
        "gemm_down": (2 * S * h * d, S * h * es + E * h * d * es + S * d * es),
        # y_sorted and shared_out read, combine weights and slot map read, out written
        "combine": (0, S * d * es + S * 8 + T * d * es * (2 if hs else 1)),
        # expert indices read twice (count, scatter), perm and inv_perm written
        "permute_scatter": (0, S * 4 * 3),
        # tokens read once, perm read, the expert-ordered copy written
        "sort_rows": (0, T * d * es + S * 4 + S * d * es),
    }
    if hs:
        w["shared_gate_up"] = (2 * T * d * 2 * hs, T * d * es + 2 * hs * d * es + T * hs * es)
        w["shared_down"] = (2 * T * hs * d, T * hs * es + hs * d * es + T * d * es)
        # shared down GEMM with the gather-sum in its epilogue: y_sorted,
        # weights and slot map read, out written (no shared_out round trip)
        w["shared_down_combine"] = (2 * T * hs * d,
                                    T * hs * es + hs * d * es + S * d * es + S * 8 + T * d * es)
    return w


def bwd_work(p):
    """Algorithmic work of each backward kernel per launch: (flops, bytes),
    counted as in ``work``. S = T*k token-slots; weight gradients are fp32."""
    T, E, k, d, h, hs = p.tokens, p.experts, p.top_k, p.d_model, p.d_hidden, p.d_shared
    S = T * k
    es = 2 if p.dtype == "bf16" else 4
    w = {
        # dA|dB and gate/up weights read, per-slot dX written
        "bwd_gate_up_dgrad": (2 * S * 2 * h * d, S * 2 * h * es + E * 2 * h * d * es + S * d * es),
        # token rows and dA|dB read, fp32 dW_gate, dW_up written
        "bwd_wgrad_gate_up": (2 * S * d * 2 * h, T * d * es + S * 2 * h * es + E * d * 2 * h * 4),
        # per-slot dX, router term and shared dx read, grad_x written
        "bwd_dx": (2 * S * d, S * d * es + E * d * 4 + S * 8 + 2 * T * d * es),
    }
    if p.dtype == "bf16":
        ks = max(1, min(64, T // 256))
        w.update({
            # tokens and the dl hi/lo table read, the splits' fp32 partials written
            "bwd_router_wgrad": (2 * T * d * 128, T * d * es + T * 128 * 2 + ks * d * 128 * 4),
            # grad_out rows (once), down weights, saved gate/up and the sorted
            # rows' combine weights read; dA|dB, w H and the dw parts written
            "bwd_down_dgrad": (2 * S * d * h, T * d * es + E * h * d * es + S * 2 * h * es + S * 4
                               + S * 2 * h * es + S * h * es + (h // 128) * S * 4),
            # grad_out rows (once) and w H read, fp32 dW_down written
            "bwd_wgrad_down": (2 * S * h * d, T * d * es + S * h * es + E * h * d * 4),
        })
    else:
        w.update({
            # grad_out and y read, dY written, weights / slot map read, dl written
            "bwd_combine": (2 * S * d, T * d * es + S * d * es + S * d * es + S * 12),
            # token rows and dl read, per-piece partials written
            "bwd_router_partial": (2 * S * d, T * d * es + S * 8 + ((S + p.block_m - 1) // p.block_m + E) * d * 4),
            # dY, down weights and saved gate/up read, dA|dB written
            "bwd_down_dgrad": (2 * S * d * h, S * d * es + E * h * d * es + 2 * S * 2 * h * es),
            # H and dY read, fp32 dW_down written
            "bwd_wgrad_down": (2 * S * h * d, S * h * es + S * d * es + E * h * d * 4),
        })
    if hs:
        w.update({
            "bwd_shared_down_dgrad": (2 * T * d * hs, T * d * es + hs * d * es + 2 * T * 2 * hs * es),
            "bwd_shared_gate_up_dgrad": (2 * T * 2 * hs * d, T * 2 * hs * es + 2 * hs * d * es + T * d * es),
            "bwd_shared_wgrad_down": (2 * T * hs * d, T * hs * es + T * d * es + hs * d * 4),
            "bwd_shared_wgrad_gate_up": (2 * T * d * 2 * hs, T * d * es + T * 2 * hs * es + d * 2 * hs * 4),
        })
    return w


def roofline_of(kname, flops, nbytes, avg_ms, dtype):
    """Roofline position of one launch: the bound is whichever of compute
    (MFMA, or fp32 VALU for the router) and HBM takes longer at peak."""
    t = avg_ms * 1e-3
    if kname == "route":
        cpeak, cunit, cbound = PEAK_VALU_TFLOPS, "TFLOP/s", "alu"
    else:
        cpeak, cunit, cbound = PEAK_TFLOPS[dtype], "TFLOP/s", "mfma"
    t_compute = flops / (cpeak * 1e12)
    t_mem = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_compute >= t_mem:
        ach = flops / t / 1e12
        return {"kernel": kname, "bound": cbound, "achieved": ach, "peak": cpeak, "unit": cunit,
                "frac": ach / cpeak}
    ach = nbytes / t / 1e9
    return {"kernel": kname, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBS}


def trace_name(kernel):
    """libmoe trace name of a compiled kernel, from its signature. Kernels
    that serve two stages of one step get the first stage's name here;
    ``step_trace_names`` tells the launches apart by their order."""
    import re
    if "route_kernel" in kernel or "route_resident_kernel" in kernel:
        return "route"
    for k, name in (("combine_bwd", "bwd_combine"), ("router_partial", "bwd_router_partial"),
                    ("router_reduce", "bwd_router_reduce"), ("router_reduce_hl", "bwd_router_reduce"),
                    ("router_transpose", "bwd_router_transpose"), ("router_dl", "bwd_router_dl"),
                    ("split_reduce", "bwd_split_reduce"), ("dx_gather", "bwd_dx"),
                    ("down_dgrad", "bwd_down_dgrad"), ("bwd_prep", "bwd_prep"),
                    ("fill_zero", "fill_zero"), ("retile", "retile")):
        if f"{k}_kernel" in kernel or f"{k}_k_kernel" in kernel:
            return name
    if "combine_kernel" in kernel or "combine_k_kernel" in kernel:
        return "combine"
    for k in ("count", "scan", "scatter"):
        if f"{k}_kernel" in kernel:
            return f"permute_{k}"
    if "pack_kernel" in kernel or "pack_bf16" in kernel:
        return "pack_weights"
    if "sort_rows_kernel" in kernel:
        return "sort_rows"
    m = re.search(r"wgrad_tr_kernel<moe::TrCfg<(\d+), \d+>, (true|false), (true|false)>", kernel)
    if m:
        if m.group(2) == "true":
            # dense: the router's split GEMM (128-row M tiles at its size) or
            # the shared expert's two weight gradients (down first)
            return "bwd_router_wgrad" if m.group(1) == "128" else "bwd_shared_wgrad_down"
        # the routed weight gradients, down first
        return "bwd_wgrad_down"
    m = re.search(r"wgrad_kernel<[^,]*, (true|false), (true|false)>", kernel)
    if m:  # fp32: <T, gathered A, dense>
        if m.group(2) == "true":
            return "bwd_shared_wgrad_down"
        return "bwd_wgrad_gate_up" if m.group(1) == "true" else "bwd_wgrad_down"
    m = (re.search(r"wide_gemm_kernel<(true|false), (\d), (true|false)>", kernel) or
         re.search(r"gemm_kernel<.*>, (true|false), (\d), (true|false)>", kernel))
    if m:
        gather, epi, dense = m.group(1) == "true", int(m.group(2)), m.group(3) == "true"
        if epi == 2:
            return "bwd_shared_down_dgrad" if dense else "bwd_down_dgrad"
        if dense:
            return {1: "shared_gate_up", 3: "shared_down_combine"}.get(epi, "shared_down")
        return "gemm_gate_up" if epi == 1 else "gemm_down"
    return None


# A compiled kernel that serves two stages of a train step: its n-th launch
# within one step is the n-th stage named here.
_SECOND_USE = {"shared_down": "bwd_shared_gate_up_dgrad", "gemm_down": "bwd_gate_up_dgrad",
               "bwd_shared_wgrad_down": "bwd_shared_wgrad_gate_up", "retile": "bwd_retile",
               "bwd_split_reduce": "bwd_split_reduce_gate_up", "bwd_wgrad_down": "bwd_wgrad_gate_up"}


def step_trace_names(kernels):
    """Trace names of a sequence of launches (in dispatch order) made by
    whole steps, each opening with the weight pack: a kernel's second launch
    within a step is the second stage it serves (``_SECOND_USE``)."""
    names, seen = [], set()
    for k in kernels:
        n = trace_name(k)
        if n == "pack_weights":
            seen = set()
        if n in seen and n in _SECOND_USE:
            n = _SECOND_USE[n]
        seen.add(n)
        names.append(n)
    return names


def reference_rates(steps, warmup):
    """Practical ceilings on this GPU, next to the published peaks: a plain
    device copy (bytes read + written per second) and the vendor BLAS
    (torch.matmul, hipBLASLt on ROCm) on the dense shapes of the 131072-token
    layer. Reference measurements only; nothing in libmoe calls a library
    GEMM."""
    import torch
    dev = "cuda:0"
    torch.cuda.set_device(0)
    steps, warmup = max(steps, 5), max(warmup, 2)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    lines = []
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src))
    lines.append({"reference": "device copy 1 GiB", "ms": round(ms, 4),
                  "GB/s": round(2 * n / ms / 1e6, 1)})
    del src, dst
    torch.manual_seed(0)
    shapes = [("shared gate/up: x[131072,512] W[512,2048]", 131072, 512, 2048),
              ("shared down: h[131072,1024] W[1024,512]", 131072, 1024, 512),
              ("routed gate/up as one dense GEMM: [1048576,512] W[512,256]", 1048576, 512, 256),
              ("routed down as one dense GEMM: [1048576,128] W[128,512]", 1048576, 128, 512),
              ("square 8192", 8192, 8192, 8192)]
    for label, M, K, N in shapes:
        a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
        bt = torch.randn(N, K, device=dev, dtype=torch.bfloat16)  # weights [N][K]
        ms = timed(lambda: a @ bt.t())
        tf = 2 * M * K * N / ms / 1e9
        lines.append({"reference": f"torch.matmul bf16 {label}", "ms": round(ms, 4),
                      "TFLOP/s": round(tf, 1), "frac_mfma_peak": round(tf / PEAK_TFLOPS["bf16"], 4)})
        del a, bt
    return lines


def load_traffic(path, workload_name):
    """Per-kernel counter bytes from a committed traffic summary, or {} when
    it was taken on another workload or before the kernel sources changed."""
    try:
        with open(path) as fh:
            tr = json.load(fh)
    except (OSError, ValueError):
        return {}
    if tr.get("source_hash") != kernel_source_hash() or tr.get("workload") != workload_name:
        return {}
    return tr.get("kernels", {})


STAGE_PROBE_MODES = {0: "no loads (operands stay in LDS)", 1: "token half loaded (32 KiB)",
                     2: "weight half loaded (32 KiB)", 3: "whole stage loaded (64 KiB)",
                     4: "64 KiB into registers", 5: "64 KiB of LDS stores, no loads",
                     6: "64 KiB issued by waves 0-3 only",
                     7: "MFMA only (fragments held in registers)",
                     8: "whole stage, four waves of 128x128",
                     9: "whole stage, token rows three-deep",
                     10: "whole stage, four waves, loads spread between MFMAs"}


def stage_probe(reps=20):
    """The wide GEMM engine's K-stage loop on its own (libmoe_probe.so):
    256 persistent 8-wave workgroups, 16 tiles of 256 x 256 x 512 each, with
    each stage's loads varied. One JSON line per configuration."""
    import ctypes

    import torch

    torch.cuda.set_device(0)
    lib = ctypes.CDLL(os.path.join(ROOT, "dropless_grouped_gemm_router_amd", "libmoe_probe.so"))
    lib.moe_stage_probe.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_float)]
    grid, items = 256, 16
    flops = 2.0 * 256 * 256 * 512 * grid * items
    regions = [(4096, 0, "4 MiB of token rows in order (L2)"),
               (131072, 1, "rows hashed over 128 MiB (Infinity Cache)"),
               (1 << 20, 1, "rows hashed over 1 GiB (HBM)")]
    # zero operands (every mode), then random bf16 operands for the modes
    # that bound a real GEMM: the MFMA pipes alone, the LDS-fed loop, and
    # the whole stage from each place the token rows can come from
    runs = ([(m, regions[0], 0) for m in range(8)] +
            [(m, r, 0) for r in regions[1:] for m in (3, 8, 9, 10)] +
            [(7, regions[0], 1), (0, regions[0], 1), (3, regions[0], 1), (3, regions[1], 1),
             (3, regions[2], 1), (8, regions[1], 1), (9, regions[1], 1), (9, regions[2], 1),
             (10, regions[1], 1), (10, regions[2], 1)])
    for mode, (rows, rnd, where), data in runs:
        ms = ctypes.c_float(0.0)
        rc = lib.moe_stage_probe(mode, rows, rnd, data, grid, items, reps, ctypes.byref(ms))
        if rc != 0:
            raise RuntimeError(f"moe_stage_probe(mode {mode}) returned {rc}")
        tf = flops / (ms.value * 1e-3) / 1e12
        print(json.dumps({"stage_probe": STAGE_PROBE_MODES[mode], "mode": mode, "tokens": where,
                          "data": "random bf16" if data else "zeros",
                          "ms": round(ms.value, 4), "TFLOP/s": round(tf, 1),
                          "frac_mfma_peak": round(tf / PEAK_TFLOPS["bf16"], 4)}), flush=True)


STORE_PROBE_MODES = {0: "256x256 tiles, neighbouring workgroups share a row block",
                     1: "128x512 tiles (whole rows)",
                     2: "256x256 tiles, both column halves of a row block per workgroup"}


def store_probe(reps=20):
    """Write rate of the GEMM epilogue's store pattern (libmoe_probe.so):
    1 GiB of bf16 [2^20][512] rows in three tile orders. One JSON line each."""
    import ctypes

    import torch

    torch.cuda.set_device(0)
    lib = ctypes.CDLL(os.path.join(ROOT, "dropless_grouped_gemm_router_amd", "libmoe_probe.so"))
    lib.moe_store_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    for mode, what in STORE_PROBE_MODES.items():
        ms = ctypes.c_float(0.0)
        rc = lib.moe_store_probe(mode, reps, ctypes.byref(ms))
        if rc != 0:
            raise RuntimeError(f"moe_store_probe(mode {mode}) returned {rc}")
        print(json.dumps({"store_probe": what, "mode": mode, "ms": round(ms.value, 4),
                          "TB/s": round(2 ** 30 / (ms.value * 1e-3) / 1e12, 3)}), flush=True)


def mfma_ceiling(reps=10):
    """Context for the bf16 rooflines, measured on this GPU with the
    stage-loop probe on random bf16 operands: the fraction of the published
    MFMA peak that the MFMA instructions alone sustain (the clock the chip
    holds under that load), and that the wide engine's K-stage loop reaches
    with its token rows gathered from a 128 MiB region, as the routed
    gate/up GEMM reads them. None if the probe library is missing."""
    import ctypes

    path = os.path.join(ROOT, "dropless_grouped_gemm_router_amd", "libmoe_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.moe_stage_probe.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_float)]
    grid, items = 256, 16
    flops = 2.0 * 256 * 256 * 512 * grid * items

    def frac(mode, rows, rnd):
        ms = ctypes.c_float(0.0)
        rc = lib.moe_stage_probe(mode, rows, rnd, 1, grid, items, reps, ctypes.byref(ms))
        if rc != 0:
            raise RuntimeError(f"moe_stage_probe(mode {mode}) returned {rc}")
        return round(flops / (ms.value * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4)

    return {"mfma_only_frac": frac(7, 4096, 0),
            "stage_loop_gathered_frac": frac(3, 131072, 1),
            "source": "libmoe_probe.so stage-loop probe (bench.py --stage-probe modes 7 and 3), "
                      "random bf16 operands, fractions of the published 2.5 PFLOP/s"}


def pmc_summary(fetch_dir, write_dir, copyf_dir, copyw_dir, workload_name, out_path):
    """HBM bytes per launch of each kernel from rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs (KiB per dispatch), each scaled by what the same counter
    reports for a plain device copy of known size. Launches are named in
    dispatch order (``step_trace_names``); a name's figure is the median over
    its launches."""
    import csv
    import statistics

    def per_dispatch(d, counter):
        rows = []
        with open(os.path.join(d, "run_counter_collection.csv")) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        rows.sort()
        return rows

    def per_name(d, counter):
        rows = per_dispatch(d, counter)
        vals = {}
        for n, (_, _, v) in zip(step_trace_names([k for _, k, _ in rows]), rows):
            if n is not None:
                vals.setdefault(n, []).append(v)
        return vals

    def copy_scale(d, counter):
        kib = [v for _, k, v in per_dispatch(d, counter) if "copyBuffer" in k]
        n = 1024 << 20  # the calibration copies 1024 MiB
        return n / (statistics.median(kib) * 1024.0)

    fs, ws = copy_scale(copyf_dir, "FETCH_SIZE"), copy_scale(copyw_dir, "WRITE_SIZE")
    fetch, write = per_name(fetch_dir, "FETCH_SIZE"), per_name(write_dir, "WRITE_SIZE")
    out = {"workload": workload_name, "source_hash": kernel_source_hash(),
           "fetch_scale": fs, "write_scale": ws, "kernels": {}}
    for name, fv in fetch.items():
        if name not in write:
            continue
        fb = statistics.median(fv) * 1024.0 * fs
        wb = statistics.median(write[name]) * 1024.0 * ws
        out["kernels"][name] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                                "launches": len(fv)}
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1, sort_keys=True))


def cpu_baseline(p, inputs, sample_tokens):
    """The CPU oracle (as it stands) on the first `sample_tokens` tokens of
    the same generated inputs: routing, permutation and every output row."""
    from oracle import oracle

    v = {n: t.value for n, t in inputs.items()}
    x = v["x"][:sample_tokens]
    nthreads = oracle.max_threads()
    t0 = time.perf_counter()
    _, idx, w = oracle.route(x, v["w_router"], p.top_k, nthreads)
    r = oracle.permute(idx, p.experts, p.block_m, capacity=p.capacity)
    keep = oracle.keep_mask(r, sample_tokens, p.top_k) if p.capacity else None
    oracle.forward_rows(x, v["w_gate"], v["w_up"], v["w_down"], idx, w, v.get("ws_gate"),
                        v.get("ws_up"), v.get("ws_down"), nthreads=nthreads, keep=keep)
    dt = time.perf_counter() - t0
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"first {sample_tokens} of the {p.tokens} tokens of the same seeded inputs: "
                      f"routing, permutation and every output row in double, {dt:.1f} s wall"}


def time_steps(step, steps, warmup):
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def pages_timing(step, ms_hint, samples=21):
    """The pages' timing protocol (kernel_gmm_gpu.json result records, fields
    median_ms, q1_ms, q3_ms and inner): samples of `inner` back-to-back
    steps, inner = clamp(round(45 ms / t), 1, 200) for a step time t, each
    sample bracketed by HIP events on the current stream; milliseconds per
    step of the median sample and of the quartiles."""
    import statistics

    import torch

    inner = max(1, min(200, round(45.0 / max(ms_hint, 1e-3))))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(samples + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(samples):
        for _ in range(inner):
            step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) / inner for i in range(samples))
    q = statistics.quantiles(per, n=4, method="inclusive")
    return {"samples": samples, "inner": inner, "median_ms": statistics.median(per),
            "q1_ms": q[0], "q3_ms": q[2], "min_ms": per[0], "max_ms": per[-1]}


def train_step_line(B, steps, warmup, tokens=0, pages=True):
    """Forward + backward on the train-step workload (16384 tokens, or
    `tokens` of the same layer)."""
    import dataclasses

    import torch

    from dropless_grouped_gemm_router_amd.inputs import WORKLOADS, make_inputs

    name, p, _ = WORKLOADS[4]
    if tokens:
        p = dataclasses.replace(p, tokens=tokens)
        name = name.replace("16384 tok", f"{tokens} tok")
    dev = B.device_inputs(make_inputs(p, seed=0, with_grad_out=True), "cuda:0")
    buf = B.allocate(p, "cuda:0", training=True, dispatch="gather")
    x, g = dev.pop("x"), dev.pop("grad_out")
    side = torch.cuda.Stream()  # the shared expert's part runs there
    torch.cuda.synchronize()

    def step():
        B.forward_dispatch(p, "gather", x, dev, buf, training=True, side_stream=side)
        B.backward(p, x, dev, g, buf, side_stream=side)

    ms = time_steps(step, steps, warmup)
    pages = pages_timing(step, ms) if pages else None
    # per-kernel times of the same steps, from libmoe's HIP events (with the
    # kernel timer on, the second stream is not used, so each duration is
    # that of the kernel alone)
    B.moe_trace_enable(True)
    time_steps(step, steps, 0)
    kern = B.moe_trace_summary()
    B.moe_trace_enable(False)
    T, E, k, d, h, hs = p.tokens, p.experts, p.top_k, p.d_model, p.d_hidden, p.d_shared
    fwd = 2 * T * d * E + 6 * T * k * d * h + 6 * T * d * hs
    wk = dict(work(p))
    wk.update(bwd_work(p))
    avg = {kn: v["ms"] / v["count"] for kn, v in kern.items()}
    roofs = {kn: roofline_of(kn, wk[kn][0], wk[kn][1], avg[kn], p.dtype) for kn in wk if kn in avg}
    traffic = load_traffic(TRAFFIC_TRAIN_FILE, name)
    return {"workload": name, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "pages_timing": pages,
            "tflops_3x_fwd": 3 * fwd / (ms * 1e-3) / 1e12, "steps": steps, "warmup": warmup,
            "kernels_ms_per_step": {kn: round(v["ms"] / steps, 5) for kn, v in sorted(kern.items())},
            "kernel_rooflines": {kn: {"frac": round(r["frac"], 4), "achieved": round(r["achieved"], 1),
                                      "unit": r["unit"], "bound": r["bound"],
                                      "traffic": (round(traffic[kn]["bytes_per_launch"])
                                                  if kn in traffic else None)}
                                 for kn, r in sorted(roofs.items())}}


def train_footprint(B, p):
    """Device bytes of one train step without allocating anything: the
    inputs (tokens, grad_out, weights), every buffer ``binding.allocate``
    makes with training=True (routing, y_sorted, out, grad_x, shared_out,
    workspace, saved activations, fp32 weight gradients)."""
    T, E, k, d, h, hs = p.tokens, p.experts, p.top_k, p.d_model, p.d_hidden, p.d_shared
    S = T * k
    es = 2 if p.dtype == "bf16" else 4
    inputs = 2 * T * d * es + d * E * 4 + 3 * E * d * h * es + 3 * d * hs * es
    routing = 2 * T * k * 4 + (E + 1) * 4 + 2 * S * 4 + max(1, B.moe_max_tiles(p)) * 12 + 4
    acts = S * d * es + T * d * es * (3 if hs else 2)
    grads = (d * E + 3 * E * d * h + 3 * d * hs) * 4
    return (inputs + routing + acts + grads + B.moe_workspace_bytes(p, True)
            + B.moe_saved_bytes(p))


MAXTOK_BLOCK = 131072


def maxtok_line(B, steps, warmup):
    """Largest train step that fits this GPU at the pages' max-token shape
    (kernel_gmm_gpu.json "maxtok" suite: E=8, top-2, d_model 512, d_hidden
    1024, bf16), with peak device memory and step time at token counts up to
    it. Tokens and grad_out are the seeded 131072-token block repeated."""
    import dataclasses

    import torch

    from dropless_grouped_gemm_router_amd.inputs import Problem, make_inputs

    p0 = Problem(MAXTOK_BLOCK, 8, 2, 512, 1024, 0, "bf16", 128)
    dev = B.device_inputs(make_inputs(p0, seed=0, with_grad_out=True), "cuda:0")
    x0, g0 = dev.pop("x"), dev.pop("grad_out")
    torch.cuda.synchronize()
    free, total = torch.cuda.mem_get_info()
    budget = int(free * 0.96)
    tmax = MAXTOK_BLOCK
    while train_footprint(B, dataclasses.replace(p0, tokens=tmax + MAXTOK_BLOCK)) <= budget:
        tmax += MAXTOK_BLOCK
    points = sorted({t for t in (MAXTOK_BLOCK, 1 << 20, 1 << 22, tmax) if t <= tmax})
    out = []
    for T in points:
        p = dataclasses.replace(p0, tokens=T)
        print(f"bench: maxtok {T} tokens", file=sys.stderr, flush=True)
        reps = -(-T // MAXTOK_BLOCK)
        x = x0.repeat(reps, 1)[:T].contiguous()
        g = g0.repeat(reps, 1)[:T].contiguous()
        buf = B.allocate(p, "cuda:0", training=True)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()

        def step():
            B.forward(p, x, dev, buf, training=True)
            B.backward(p, x, dev, g, buf)

        ms = time_steps(step, steps, warmup)
        peak = torch.cuda.max_memory_allocated()
        out.append({"tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
                    "peak_mb": peak / 2 ** 20, "footprint_mb": train_footprint(B, p) / 2 ** 20})
        del buf, x, g
        torch.cuda.empty_cache()
    return {"metric": "largest train step on one GPU (max tokens)", "value": tmax,
            "unit": "tokens", "higher_is_better": True, "n_gpus": 1,
            "config": {"workload": "train bf16, E8 top-2, d512 h1024 (max-token shape)",
                       "experts": 8, "top_k": 2, "d_model": 512, "d_hidden": 1024,
                       "block_m": p0.block_m, "dtype": "bf16"},
            "device_free_mb_at_start": free / 2 ** 20, "device_total_mb": total / 2 ** 20,
            "budget_frac": 0.96, "bytes_per_token": (train_footprint(B, dataclasses.replace(p0, tokens=2 * MAXTOK_BLOCK))
                                                     - train_footprint(B, p0)) / MAXTOK_BLOCK,
            "points": out, "data": "synthetic: a seeded 131072-token block repeated"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, help="index into inputs.WORKLOADS")
    ap.add_argument("--block-m", type=int, default=None)
    ap.add_argument("--dispatch", choices=["gather", "sorted", "fused_gsum"], default="gather",
                    help="forward dispatch variant (moe_forward)")
    ap.add_argument("--capacity-factor", type=float, default=0.0,
                    help="capacity routing: per-expert capacity ceil(F * tokens * top_k / "
                         "experts); 0 = dropless")
    ap.add_argument("--skew", type=float, default=0.0,
                    help="routing skew of the synthetic router (inputs.Problem.skew)")
    ap.add_argument("--cpu-sample", type=int, default=131072,
                    help="tokens the CPU oracle runs on (about 10 s on 16 cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--no-pages", action="store_true",
                    help="skip the pages' sampled timing and the MFMA ceiling probe (short runs "
                         "under a profiler)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one forward step captured in a HIP graph")
    ap.add_argument("--maxtok", action="store_true",
                    help="largest train step that fits (E8 top-2 d512 h1024 bf16) and peak memory")
    ap.add_argument("--train-tokens", type=int, default=0, metavar="T",
                    help="only time the train step (forward + backward) of the train-step layer "
                         "at T tokens, one JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (counter calibration)")
    ap.add_argument("--reference", action="store_true",
                    help="only time reference rates on this GPU: a plain device copy and the "
                         "vendor BLAS (torch.matmul) on this layer's GEMM shapes")
    ap.add_argument("--store-probe", action="store_true",
                    help="write rate of the GEMM epilogues' store pattern in three tile orders")
    ap.add_argument("--stage-probe", action="store_true",
                    help="only run the stage-loop probe of the wide GEMM engine (libmoe_probe.so)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH", "WRITE", "COPYF", "COPYW"),
                    help="write profiles/traffic.json (with --train-tokens: traffic_train.json) "
                         "from rocprofv3 --pmc output directories")
    args = ap.parse_args()
    if args.pmc_summary:
        from dropless_grouped_gemm_router_amd.inputs import WORKLOADS
        if args.train_tokens:
            name = WORKLOADS[4][0].replace("16384 tok", f"{args.train_tokens} tok")
            pmc_summary(*args.pmc_summary, name, TRAFFIC_TRAIN_FILE)
        else:
            pmc_summary(*args.pmc_summary, WORKLOADS[args.workload][0], TRAFFIC_FILE)
        return
    if args.stage_probe:
        stage_probe()
        return
    if args.store_probe:
        store_probe()
        return
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
    if args.reference:
        for line in reference_rates(args.steps, args.warmup):
            print(json.dumps(line), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: libmoe has no multi-GPU path (--gpus {args.gpus} "
              "requested); the design notes describe how the path would shard.", file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import torch

    from dropless_grouped_gemm_router_amd import binding as B
    from dropless_grouped_gemm_router_amd.inputs import WORKLOADS, capacity_for, make_inputs

    if args.maxtok:
        torch.cuda.set_device(0)
        print(json.dumps(maxtok_line(B, max(1, min(args.steps, 3)), 1)), flush=True)
        return
    if args.train_tokens:
        torch.cuda.set_device(0)
        print(json.dumps({"train_step": train_step_line(B, max(3, min(args.steps, 20)),
                                                        max(2, args.warmup), args.train_tokens,
                                                        pages=not args.no_pages)}),
              flush=True)
        return

    name, p, _ = WORKLOADS[args.workload]
    if args.block_m:
        p = dataclasses.replace(p, block_m=args.block_m)
    if args.skew:
        p = dataclasses.replace(p, skew=args.skew)
    if args.capacity_factor:
        p = dataclasses.replace(p, capacity=capacity_for(p, args.capacity_factor))
    torch.cuda.set_device(0)
    print(f"bench: {name} bm={p.block_m}: generating inputs", file=sys.stderr, flush=True)
    inputs = make_inputs(p, seed=0)
    dev = B.device_inputs(inputs, "cuda:0")
    buf = B.allocate(p, "cuda:0", dispatch=args.dispatch)
    x = dev.pop("x")
    w = dev
    side = torch.cuda.Stream()  # the shared expert runs there beside the routed path
    torch.cuda.synchronize()

    def step():
        B.forward_dispatch(p, args.dispatch, x, w, buf, side_stream=side)

    def staged_step():
        # the same kernels one after another on one stream
        B.forward(p, x, w, buf)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timed = step
    if args.graph:
        # One step captured in a HIP graph (the side-stream fork and join
        # included), replayed as the timed step.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        timed = graph.replay
        for _ in range(args.warmup):
            timed()
        torch.cuda.synchronize()
    print(f"bench: warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)
    ms = time_steps(timed, args.steps, 0)
    pages = None
    if not args.no_pages:
        print("bench: pages' timing protocol", file=sys.stderr, flush=True)
        pages = pages_timing(timed, ms)
    # Per-kernel times: libmoe's HIP events bracket every launch. In the
    # timed steps the shared expert runs beside the routed path on a second
    # stream, so kernel durations there include time shared with other
    # kernels; each kernel's own duration comes from a pass of the staged
    # calls (gather dispatch: the same kernels, serialised).
    serial = args.dispatch == "gather"
    B.moe_trace_enable(True)
    ms_serial = time_steps(staged_step if serial else step, args.steps, 0)
    kern = B.moe_trace_summary()
    B.moe_trace_enable(False)

    wk = work(p, args.dispatch)
    per_step = {k: v["ms"] / args.steps for k, v in kern.items()}
    avg = {k: v["ms"] / v["count"] for k, v in kern.items()}
    dom = max(per_step, key=per_step.get)
    rooflines = {k: roofline_of(k, wk[k][0], wk[k][1], avg[k], p.dtype) for k in wk if k in avg}
    roof = dict(rooflines[dom]) if dom in rooflines else None
    if roof is not None:
        ent = load_traffic(TRAFFIC_FILE, name).get(dom)
        roof["traffic"] = ent["bytes_per_launch"] if ent else None
    peak = PEAK_TFLOPS[p.dtype]
    routed_ms = sum(avg[k] for k in ("gemm_gate_up", "gemm_down") if k in avg)
    routed_fl = wk["gemm_gate_up"][0] + wk["gemm_down"][0]
    total_fl = sum(wk[k][0] for k in avg if k in wk)
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
        "data": ("synthetic: seeded N(0,1) tokens, N(0,1/fan_in) weights, "
                 + ("unskewed random router" if not p.skew else f"router skew {p.skew}")),
        "config": {"workload": name, "tokens": p.tokens, "experts": p.experts, "top_k": p.top_k,
                   "d_model": p.d_model, "d_hidden": p.d_hidden, "d_shared": p.d_shared,
                   "block_m": p.block_m, "skew": p.skew, "dispatch": args.dispatch,
                   "routing": "capacity" if p.capacity else "dropless", "capacity": p.capacity,
                   "hip_graph": bool(args.graph)},
        "pages_timing": (dict(pages, tokens_per_s_median=p.tokens / (pages["median_ms"] * 1e-3))
                         if pages else None),
        "tflops": total_fl / (ms * 1e-3) / 1e12,
        "grouped_gemm_pct_mfma_peak": 100.0 * routed_fl / (routed_ms * 1e-3) / 1e12 / peak,
        "roofline": roof,
        "kernel_timing": ("serial pass of the staged calls after the timed steps "
                          f"({ms_serial:.3f} ms per step serialised)" if serial else
                          "traced pass of the same calls after the timed steps"),
        "kernels_ms_per_step": {k: round(v, 5) for k, v in sorted(per_step.items())},
        "kernel_rooflines": {k: {"frac": round(r["frac"], 4), "achieved": round(r["achieved"], 1),
                                 "unit": r["unit"], "bound": r["bound"]}
                             for k, r in rooflines.items()},
    }
    # (skipped with --no-pages, the short runs under a profiler)
    if p.dtype == "bf16" and not args.no_pages:
        print("bench: MFMA ceiling probe", file=sys.stderr, flush=True)
        line["mfma_ceiling"] = mfma_ceiling()
    if not args.no_train:
        print("bench: train step", file=sys.stderr, flush=True)
        line["train_step"] = train_step_line(B, max(5, args.steps // 5), 3, pages=not args.no_pages)
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(p, inputs, min(args.cpu_sample, p.tokens))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
