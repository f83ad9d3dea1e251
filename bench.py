#!/usr/bin/env python3
"""Benchmark of the sparse lightning-indexer KL-loss backward on one MI355X.

One step = the whole hot path over one batch of synthetic input: the
load-balancing metadata pre-pass, the accumulator fill, the fused backward
kernel and the dK finalisation (dq, dk, dw and softmax_out all produced).
Inputs are resident in HBM before the timed region starts.

Default workload: the DeepSeek-V3.2-shaped indexer (BSND B=1, S1=S2=4096,
N1=64, N2=1, D=128, topk=2048, bf16, causal indices).

Prints one JSON line.  Fields beyond the common contract:
  roofline      the fused kernel against the bf16 dense MFMA peak; `achieved`
                is the nominal 6*N1*D*topk FLOP per query token times the
                tokens of one launch, divided by the launch window measured
                with HIP events on the launch stream (window = accumulator
                fill + fused kernel + dK finalisation);
  cpu_baseline  the fp64 oracle on a bounded row sample, on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query tokens/sec at N1=64 D=128 topk=2048 bf16; % of MFMA bf16 peak"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv32_indexer")
    ap.add_argument("--deterministic", type=int, default=None, help="override the workload's mode")
    ap.add_argument("--cpu-rows", type=int, default=1024, help="oracle sample size (rows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def cpu_baseline(x, n_rows):
    import numpy as np
    from oracle import slikl_grad_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:       # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    stride = max(1, x.t1 // max(1, n_rows))
    rows = np.arange(0, x.t1, stride)[:n_rows]
    t0 = time.perf_counter()
    slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                   cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(rows)} query rows (every {stride}th row) of the same workload, "
                      f"fp64 NumPy oracle, {dt:.1f} s wall"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        return 2

    import numpy as np
    import torch

    import sparse_attention_indexer_token_amd as slikl
    from workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 2
    slikl.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = WORKLOADS[args.workload]
    det = wl.deterministic if args.deterministic is None else bool(args.deterministic)
    x = make_inputs(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16

    def b16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

    q, k = b16(x.q_bits), b16(x.k_bits)
    w = torch.from_numpy(x.w).to(dev)
    idx = torch.from_numpy(x.idx).to(dev)
    p = torch.from_numpy(x.p).to(dev)
    cu_q = None if x.cu_q is None else torch.from_numpy(x.cu_q).to(dev)
    cu_k = None if x.cu_k is None else torch.from_numpy(x.cu_k).to(dev)
    kw = dict(layout_q=x.layout_q, layout_k=x.layout_k, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
              deterministic=det)
    desc = slikl.make_desc(q, k, idx, **kw)
    ws = torch.empty(slikl.slikl_grad_workspace_size(desc), dtype=torch.uint8, device=dev)
    md = torch.empty(slikl.METADATA_INTS, dtype=torch.int32, device=dev)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(w), torch.empty_like(p))
    stream = torch.cuda.current_stream(dev)

    def step(ev0=None, ev1=None):
        slikl.slikl_grad_metadata(q, k, idx, metadata=md, workspace=ws, **kw)
        if ev0 is not None:
            ev0.record(stream)
        slikl.slikl_grad(q, k, w, idx, p, metadata=md, workspace=ws, out=out, **kw)
        if ev1 is not None:
            ev1.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for e0, e1 in evs:
        step(e0, e1)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    win_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))

    T1 = x.t1
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T1 * args.steps / elapsed
    flop_nominal = 6.0 * wl.n1 * wl.d * wl.topk * T1
    flop_valid = 6.0 * (wl.n1 // wl.n2) * wl.d * x.valid_slots
    achieved = flop_nominal / (win_ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded generators, shapes of the workload)",
        "config": {"workload": wl.name, "layout": wl.layout, "batch": x.batch, "T1": T1,
                   "T2": x.t2, "N1": wl.n1, "N2": wl.n2, "D": wl.d, "topk": wl.topk,
                   "valid_slots": x.valid_slots, "deterministic": det},
        "tflops_nominal_step": flop_nominal / (ms_per_step * 1e-3) / 1e12,
        "tflops_valid_step": flop_valid / (ms_per_step * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": None,
                     "kernel": "grad_fused_kernel", "window_ms": win_ms},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(x, args.cpu_rows)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
