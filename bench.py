"""Benchmark of the sparse lightning-indexer KL-loss backward on one MI355X.

One step = the whole hot path over one batch of synthetic input: the
load-balancing metadata pre-pass and slikl_grad (accumulator / record fills,
fp16 key copy, the fused S / softmax / dI / dW / dq kernel, the dK kernel and
its finalisation): dq, dk, dw and softmax_out are all produced.  Inputs are
resident in HBM before the timed region starts.

Default workload: the DeepSeek-V3.2-shaped indexer (BSND B=1, S1=S2=4096,
N1=64, N2=1, D=128, topk=2048, bf16, causal indices).

Prints one JSON line.  Fields beyond the common contract:
  roofline      the dominant kernel (the fused kernel) against the bf16 dense
                MFMA peak.  `achieved` = its algorithmic FLOP per launch (the S
                and dq contractions over the valid slots, 4 * N1 * D per valid
                slot and key head) / its average launch time, measured with HIP
                events recorded on the launch stream (slikl_grad_profiled).
                `traffic` = HBM bytes per launch from rocprofv3 FETCH_SIZE /
                WRITE_SIZE counters kept under profiles/, scaled by the same
                counters read for a plain copy of known size; null when the
                kernel source changed since the counters were taken.
  phases_ms     average per-phase milliseconds of the profiled calls.
  cpu_baseline  the fp64 oracle on a bounded row sample, on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query tokens/sec at N1=64 D=128 topk=2048 bf16; % of MFMA bf16 peak"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}
CSRC = os.path.join(ROOT, "sparse_attention_indexer_token_amd", "csrc")
# sources each fused kernel is compiled from (a change to any voids its traffic figure)
KERNEL_SOURCES = {
    kern: [os.path.join(CSRC, f) for f in (src, "device_common.h", "slikl_internal.h")]
    for kern, src in (("grad_dense8_kernel", "grad_dense8.hip"), ("grad_dense_kernel", "grad_dense.hip"),
                      ("grad_fused_kernel", "grad_fused.hip"))
}


def traffic_file(kernel, workload):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")


def fused_kernel(strategy, group):
    """The fused kernel a call runs: the eight-wave kernel for head groups padded to at
    most 64 heads (every strategy), above that the four-wave kernel of the dense
    strategy or of the scatter strategy."""
    if group <= 64:
        return "grad_dense8_kernel"
    return "grad_dense_kernel" if strategy == "dense" else "grad_fused_kernel"


def sources_sha256(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # steady state: the first calls run while the clocks ramp up (a few percent slower)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv32_indexer")
    ap.add_argument("--deterministic", type=int, default=None, help="override the workload's mode")
    ap.add_argument("--dk-mode", default="auto", choices=["auto", "scatter", "dense", "sorted"],
                    help="dK strategy (auto: the library's choice)")
    ap.add_argument("--kl-loss", action="store_true",
                    help="also write each unit's KL(p || softmax_out) (the loss terms)")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="oracle sample size (rows)")
    ap.add_argument("--profiled-calls", type=int, default=5, help="calls timed per phase")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
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
    which = f"all {len(rows)} query rows" if stride == 1 else f"{len(rows)} query rows (every {stride}th row)"
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{which} of the same workload, fp64 NumPy oracle, {dt:.1f} s wall"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        return 2

    import numpy as np
    import torch

    if args.copy_bytes > 0:
        # reference point for the HBM byte counters: one read and one write of a known size
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes}), flush=True)
        return 0

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
    # TND sides: the longest sequence is known on the host (it sizes the dense dK records)
    mx = lambda cu: int(np.diff(cu).max()) if cu is not None and len(cu) > 1 else 0
    kw = dict(layout_q=x.layout_q, layout_k=x.layout_k, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
              deterministic=det, max_seqlen_q=mx(x.cu_q) if x.layout_q == "TND" else 0,
              max_seqlen_k=mx(x.cu_k) if x.layout_k == "TND" else 0, dk_mode=args.dk_mode)
    desc = slikl.make_desc(q, k, idx, **kw)
    strategy = slikl.slikl_grad_dk_strategy(desc)
    ws = torch.empty(slikl.slikl_grad_workspace_size(desc), dtype=torch.uint8, device=dev)
    md = torch.empty(slikl.METADATA_INTS, dtype=torch.int32, device=dev)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(w), torch.empty_like(p))
    stream = torch.cuda.current_stream(dev)
    gkw = dict(kl_loss=torch.empty(p.shape[:-1], dtype=torch.float32, device=dev)) if args.kl_loss else {}

    def step():
        slikl.slikl_grad_metadata(q, k, idx, metadata=md, workspace=ws, **kw)
        slikl.slikl_grad(q, k, w, idx, p, metadata=md, workspace=ws, out=out, **kw, **gkw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0

    # per-phase times of the same call (HIP events on the launch stream), outside the
    # timed region
    phases = []
    for _ in range(max(1, args.profiled_calls)):
        _, ms = slikl.slikl_grad_profiled(q, k, w, idx, p, metadata=md, workspace=ws, out=out, **kw, **gkw)
        phases.append(ms)
    phase_ms = {name: float(np.mean([ph[name] for ph in phases])) for name in phases[0]}
    T1 = x.t1
    G = wl.n1 // wl.n2
    kernel = fused_kernel(strategy, G)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T1 * args.steps / elapsed
    flop_nominal = 6.0 * wl.n1 * wl.d * wl.topk * T1
    flop_valid = 6.0 * G * wl.d * x.valid_slots
    # the fused kernel's own arithmetic: S and dq over the valid slots
    flop_kernel = 4.0 * G * wl.d * x.valid_slots
    kernel_ms = phase_ms["fused"]
    achieved = flop_kernel / (kernel_ms * 1e-3) / 1e12
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
        "data": "synthetic (seeded generators with the workload's shapes and value recipes)",
        "config": {"workload": wl.name, "layout": wl.layout, "batch": x.batch, "T1": T1,
                   "T2": x.t2, "N1": wl.n1, "N2": wl.n2, "D": wl.d, "topk": wl.topk,
                   "valid_slots": x.valid_slots, "deterministic": det, "dk_strategy": strategy,
                   "kl_loss": bool(args.kl_loss)},
        "tflops_nominal_step": flop_nominal / (ms_per_step * 1e-3) / 1e12,
        "tflops_valid_step": flop_valid / (ms_per_step * 1e-3) / 1e12,
        "frac_peak_nominal_step": flop_nominal / (ms_per_step * 1e-3) / 1e12 / peak,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic_bytes(kernel, wl.name),
                     "kernel": kernel, "kernel_ms": kernel_ms, "flop_per_launch": flop_kernel},
        "phases_ms": phase_ms,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(x, args.cpu_rows)
    print(json.dumps(res), flush=True)
    return 0


def traffic_bytes(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on this workload and on the current kernel sources; else None."""
    try:
        text = open(traffic_file(kernel, workload)).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line and not line.startswith("#"))
    fields = {k_.strip(): v.strip() for k_, v in fields.items()}
    if fields.get("kernel") != kernel or fields.get("workload") != workload:
        return None
    if fields.get("sources_sha256") != sources_sha256(kernel):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


if __name__ == "__main__":
    sys.exit(main())
