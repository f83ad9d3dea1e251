"""Benchmark of the sparse lightning-indexer KL-loss backward on one MI355X.

One step = the whole hot path over one batch of synthetic input: the
load-balancing metadata pre-pass and slikl_grad (accumulator / record fills,
fp16 key copy, the fused S / softmax / dI / dW / dq kernel, the dK kernel and
its finalisation): dq, dk, dw and softmax_out are all produced.  Inputs are
resident in HBM before the timed region starts.

Default workload: the DeepSeek-V3.2-shaped indexer (BSND B=1, S1=S2=4096,
N1=64, N2=1, D=128, topk=2048, bf16, causal indices).

Prints one JSON line.  Fields beyond the common contract:
  roofline      the dominant kernel (the phase that takes longest) against its own
                bound: the fused kernel and the dense dK kernel against the bf16 /
                fp16 dense MFMA peak, the sorted strategy's parts and per-key sum
                kernels against HBM.  `achieved` = the kernel's algorithmic work per
                launch (FLOP of the method's contractions over the valid slots, or
                the bytes each input and output needs once) / its average launch
                time, measured with HIP events recorded on the launch stream
                (slikl_grad_profiled).  `traffic` = HBM bytes per launch from
                rocprofv3 FETCH_SIZE / WRITE_SIZE counters kept under profiles/,
                scaled by the same counters read for a plain copy of known size;
                null when the kernel source changed since the counters were taken.
  rooflines     the same for every timed phase.
  step_bound    the whole step against the workload's own bound: nominal MFMA
                FLOP (6 N1 D topk per query token), HBM on the compulsory bytes,
                the K gather and the dK scatter rates.
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
HEADLINE = "dsv32_indexer"          # the workload METRIC is quoted on
# MI355X published peaks: dense bf16 / fp16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz) and
# HBM3E bandwidth
PEAK_MFMA_TFLOPS = 2516.6
PEAK_HBM_GBPS = 8000.0
CSRC = os.path.join(ROOT, "sparse_attention_indexer_token_amd", "csrc")
# sources each kernel is compiled from (a change to any voids its traffic figure)
_COMMON = ("device_common.h", "slikl_internal.h")
KERNEL_SOURCES = {
    kern: [os.path.join(CSRC, f) for f in (src,) + _COMMON]
    for kern, src in (("grad_dense64_kernel", "grad_dense64.hip"), ("grad_dense_kernel", "grad_dense.hip"),
                      ("grad_fused_kernel", "grad_fused.hip"), ("dense_dk_kernel", "dense_dk.hip"),
                      ("scatter_dk_kernel", "scatter_dk.hip"), ("sorted_reduce_kernel", "sorted_dk.hip"))
}


def metric_for(wl):
    if wl.name == HEADLINE:
        return METRIC
    return (f"query tokens/sec at N1={wl.n1} D={wl.d} topk={wl.topk} {wl.dtype} ({wl.name}); "
            f"% of MFMA {wl.dtype} peak")


def traffic_file(kernel, workload):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")


def fused_kernel(strategy, group):
    """The fused kernel a call runs: with the dense and sorted dK strategies the
    64-head kernel for head groups padded to at most 64 heads, the 128-head one
    above; with the scatter strategy its own four-wave kernel (which also forms and
    adds the dK parts)."""
    if strategy == "scatter":
        return "grad_fused_kernel"
    return "grad_dense64_kernel" if group <= 64 else "grad_dense_kernel"


# the library's parts format: 16-bit rows when no key row takes more than this many
# parts, fp32 rows otherwise (the same threshold as the library's)
PARTS_I16_MAX_REFS = 1024


def max_key_refs(x):
    """Most valid slots naming one key row (per key head) of the workload."""
    import numpy as np
    n2 = x.idx.shape[-2]
    flat = x.idx.reshape(-1, n2, x.idx.shape[-1])
    if x.layout_q == "BSND":
        rows_b = np.repeat(np.arange(x.batch), flat.shape[0] // x.batch)
    else:
        rows_b = np.repeat(np.arange(x.batch), np.diff(x.cu_q))
    if x.layout_k == "BSND":
        kbase = np.arange(x.batch) * x.k.shape[1]
    else:
        kbase = np.asarray(x.cu_k[:-1])
    best = 0
    for g in range(n2):
        ids = flat[:, g, :]
        keys = (ids + kbase[rows_b][:, None])[ids >= 0]
        if keys.size:
            best = max(best, int(np.bincount(keys).max()))
    return best


def phase_work(strategy, wl, x, det):
    """Algorithmic work of each timed phase's kernel per launch:
    {phase: (kernel, bound, amount, unit)} with amount in FLOP ("mfma") or HBM bytes
    ("hbm").  V = valid (unit, slot) pairs, G = N1 / N2 heads per unit."""
    G = wl.n1 // wl.n2
    V = x.valid_slots
    D = wl.d
    U = x.t1 * wl.n2
    nh = max(1, (32 if G <= 32 else 64 if G <= 64 else 128) // 32)
    acc_elem = 8 if det else 4          # int64 fixed point when deterministic
    work = {}
    if strategy == "scatter":
        # S, dq and the dK parts: three G x D contractions per valid slot
        work["fused"] = ("grad_fused_kernel", "mfma", 6.0 * G * D * V, "FLOP")
        work["dk_final"] = ("finalize_kernel", "hbm", x.t2 * wl.n2 * D * (acc_elem + 2.0), "B")
    else:
        # S and dq (U = K^T dS^T): two G x D contractions per valid slot
        work["fused"] = (fused_kernel(strategy, G), "mfma", 4.0 * G * D * V, "FLOP")
    if strategy == "dense":
        # the method's dK contraction dS^T q: one G x D contraction per valid slot
        work["dk"] = ("dense_dk_kernel", "mfma", 2.0 * G * D * V, "FLOP")
    if strategy == "sorted":
        # each valid slot's part written once (16-bit elements carrying their exponent,
        # or fp32), with its record (key, dI, head words) read; q read once
        eb = 2.0 if max_key_refs(x) <= PARTS_I16_MAX_REFS else 4.0
        work["dk"] = ("scatter_dk_kernel", "hbm", V * (eb * D + 8 + 4 * nh) + x.t1 * wl.n1 * D * 2.0, "B")
        # the parts and the sorted list read once, the fp32 accumulator written once
        work["dk_reduce"] = ("sorted_reduce_kernel", "hbm", V * (eb * D + 4) + x.t2 * wl.n2 * D * 4.0, "B")
        work["dk_final"] = ("finalize_kernel", "hbm", x.t2 * wl.n2 * D * (acc_elem + 2.0), "B")
    return work


def compulsory_bytes(wl, x):
    """Bytes every step must move to and from HBM: q in and dq out, w and dw, the
    indices, p and softmax_out, k in and dk out (each once)."""
    e16 = 2.0
    return (x.t1 * wl.n1 * wl.d * e16 * 2 + x.t1 * wl.n1 * 4.0 * 2 + x.t1 * wl.n2 * wl.topk * 4.0 * 3
            + x.t2 * wl.n2 * wl.d * e16 * 2)


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
    ap.add_argument("--attn-p-lse", action="store_true",
                    help="p producer workloads: give each head's log-sum-exp (one pass over the keys)")
    return ap.parse_args()


def host_threads():
    """(cores this process may run on, BLAS threads of the NumPy oracle)."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:       # threadpoolctl missing: the BLAS count is unknown
        blas = None
    return cores, blas


def cpu_baseline(x, n_rows):
    import numpy as np
    from oracle import slikl_grad_ref
    cores, blas = host_threads()
    stride = max(1, x.t1 // max(1, n_rows))
    rows = np.arange(0, x.t1, stride)[:n_rows]
    t0 = time.perf_counter()
    slikl_grad_ref(x.q, x.k, x.w, x.idx, x.p, layout_q=x.layout_q, layout_k=x.layout_k,
                   cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k, rows=rows)
    dt = time.perf_counter() - t0
    which = f"all {len(rows)} query rows" if stride == 1 else f"{len(rows)} query rows (every {stride}th row)"
    # the oracle loops over units in Python and calls BLAS per unit: the BLAS threads
    # are the threads it uses
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": int(blas or cores), "kind": "oracle",
            "affinity_cores": cores, "blas_threads": blas,
            "sample": f"{which} of the same workload, fp64 NumPy oracle, {dt:.1f} s wall"}


def run_attn_p(args, wl_name):
    """Bench of the p producer (slikl_attn_softmax_l1norm) on a main-attention workload:
    one step = one call over all query rows.  Without lse the call makes two passes over
    the keys (the heads' log-sum-exp over the slots, then p); with --attn-p-lse it is
    given (computed beforehand with torch in fp32) and one pass runs."""
    import numpy as np
    import torch
    import sparse_attention_indexer_token_amd as slikl
    from workloads import ATTN_P_WORKLOADS, make_attn_p_inputs

    slikl.load()
    dev = torch.device("cuda:0")
    wl = ATTN_P_WORKLOADS[wl_name]
    x = make_attn_p_inputs(wl)
    tdt = torch.bfloat16 if wl.index.dtype == "bf16" else torch.float16

    def b16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

    qm, km = b16(x.qm_bits), b16(x.km_bits)
    idx = torch.from_numpy(np.ascontiguousarray(x.idx)).to(dev)
    nm, dm = x.qm.shape[-2:]
    n2, topk = x.idx.shape[-2:]
    lse = None
    if args.attn_p_lse:
        # each head's log-sum-exp over its unit's valid slots, in fp32 with torch
        qf = qm.reshape(-1, nm, dm)
        kf = km.reshape(-1, n2, dm)
        idf = idx.reshape(-1, n2, topk).long()
        if x.layout_q != "BSND":
            raise SystemExit("--attn-p-lse is built for BSND workloads")
        # key base of each query row's batch
        base = (torch.arange(qf.shape[0], device=dev) // x.idx.shape[1]) * km.shape[1]
        lse = torch.empty(qf.shape[0], nm, dtype=torch.float32, device=dev)
        hm = nm // n2
        for r0 in range(0, qf.shape[0], 128):
            r1 = min(qf.shape[0], r0 + 128)
            for g in range(n2):
                ids = idf[r0:r1, g]
                valid = ids >= 0
                rows = (ids.clamp(min=0) + base[r0:r1, None])
                ksel = kf[rows, g].float().contiguous()                     # [R, topk, dm]
                qsel = qf[r0:r1, g * hm:(g + 1) * hm].float().contiguous()  # [R, hm, dm]
                z = torch.bmm(qsel, ksel.transpose(1, 2).contiguous()) * wl.scale
                z = z.masked_fill(~valid[:, None, :], float("-inf"))
                lse[r0:r1, g * hm:(g + 1) * hm] = torch.logsumexp(z, dim=-1)
        lse = lse.reshape(x.qm.shape[:-1]).contiguous()
    out = torch.empty(idx.shape, dtype=torch.float32, device=dev)
    kw = dict(lse=lse, out=out, layout_q=x.layout_q, layout_k=x.layout_k)

    def step():
        slikl.slikl_attn_softmax_l1norm(qm, km, idx, wl.scale, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = elapsed * 1e3 / args.steps
    passes = 1 if lse is not None else 2
    hm = nm // n2
    flop = passes * 2.0 * hm * dm * x.valid_slots
    ach = flop / (kernel_ms * 1e-3) / 1e12
    res = {
        "metric": f"query tokens/sec of the p producer (attnSoftmaxL1Norm) at Nm={nm} Dm={dm} topk={topk} "
                  f"{wl.index.dtype}; % of MFMA {wl.index.dtype} peak",
        "value": x.t1 * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.index.dtype,
        "data": "synthetic (seeded generators with the workload's shapes and value recipes)",
        "config": {"workload": wl.name, "layout": x.layout_q, "T1": x.t1, "Nm": nm, "N2": n2, "Dm": dm,
                   "topk": topk, "valid_slots": x.valid_slots, "lse_given": lse is not None, "passes": passes},
        # one kernel per step: the events bracket the timed steps on the launch stream
        "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / PEAK_MFMA_TFLOPS, "traffic": None, "kernel": "attn_p_kernel",
                     "kernel_ms": kernel_ms, "flop_per_launch": flop},
    }
    if not args.no_cpu_baseline:
        from oracle import attn_softmax_l1norm_ref
        # about 10 s of oracle work: each row is Nm x Dm x topk fp64 products
        n = max(1, min(x.t1, args.cpu_rows // 2))
        rows = np.arange(0, x.t1, max(1, x.t1 // n))[:n]
        cores, blas = host_threads()
        t0 = time.perf_counter()
        attn_softmax_l1norm_ref(x.qm, x.km, x.idx, scale=wl.scale, layout_q=x.layout_q, layout_k=x.layout_k,
                                cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k, rows=rows)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": len(rows) / dt, "unit": "tokens/s", "cores": int(blas or cores),
                               "kind": "oracle", "affinity_cores": cores, "blas_threads": blas,
                               "sample": f"{len(rows)} query rows (evenly spaced) of the same workload, fp64 "
                                         f"NumPy oracle of p, {dt:.1f} s wall"}
    print(json.dumps(res), flush=True)
    return 0


def run_dense(args, wl_name):
    """Bench of the dense sibling operator (slikl_dense_grad): one step = the dense
    pre-pass (index lists and metadata) and the call, all outputs produced."""
    import types
    import numpy as np
    import torch
    import sparse_attention_indexer_token_amd as slikl
    from workloads import DENSE_WORKLOADS, make_dense_inputs

    slikl.load()
    dev = torch.device("cuda:0")
    wl, mask = DENSE_WORKLOADS[wl_name]
    det = wl.deterministic if args.deterministic is None else bool(args.deterministic)
    x = make_dense_inputs(wl, mask)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16

    def b16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

    q, k = b16(x.q_bits), b16(x.k_bits)
    w = torch.from_numpy(np.ascontiguousarray(x.w)).to(dev)
    p = torch.from_numpy(np.ascontiguousarray(x.p)).to(dev)
    kw = dict(mask_mode=mask, deterministic=det, dk_mode=args.dk_mode, layout_q=x.layout_q, layout_k=x.layout_k)
    desc = slikl.make_dense_desc(q, k, p, **kw)
    ws = torch.empty(slikl.slikl_dense_grad_workspace_size(desc), dtype=torch.uint8, device=dev)
    md = torch.empty(slikl.METADATA_INTS, dtype=torch.int32, device=dev)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(w), torch.empty_like(p))
    sdesc = desc.base
    sdesc.topk = p.shape[-1]
    strategy = slikl.slikl_grad_dk_strategy(sdesc)

    def step():
        slikl.slikl_dense_grad_metadata(q, k, p, metadata=md, workspace=ws, **kw)
        slikl.slikl_dense_grad(q, k, w, p, metadata=md, workspace=ws, out=out, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    phases = [slikl.slikl_dense_grad_profiled(q, k, w, p, metadata=md, workspace=ws, out=out, **kw)[1]
              for _ in range(max(1, args.profiled_calls))]
    phase_ms = {name: float(np.mean([ph[name] for ph in phases])) for name in phases[0]}
    V = x.visible // 1
    xs = types.SimpleNamespace(t1=x.t1, t2=int(np.prod(x.k.shape[:-2])), valid_slots=V)
    rooflines = {}
    for phase, (kern, bound, amount, unit) in phase_work(strategy, wl, xs, det).items():
        ms = phase_ms.get(phase, 0.0)
        if ms <= 0:
            continue
        if bound == "mfma":
            ach, peak, u = amount / (ms * 1e-3) / 1e12, PEAK_MFMA_TFLOPS, "TFLOP/s"
        else:
            ach, peak, u = amount / (ms * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"
        rooflines[phase] = {"bound": bound, "achieved": ach, "peak": peak, "unit": u, "frac": ach / peak,
                            "kernel": kern, "kernel_ms": ms,
                            ("flop_per_launch" if bound == "mfma" else "bytes_per_launch"): amount}
    dom = max(rooflines, key=lambda ph: rooflines[ph]["kernel_ms"])
    ms_per_step = elapsed * 1e3 / args.steps
    G = wl.n1 // wl.n2
    flop_valid = 6.0 * G * wl.d * V
    res = {
        "metric": f"query tokens/sec of the dense operator (maskMode {mask}) at N1={wl.n1} D={wl.d} "
                  f"S2={x.k.shape[1] if x.layout_k == 'BSND' else x.max_seqlen_k} {wl.dtype}; % of MFMA {wl.dtype} peak",
        "value": x.t1 * args.steps / elapsed,
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
        "config": {"workload": wl_name, "layout": x.layout_q, "batch": x.batch, "T1": x.t1, "N1": wl.n1,
                   "N2": wl.n2, "D": wl.d, "mask_mode": mask, "visible_pairs": V, "deterministic": det,
                   "dk_strategy": strategy},
        "tflops_valid_step": flop_valid / (ms_per_step * 1e-3) / 1e12,
        "roofline": dict(rooflines[dom], traffic=None),
        "rooflines": rooflines,
        "phases_ms": phase_ms,
    }
    if not args.no_cpu_baseline:
        from oracle import dense_grad_ref
        n = max(1, min(x.t1, args.cpu_rows))
        rows = np.arange(0, x.t1, max(1, x.t1 // n))[:n]
        cores, blas = host_threads()
        t0 = time.perf_counter()
        dense_grad_ref(x.q, x.k, x.w, x.p, mask_mode=mask, layout_q=x.layout_q, layout_k=x.layout_k,
                       cu_seqlens_q=x.cu_q, cu_seqlens_k=x.cu_k, rows=rows)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": len(rows) / dt, "unit": "tokens/s", "cores": int(blas or cores),
                               "kind": "oracle", "affinity_cores": cores, "blas_threads": blas,
                               "sample": f"{len(rows)} query rows (evenly spaced) of the same workload, fp64 "
                                         f"NumPy oracle of the dense operator, {dt:.1f} s wall"}
    print(json.dumps(res), flush=True)
    return 0


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
    from workloads import ATTN_P_WORKLOADS, DENSE_WORKLOADS, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 2
    slikl.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in ATTN_P_WORKLOADS:
        return run_attn_p(args, args.workload)
    if args.workload in DENSE_WORKLOADS:
        return run_dense(args, args.workload)

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
    ms_per_step = elapsed * 1e3 / args.steps
    t_step = ms_per_step * 1e-3
    tokens_per_s = T1 * args.steps / elapsed
    flop_nominal = 6.0 * wl.n1 * wl.d * wl.topk * T1
    flop_valid = 6.0 * G * wl.d * x.valid_slots

    # per-phase rooflines (HIP events on the launch stream, the phases' average over the
    # profiled calls); the dominant kernel is the phase that takes longest
    rooflines = {}
    for phase, (kern, bound, amount, unit) in phase_work(strategy, wl, x, det).items():
        ms = phase_ms.get(phase, 0.0)
        if ms <= 0:
            continue
        if bound == "mfma":
            ach, peak, u = amount / (ms * 1e-3) / 1e12, PEAK_MFMA_TFLOPS, "TFLOP/s"
        else:
            ach, peak, u = amount / (ms * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"
        rooflines[phase] = {"bound": bound, "achieved": ach, "peak": peak, "unit": u, "frac": ach / peak,
                            "kernel": kern, "kernel_ms": ms,
                            ("flop_per_launch" if bound == "mfma" else "bytes_per_launch"): amount}
    dom = max(rooflines, key=lambda ph: rooflines[ph]["kernel_ms"])
    roof = dict(rooflines[dom])
    roof["traffic"] = traffic_bytes(roof["kernel"], wl.name)

    # the workload's own bound: MFMA on the nominal FLOP, HBM on the compulsory bytes,
    # the K gather (both passes read D 16-bit values per valid slot) and the dK scatter
    # (D fp32 adds per valid slot); in deterministic mode with the sorted or scatter
    # strategy also the parts' round trip (written and read once)
    comp = compulsory_bytes(wl, x)
    gather = 2.0 * x.valid_slots * wl.d * 2.0
    scatter = x.valid_slots * wl.d * 4.0
    dk_ms = sum(phase_ms.get(ph, 0.0) for ph in ("dk", "dk_prep", "dk_reduce", "dk_final"))
    step_bound = {
        "mfma_nominal_tflops": flop_nominal / t_step / 1e12,
        "mfma_frac_nominal": flop_nominal / t_step / 1e12 / PEAK_MFMA_TFLOPS,
        "hbm_compulsory_bytes": comp,
        "hbm_frac_compulsory": comp / t_step / 1e9 / PEAK_HBM_GBPS,
        "gather_bytes": gather,
        "gather_gbps_fused": gather / (phase_ms["fused"] * 1e-3) / 1e9 if phase_ms.get("fused") else None,
        "scatter_bytes": scatter,
        "scatter_gbps": scatter / ((phase_ms["fused"] if strategy == "scatter" else dk_ms) * 1e-3) / 1e9
        if (phase_ms.get("fused") if strategy == "scatter" else dk_ms) else None,
    }
    if det and strategy in ("sorted", "scatter"):
        eb = 2.0 if strategy == "sorted" and max_key_refs(x) <= PARTS_I16_MAX_REFS else 4.0
        parts = 2.0 * x.valid_slots * wl.d * eb
        step_bound["hbm_bytes_with_parts"] = comp + parts
        step_bound["hbm_frac_with_parts"] = (comp + parts) / t_step / 1e9 / PEAK_HBM_GBPS
    step_bound["bound"] = {"long_context": "gather", "contention_det": "hbm"}.get(wl.name, "mfma")
    res = {
        "metric": metric_for(wl),
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
        "tflops_nominal_step": flop_nominal / t_step / 1e12,
        "tflops_valid_step": flop_valid / t_step / 1e12,
        "frac_peak_nominal_step": flop_nominal / t_step / 1e12 / PEAK_MFMA_TFLOPS,
        "roofline": roof,
        "rooflines": rooflines,
        "step_bound": step_bound,
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
