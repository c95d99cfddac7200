"""Benchmark of the fused attention forward + backward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
attn_fwd, then the backward stages (pre-pass (fp32 only; the bf16 dQ kernel
does it), dQ, dK/dV, sink-gradient reduce).  Inputs are resident in HBM before the timed region.  Prints one JSON
line with whole-job effective TFLOP/s, counting only visible (query, key)
pairs: forward 2 * pairs * (d_qk + d_v), backward 2 * pairs * (3 d_qk + 2 d_v).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--case 0]
                       [--no-cpu-baseline] [--cpu-groups G]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_F32_VALU_TFLOPS = 157.3
METRIC = "fwd+bwd effective TFLOP/s (bf16 GQA+SWA, S=4096) and % of MFMA bf16 peak"


TRAFFIC_RECORDS = {2: os.path.join(ROOT, "profiles", "attn_gqa_swa_s4096_hbm_traffic.json")}


def kernel_source_hash():
    """sha256 over the HIP sources and the build script (names and bytes): the
    build script holds the compile flags, which change register allocation and
    so the kernels' traffic; counter records are tied to this hash."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "scaled_dot_product_15_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "scaled_dot_product_15_amd", "build.py"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(config, kernel):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE/WRITE_SIZE
    record (each counter scaled by its reading for a plain copy of known size),
    or None when there is no record or the kernels changed since it was taken."""
    path = TRAFFIC_RECORDS.get(config)
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["hbm_bytes_per_launch"]


def visible_pairs(S, L, causal, window_left, window_right):
    """Visible (query, key) pairs of one (batch, query head), in closed form:
    row i < L sees keys max(0, i - left) .. min(L - 1, i [causal], i + right)
    (windows inclusive, -1 unbounded), i.e. max(0, hi - lo + 1) keys."""
    import numpy as np
    L = max(0, min(int(L), int(S)))
    i = np.arange(L, dtype=np.int64)
    hi = np.full(L, L - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, i)
    if window_right >= 0:
        hi = np.minimum(hi, i + window_right)
    lo = np.maximum(0, i - window_left) if window_left >= 0 else np.zeros(L, dtype=np.int64)
    return int(np.maximum(0, hi - lo + 1).sum())


def effective_flops(pairs, d_qk, d_v):
    """Effective FLOPs of the metric, counted on visible pairs only: forward
    2 * pairs * (d_qk + d_v) (S = QK^T, O = PV); backward
    2 * pairs * (3 d_qk + 2 d_v) (S recomputed, dP = dO V^T, dV = P^T dO,
    dK = dS^T Q, dQ = dS K)."""
    return 2 * pairs * (d_qk + d_v), 2 * pairs * (3 * d_qk + 2 * d_v)


def kernel_flops_per_pair(d_qk, d_v):
    """Algorithmic MFMA FLOPs per visible pair of each kernel."""
    return {
        "fwd": 2 * (d_qk + d_v),                 # S = QK^T, O = PV
        "bwd_dkdv": 2 * (2 * d_qk + 2 * d_v),    # S, dP = dO V^T, dV = P^T dO, dK = dS^T Q
        "bwd_dq": 2 * (2 * d_qk + d_v),          # S, dP, dQ = dS K
    }


def workload_pairs(p, seqlens):
    """Visible pairs over all batches and query heads of workload p."""
    return sum(visible_pairs(p.S, p.S if seqlens is None else int(seqlens[b]), p.causal,
                             p.window[0], p.window[1]) for b in range(p.B)) * p.Hq


def cpu_baseline(p, arr, groups):
    """Time the float64 oracle on `groups` (batch, kv-head) groups of the workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    from scaled_dot_product_15_amd import inputs
    groups = min(groups, p.B * p.Hkv)
    nb = -(-groups // p.Hkv)  # batches the sample touches
    sub = {n: arr[n][:nb] for n in ("q", "k", "v", "do")}
    sub.update(alpha=arr["alpha"], seqlens=None if arr["seqlens"] is None else arr["seqlens"][:nb])
    t = inputs.to_torch(sub, p.dtype, "cpu")
    f64 = inputs.exact_f64
    q, k, v, do = f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"])
    seq = sub["seqlens"]
    t0 = time.perf_counter()
    pairs = 0
    for n in range(groups):
        b, g = n // p.Hkv, n % p.Hkv
        oracle.attention_group(q, k, v, do, b=b, g=g, num_gqa_groups=p.Hkv, causal=p.causal,
                               window=p.window, scale_factor=p.scale_factor or None,
                               softmax_type=p.softmax_type, softmax_offset=arr["alpha"],
                               seqlens=seq)
    dt = time.perf_counter() - t0
    for n in range(groups):
        b = n // p.Hkv
        L = p.S if seq is None else int(seq[b])
        pairs += visible_pairs(p.S, L, p.causal, p.window[0], p.window[1]) * (p.Hq // p.Hkv)
    ff, fb = effective_flops(pairs, p.d_qk, p.d_v)
    return {"value": (ff + fb) / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": dt,
            "sample": f"{groups} of {p.B * p.Hkv} (batch, kv-head) groups of the workload: "
                      f"{groups * (p.Hq // p.Hkv)} query heads x S={p.S}, fwd+bwd, numpy float64"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--case", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-groups", type=int, default=12)
    ap.add_argument("--layout", choices=("bshd", "thd"), default="bshd",
                    help="thd: the batch's sequences packed back to back at their valid lengths "
                         "(seq_offsets), no padding tokens stored")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="attention dropout rate (Philox keep mask regenerated in forward and backward)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (5 launches) to "
                         "calibrate the HBM byte counters, then exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the attention path here is single-GPU; no multi-GPU figure is produced.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4, "launches": 5}), flush=True)
        return

    from scaled_dot_product_15_amd import binding, inputs

    p = inputs.workload_configs()[args.config][args.case]
    seed = 1000 * args.config + args.case
    arr = inputs.draw(p, seed)
    dev = torch.cuda.get_device_properties(0)
    packed = args.layout == "thd"
    if packed:
        sizes = [p.S] * p.B if arr["seqlens"] is None else [int(x) for x in arr["seqlens"]]
        t = inputs.to_torch_packed(inputs.pack(arr, sizes), p.dtype, "cuda")
        t["seqlens"] = None  # every segment is exactly its valid tokens
    else:
        t = inputs.to_torch(arr, p.dtype, "cuda")

    kw = dict(num_gqa_groups=p.Hkv, attn_mask_type="causal" if p.causal else "no_mask",
              window_size=p.window, scale_factor=p.scale_factor or None,
              softmax_type=p.softmax_type, softmax_offset=t["alpha"], seqlens=t["seqlens"])
    if packed:
        kw.update(seq_offsets=t["seq_offsets"], max_seqlen=p.S)
    if args.dropout:
        kw.update(dropout_p=args.dropout, rng_state=(seed, 0))
    o, lse = binding.attn_fwd(t["q"], t["k"], t["v"], **kw)
    want = p.softmax_type != "vanilla"
    dq, dk, dv, doff = binding.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], want_d_offset=want, **kw)
    outs = (dq, dk, dv, doff)
    pp = binding.make_params(p.B, p.S, p.Hq, p.Hkv, p.d_qk, p.d_v, p.dtype, kw["attn_mask_type"],
                             p.window, kw["scale_factor"], p.softmax_type, args.dropout)
    ws = torch.empty(binding.attn_bwd_workspace_size(pp), dtype=torch.uint8, device="cuda")
    fast = dict(kw, check_seqlens=False)
    stream = torch.cuda.current_stream()
    # Backward stages (1..4) that launch a kernel for this workload: in bf16 the
    # pre-pass runs inside the dQ kernel, and the offset-gradient reduction
    # runs only when a softmax-offset gradient is requested.
    stages = [(s, n) for s, n in ((1, "bwd_pre"), (2, "bwd_dq"), (3, "bwd_dkdv"), (4, "bwd_offset"))
              if not (s == 1 and p.dtype == "bf16") and not (s == 4 and not want)]
    names = ["fwd"] + [n for _, n in stages]

    def step():
        binding.attn_fwd(t["q"], t["k"], t["v"], out=o, lse=lse, **fast)
        binding.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], want_d_offset=want, workspace=ws,
                         outs=outs, **fast)

    def staged_step(ev):
        """The same work with HIP events between the kernels (per-kernel times)."""
        ev[0].record(stream)
        binding.attn_fwd(t["q"], t["k"], t["v"], out=o, lse=lse, **fast)
        for i, (s, _) in enumerate(stages):
            ev[i + 1].record(stream)
            binding.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], want_d_offset=want, workspace=ws,
                             outs=outs, stage=s, **fast)
        ev[len(stages) + 1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Forward / backward split and per-kernel breakdown first: passes of the
    # same number of steps with HIP events on the launch stream.  They also
    # bring the GPU to its steady clock before the event-free timed loop.
    split = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for ev in split:
        ev[0].record(stream)
        binding.attn_fwd(t["q"], t["k"], t["v"], out=o, lse=lse, **fast)
        ev[1].record(stream)
        binding.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], want_d_offset=want, workspace=ws,
                         outs=outs, **fast)
        ev[2].record(stream)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        staged_step(events[i])
    torch.cuda.synchronize()
    # The timed region: exactly K steps, no events, synchronised on both sides.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    per = {n: [] for n in names}
    for ev in events:
        for s, n in enumerate(names):
            per[n].append(ev[s].elapsed_time(ev[s + 1]))
    avg_ms = {n: statistics.fmean(v) for n, v in per.items()}
    med_ms = {n: statistics.median(v) for n, v in per.items()}

    seq = arr["seqlens"]
    pairs = workload_pairs(p, seq)
    f_fwd, f_bwd = effective_flops(pairs, p.d_qk, p.d_v)
    ms_per_step = elapsed / args.steps * 1e3
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12
    t_fwd = statistics.median(ev[0].elapsed_time(ev[1]) for ev in split)
    t_bwd = statistics.median(ev[1].elapsed_time(ev[2]) for ev in split)

    kflops = kernel_flops_per_pair(p.d_qk, p.d_v)
    dominant = max(("fwd", "bwd_dkdv", "bwd_dq"), key=lambda n: avg_ms[n])
    achieved = kflops[dominant] * pairs / (avg_ms[dominant] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": (measured_traffic(args.config, dominant)
                            if args.case == 0 and not packed and not args.dropout else None),
                "flops_per_launch": kflops[dominant] * pairs, "avg_launch_ms": round(avg_ms[dominant], 4)}

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": p.name, "batch": p.B, "seq_len": p.S, "num_heads": p.Hq,
                   "num_gqa_groups": p.Hkv, "head_dim_qk": p.d_qk, "head_dim_v": p.d_v,
                   "mask": "causal" if p.causal else "none", "window": list(p.window),
                   "softmax_type": p.softmax_type, "seed": seed,
                   "seqlens": None if seq is None else [int(x) for x in seq], "layout": args.layout, "dropout": args.dropout,
                   "tokens": int(t["q"].shape[0]) if packed else p.B * p.S},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "pairs": pairs,
        "gflop_fwd": round(f_fwd / 1e9, 3),
        "gflop_bwd": round(f_bwd / 1e9, 3),
        "t_fwd_ms": round(t_fwd, 4),
        "t_bwd_ms": round(t_bwd, 4),
        "tflops_fwd": round(f_fwd / (t_fwd * 1e-3) / 1e12, 2),
        "tflops_bwd": round(f_bwd / (t_bwd * 1e-3) / 1e12, 2),
        "kernel_avg_ms": {n: round(v, 4) for n, v in avg_ms.items()},
        "kernel_median_ms": {n: round(v, 4) for n, v in med_ms.items()},
        "roofline": roofline,
        "device": {"name": dev.name, "compute_units": dev.multi_processor_count,
                   "gcn_arch": getattr(dev, "gcnArchName", "")},
        "context": "pages report only a ~52x fwd+bwd speedup of a fused call over a score-materialising "
                   "XLA baseline on one GB200 (no absolute figure)",
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(p, arr, args.cpu_groups)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
