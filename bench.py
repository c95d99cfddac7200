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
PEAK_FP8_TFLOPS = 5033.2    # dense fp8 MFMA: 256 CU x 2.4 GHz x 8192 FLOP/clk
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


def kernel_flops_per_pair(d_qk, d_v, stored_ds=False):
    """Algorithmic MFMA FLOPs per visible pair of each kernel (with stored dS
    the dQ kernel only contracts dS with K)."""
    return {
        "fwd": 2 * (d_qk + d_v),                 # S = QK^T, O = PV
        "bwd_dkdv": 2 * (2 * d_qk + 2 * d_v),    # S, dP = dO V^T, dV = P^T dO, dK = dS^T Q
        "bwd_dq": 2 * d_qk if stored_ds else 2 * (2 * d_qk + d_v),  # [S, dP,] dQ = dS K
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


def cpu_baseline_fp8(p, q8, k8, v8, do8, descales, s_ds, offsets, heads):
    """Time the float64 FP8 oracle, forward then backward, on `heads` query
    heads of the workload (each a sub-problem of that head and its K/V head)."""
    from oracle import fp8
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    G = p.Hq // p.Hkv
    heads = min(heads, p.B * p.Hq)
    kw = dict(num_gqa_groups=1, causal=p.causal, window=p.window, scale_factor=p.scale_factor or None,
              softmax_type=p.softmax_type)
    t0 = time.perf_counter()
    for n in range(heads):
        b, h = n // p.Hq, n % p.Hq
        g = h // G
        sub = dict(q8=q8[b:b + 1, :, h:h + 1], k8=k8[b:b + 1, :, g:g + 1], v8=v8[b:b + 1, :, g:g + 1],
                   do8=do8[b:b + 1, :, h:h + 1])
        off = None if offsets is None else offsets[h:h + 1]
        f = fp8.attention_fp8(sub["q8"], sub["k8"], sub["v8"], *descales[:3], softmax_offset=off, **kw)
        fp8.attention_fp8_bwd(sub["q8"], sub["k8"], sub["v8"], f["o"], sub["do8"], f["lse"], *descales, s_ds,
                              softmax_offset=off, **kw)
    dt = time.perf_counter() - t0
    pairs = visible_pairs(p.S, p.S, p.causal, p.window[0], p.window[1]) * heads
    ff, fb = effective_flops(pairs, p.d_qk, p.d_v)
    return {"value": (ff + fb) / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": dt,
            "sample": f"{heads} of {p.B * p.Hq} (batch, query head) pairs of the workload (S={p.S}), FP8 forward "
                      f"+ backward, numpy float64"}


def bench_fp8(args, p, arr, t, seed, dev, packed):
    """FP8 line: Q, K, V quantized to E4M3 and dO to E5M2 on the device (one
    delayed-scaling step sets each scale from its amax; the dS scale is the
    recipe's for E5M2 after one step on dS's amax), then a step of
    attn_fwd_fp8 + attn_bwd_fp8 timed with the codes resident in HBM.
    Effective FLOPs as the bf16 line's: forward 2 * pairs * (d_qk + d_v),
    backward 2 * pairs * (3 d_qk + 2 d_v)."""
    import numpy as np
    import torch
    from scaled_dot_product_15_amd import binding
    if p.d_qk != p.d_v or p.d_qk not in (64, 128) or args.dropout or args.bias != "none" or packed:
        print("the FP8 forward line runs head dims 64/128, bshd, without dropout or bias", file=sys.stderr)
        sys.exit(2)
    kw = dict(num_gqa_groups=p.Hkv, attn_mask_type="causal" if p.causal else "no_mask", window_size=p.window,
              scale_factor=p.scale_factor or None, softmax_type=p.softmax_type, softmax_offset=t["alpha"],
              seqlens=t["seqlens"])
    codes, descale, scales = [], [], []
    for name, fmt in (("q", "e4m3"), ("k", "e4m3"), ("v", "e4m3"), ("do", "e5m2")):
        hist = torch.zeros(1024, dtype=torch.float32, device="cuda")
        scale = torch.ones(1, dtype=torch.float32, device="cuda")
        dsc = torch.ones(1, dtype=torch.float32, device="cuda")
        _, amax = binding.fp8_quantize(t[name], scale, fmt)
        binding.fp8_update_scale(hist, amax, scale, dsc, fmt, margin=0)
        c, _ = binding.fp8_quantize(t[name], scale, fmt)
        codes.append(c)
        descale.append(dsc)
        scales.append(scale)
    q8, k8, v8, do8 = codes
    desc = torch.cat(descale[:3])
    desc4 = torch.cat(descale)
    o, lse = binding.attn_fwd_fp8(q8, k8, v8, desc, **kw)
    # dS scale: one recipe step on the amax of dS a first backward reports
    ds_scale = torch.ones(1, dtype=torch.float32, device="cuda")
    want = p.softmax_type != "vanilla"
    dq, dk, dv, doff, amax_ds = binding.attn_bwd_fp8(q8, k8, v8, o, do8, lse, desc4, ds_scale, want_d_offset=want,
                                                     **kw)
    binding.fp8_update_scale(torch.zeros(1024, dtype=torch.float32, device="cuda"), amax_ds, ds_scale,
                             torch.ones(1, dtype=torch.float32, device="cuda"), "e5m2", margin=0)
    pp = binding.make_params(p.B, p.S, p.Hq, p.Hkv, p.d_qk, p.d_v, "fp8", kw["attn_mask_type"], p.window,
                             kw["scale_factor"], p.softmax_type)
    ws = torch.empty(max(binding.attn_fwd_workspace_size(pp), 1), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(binding.attn_bwd_workspace_size(pp), 1), dtype=torch.uint8, device="cuda")
    fast = dict(kw, check_seqlens=False, out=o, lse=lse, workspace=ws)
    fastb = dict(kw, check_seqlens=False, outs=(dq, dk, dv, doff), amax=amax_ds, workspace=wsb, want_d_offset=want)
    stream = torch.cuda.current_stream()

    def step():
        binding.attn_fwd_fp8(q8, k8, v8, desc, **fast)
        binding.attn_bwd_fp8(q8, k8, v8, o, do8, lse, desc4, ds_scale, **fastb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in ev:
        e[0].record(stream)
        binding.attn_fwd_fp8(q8, k8, v8, desc, **fast)
        e[1].record(stream)
        binding.attn_bwd_fp8(q8, k8, v8, o, do8, lse, desc4, ds_scale, **fastb)
        e[2].record(stream)
    qev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    qev[0].record(stream)
    for name, c, sc, fmt in zip(("q", "k", "v", "do"), codes, scales, ("e4m3", "e4m3", "e4m3", "e5m2")):
        binding.fp8_quantize(t[name], sc, fmt, out=c)  # same scales: the codes are unchanged
    qev[1].record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in ev]
    avg = statistics.fmean(fwd_ms)
    seq = arr["seqlens"]
    pairs = workload_pairs(p, seq)
    f_fwd, f_bwd = effective_flops(pairs, p.d_qk, p.d_v)
    ms = elapsed / args.steps * 1e3
    value = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
    achieved = f_fwd / (avg * 1e-3) / 1e12
    t_bwd = statistics.median(bwd_ms)
    res = {
        "metric": "fwd+bwd effective TFLOP/s (FP8: E4M3 Q, K, V, P; E5M2 dO, dS) and % of MFMA fp8 peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3/e5m2", "data": "synthetic",
        "config": {"workload": p.name, "batch": p.B, "seq_len": p.S, "num_heads": p.Hq, "num_gqa_groups": p.Hkv,
                   "head_dim_qk": p.d_qk, "head_dim_v": p.d_v, "mask": "causal" if p.causal else "none",
                   "window": list(p.window), "softmax_type": p.softmax_type, "seed": seed,
                   "fp8": "E4M3 Q, K, V, P; E5M2 dO, dS",
                   "seqlens": None if seq is None else [int(x) for x in seq], "tokens": p.B * p.S},
        "pct_of_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "pairs": pairs, "gflop_fwd": round(f_fwd / 1e9, 3), "gflop_bwd": round(f_bwd / 1e9, 3),
        "t_fwd_ms": round(statistics.median(fwd_ms), 4), "t_bwd_ms": round(t_bwd, 4),
        "tflops_fwd": round(f_fwd / (statistics.median(fwd_ms) * 1e-3) / 1e12, 2),
        "tflops_bwd": round(f_bwd / (t_bwd * 1e-3) / 1e12, 2),
        "t_quantize_qkvdo_ms": round(qev[0].elapsed_time(qev[1]), 4),
        "roofline": {"bound": "mfma", "kernel": "fwd_fp8", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": f_fwd, "avg_launch_ms": round(avg, 4),
                     "note": "avg_launch_ms brackets the call: the V transpose kernel and the forward kernel"},
        "device": {"name": dev.name, "compute_units": dev.multi_processor_count,
                   "gcn_arch": getattr(dev, "gcnArchName", "")},
    }
    if not args.no_cpu_baseline:
        qc, kc, vc, dc = (c.cpu().numpy() for c in codes)
        res["cpu_baseline"] = cpu_baseline_fp8(p, qc, kc, vc, dc, [float(x) for x in desc4.cpu()],
                                               float(ds_scale.cpu()[0]), arr["alpha"].astype(np.float64),
                                               max(1, args.cpu_groups // 12))  # one head at the default
    print(json.dumps(res), flush=True)


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
    ap.add_argument("--bias", choices=("none", "full", "heads", "batch", "shared"), default="none",
                    help="additive post-scale attention bias [B|1, Hq|1, S, S] (bf16, N(0,1)) in forward and "
                         "backward, with its gradient")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 (E4M3) forward instead: Q, K, V quantized on the device with "
                         "delayed-scaling scales, then attn_fwd_fp8")
    ap.add_argument("--dq-path", choices=("default", "recompute", "stored-ds"), default="default",
                    help="backward path: the dQ kernel recomputes S and dP (smaller workspace), or computes "
                         "dQ from the dS the dK/dV kernel stores; default = the binding's choice "
                         "(binding.prefers_stored_ds)")
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
    if args.fp8:
        return bench_fp8(args, p, arr, t, seed, dev, packed)

    kw = dict(num_gqa_groups=p.Hkv, attn_mask_type="causal" if p.causal else "no_mask",
              window_size=p.window, scale_factor=p.scale_factor or None,
              softmax_type=p.softmax_type, softmax_offset=t["alpha"], seqlens=t["seqlens"])
    if packed:
        kw.update(seq_offsets=t["seq_offsets"], max_seqlen=p.S)
    if args.dropout:
        kw.update(dropout_p=args.dropout, rng_state=(seed, 0))
    bias_kw = {}
    if args.bias != "none":
        per_b, per_h = {"full": (1, 1), "heads": (0, 1), "batch": (1, 0), "shared": (0, 0)}[args.bias]
        gen = torch.Generator(device="cuda").manual_seed(seed)
        bias = torch.randn((p.B if per_b else 1, p.Hq if per_h else 1, p.S, p.S), generator=gen, device="cuda",
                           dtype=torch.float32).to(torch.bfloat16)
        kw.update(bias=bias)
    o, lse = binding.attn_fwd(t["q"], t["k"], t["v"], **kw)
    want = p.softmax_type != "vanilla"
    res = binding.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], want_d_offset=want, **kw)
    dq, dk, dv, doff = res[:4]
    if args.bias != "none":
        bias_kw = dict(d_bias=res[4])
    outs = (dq, dk, dv, doff)
    pp = binding.make_params(p.B, p.S, p.Hq, p.Hkv, p.d_qk, p.d_v, p.dtype, kw["attn_mask_type"],
                             p.window, kw["scale_factor"], p.softmax_type, args.dropout)
    # The workspace decides the backward's path: with room for the dS blocks
    # the dK/dV kernel stores dS and the dQ kernel contracts it with K.
    ds_size = binding.attn_bwd_ds_workspace_size(pp)
    stored_ds = ds_size > 0 and (args.dq_path == "stored-ds" or
                                 (args.dq_path == "default" and binding.prefers_stored_ds(pp, kw.get("bias"))))
    ws = torch.empty(ds_size if stored_ds else binding.attn_bwd_workspace_size(pp), dtype=torch.uint8,
                     device="cuda")
    fast = dict(kw, check_seqlens=False)
    stream = torch.cuda.current_stream()
    # Backward stages that launch a kernel for this workload, in the order the
    # one-call backward runs them: 1, 2, 3, 4, where in bf16 the pre-pass runs
    # inside the dQ kernel; with stored dS 1, 3, 2, 4.  The offset-gradient
    # reduction runs only when a softmax-offset gradient is requested.
    order = ((1, "bwd_pre"), (3, "bwd_dkdv"), (2, "bwd_dq"), (4, "bwd_offset")) if stored_ds else \
        ((1, "bwd_pre"), (2, "bwd_dq"), (3, "bwd_dkdv"), (4, "bwd_offset"))
    stages = [(s, n) for s, n in order
              if not (s == 1 and p.dtype == "bf16" and not stored_ds) and not (s == 4 and not want)]
    if args.bias != "none":
        stages = [(0, "bwd")]  # the biased backward runs as one call (dQ, dK/dV, dBias)
    names = ["fwd"] + [n for _, n in stages]

    def step():
        binding.attn_fwd(t["q"], t["k"], t["v"], out=o, lse=lse, **fast)
        binding.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], want_d_offset=want, workspace=ws,
                         outs=outs, **fast, **bias_kw)

    def staged_step(ev):
        """The same work with HIP events between the kernels (per-kernel times)."""
        ev[0].record(stream)
        binding.attn_fwd(t["q"], t["k"], t["v"], out=o, lse=lse, **fast)
        for i, (s, _) in enumerate(stages):
            ev[i + 1].record(stream)
            binding.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], want_d_offset=want, workspace=ws,
                             outs=outs, stage=s, **fast, **bias_kw)
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
                         outs=outs, **fast, **bias_kw)
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

    kflops = kernel_flops_per_pair(p.d_qk, p.d_v, stored_ds)
    # With a bias the backward is timed as one call; the roofline then covers
    # the forward, the one kernel its events bracket alone.
    dominant = max((n for n in ("fwd", "bwd_dkdv", "bwd_dq") if n in avg_ms), key=lambda n: avg_ms[n])
    achieved = kflops[dominant] * pairs / (avg_ms[dominant] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": (measured_traffic(args.config, dominant)
                            if args.case == 0 and not packed and not args.dropout and args.bias == "none"
                            else None),
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
                   "seqlens": None if seq is None else [int(x) for x in seq], "layout": args.layout,
                   "dropout": args.dropout, "bias": args.bias, "dq_from_stored_ds": stored_ds,
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
        res["cpu_baseline"]["gpu_over_cpu"] = round(value / res["cpu_baseline"]["value"], 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
