"""Float64 CPU oracle for FP8 attention (forward) and FP8 per-tensor scaling.

TEST INFRASTRUCTURE ONLY, like sdpa_oracle: only the test suite, the smoke
entry point and the benchmark's CPU-baseline leg may import it.  It shares no
code with the HIP path.

The codelab "Speed up attention on GPU with cuDNN and TransformerEngine",
section 10, runs attention under FP8 autocast with a DelayedScaling recipe:
HYBRID format (E4M3 for forward tensors, E5M2 for backward ones), an amax
history of 1024 steps and the "max" rule over that history.  The page shows
neither the formats' bit layouts nor the attention arithmetic under FP8, so
this module takes these readings (each also listed in the design notes):

  * formats: the two 8-bit formats of the OCP 8-bit floating point
    specification (OFP8): E4M3 (bias 7, no infinities, one NaN pattern per
    sign, largest finite 448) and E5M2 (bias 15, IEEE-like infinities and
    NaNs, largest finite 57344), both with subnormals.
  * rounding: a real value is encoded by round-to-nearest, ties to the even
    code; magnitudes beyond the largest finite value saturate to it
    (NaN stays NaN).
  * per-tensor scaling: a tensor x is stored as codes encode(x * scale) with a
    float32 scale; its real value is decode(code) * descale, descale = 1/scale.
  * delayed scaling: each step's amax = max |x| enters an amax history of a
    fixed length (newest first); the next scale is fmt_max / max(history) /
    2^margin while that max is positive and finite, else the old scale.
  * FP8 attention forward: Q, K, V are E4M3 codes with descales; scores
    s = scale * (dq Q8) . (dk K8); row max m_i and sum l_i of exp(s - m_i)
    over visible keys (plus the sink) as in sdpa_oracle; the probabilities
    relative to the row max are quantized to E4M3 as P8 = encode(256 exp(s -
    m_i)) (every value at most 256, below the E4M3 maximum; 256 a power of
    two, so the scaling adds no rounding); O_i = dv / (256 l_i) * sum_j P8_ij
    V8_j, LSE_i = m_i + ln l_i.  The normalisation uses the unquantized sum,
    so O is not exactly a convex combination: the quantization of P is part
    of the definition.
  * FP8 attention backward (HYBRID: the gradient entering the backward, dO,
    is E5M2): inputs Q8, K8, V8 (E4M3) with descales, dO8 (E5M2) with its
    descale, the forward's O (bf16 values) and LSE.  With P = exp(s - LSE) on
    visible pairs, delta_i = dO_i . O_i, dP = dO V^T and dS = P (dP - delta)
    computed from the dequantized values, the three gradient products take
    FP8 operands: dV = sum_i E4M3(256 P_ij) / 256 dO_i, and with dS quantized
    as dS8 = E5M2(s_ds dS) under a caller-given per-tensor scale s_ds (the
    recipe's delayed scale for dS; the call also returns this step's amax of
    dS), dK_j = scale / s_ds sum_i dS8_ij Q_i and dQ_i = scale / s_ds sum_j
    dS8_ij K_j (dK and dV summed over the query heads of the KV head's
    group).  The sink gradient is the bf16 path's, -sum_i exp(z - LSE_i)
    delta_i, per head over batches and rows.
"""
from __future__ import annotations

import math

import numpy as np

from .sdpa_oracle import kv_head, sink_logit, visible_mask, visible_rows

E4M3, E5M2 = "e4m3", "e5m2"
# (exponent bits, mantissa bits, exponent bias)
_FORMATS = {E4M3: (4, 3, 7), E5M2: (5, 2, 15)}


def fp8_decode(codes, fmt: str) -> np.ndarray:
    """Real value of each 8-bit code (float64), from the bit layout:
    sign | exponent | mantissa; exponent 0 = subnormal m * 2^(1 - bias - M).
    E4M3: exponent and mantissa all ones is NaN (no infinities).  E5M2:
    exponent all ones is infinity (mantissa 0) or NaN."""
    eb, mb, bias = _FORMATS[fmt]
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> mb) & ((1 << eb) - 1)
    m = c & ((1 << mb) - 1)
    frac = m / float(1 << mb)
    val = np.where(e == 0, frac * 2.0 ** (1 - bias), (1.0 + frac) * 2.0 ** (e - bias))
    emax = (1 << eb) - 1
    if fmt == E4M3:
        val = np.where((e == emax) & (m == (1 << mb) - 1), np.nan, val)
    else:
        val = np.where(e == emax, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


def fp8_max(fmt: str) -> float:
    """Largest finite value of the format."""
    return {E4M3: 448.0, E5M2: 57344.0}[fmt]


def _positive_table(fmt: str):
    codes = np.arange(128)
    vals = fp8_decode(codes, fmt)
    ok = np.isfinite(vals)
    return codes[ok], vals[ok]  # ascending, 0 first


def fp8_encode(x, fmt: str) -> np.ndarray:
    """uint8 codes of x: saturating round-to-nearest, ties to the even code."""
    x = np.asarray(x, dtype=np.float64)
    codes, vals = _positive_table(fmt)
    a = np.minimum(np.abs(x), fp8_max(fmt))
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    out = np.where(pick_hi, codes[hi], codes[lo])
    out = np.where(a == vals[hi], codes[hi], out)
    out = out | np.where(np.signbit(x), 0x80, 0)
    out = np.where(np.isnan(x), 0x7F, out)  # a NaN code of either format
    return out.astype(np.uint8)


def quantize(x, scale: float, fmt: str):
    """Per-tensor quantization: (codes of x * scale, amax = max |x|)."""
    x = np.asarray(x, dtype=np.float64)
    amax = float(np.abs(x).max()) if x.size else 0.0
    return fp8_encode(x * float(scale), fmt), amax


def delayed_scaling_update(history, new_amax: float, scale: float, fmt: str, margin: int = 0):
    """One step of the delayed-scaling recipe: the new amax enters the history
    (newest first, oldest dropped); the next scale is fmt_max / max(history) /
    2^margin when that max is positive and finite, else the old scale.
    Returns (history, scale, descale)."""
    h = np.concatenate([[float(new_amax)], np.asarray(history, dtype=np.float64)[:-1]])
    amax = float(h.max())
    if amax > 0.0 and math.isfinite(amax):
        scale = fp8_max(fmt) / amax / (2.0 ** margin)
    return h, float(scale), 1.0 / float(scale)


def attention_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, *, num_gqa_groups=None,
                  causal=True, window=(-1, -1), scale_factor=None, softmax_type="vanilla", softmax_offset=None,
                  seqlens=None):
    """FP8 attention forward (readings above).  q8 [B,S,Hq,Dqk], k8 [B,S,Hkv,Dqk],
    v8 [B,S,Hkv,Dv]: E4M3 codes (uint8).  Returns o [B,S,Hq,Dv], lse [B,Hq,S]
    (natural log), p8 (the quantized probability codes, [B,Hq,S,S]) and the
    unquantized e = exp(s - m) [B,Hq,S,S] and l [B,Hq,S] they come from."""
    q8, k8, v8 = (np.asarray(x, dtype=np.uint8) for x in (q8, k8, v8))
    B, S, Hq, dqk = q8.shape
    Hkv = k8.shape[2] if num_gqa_groups is None else int(num_gqa_groups)
    dv = v8.shape[3]
    scale = (1.0 / math.sqrt(dqk)) if not scale_factor else float(scale_factor)
    q = fp8_decode(q8, E4M3) * float(descale_q)
    k = fp8_decode(k8, E4M3) * float(descale_k)
    v = fp8_decode(v8, E4M3) * float(descale_v)
    o = np.zeros((B, S, Hq, dv))
    lse = np.zeros((B, Hq, S))
    p8 = np.zeros((B, Hq, S, S), dtype=np.uint8)
    e_all = np.zeros((B, Hq, S, S))
    l_all = np.zeros((B, Hq, S))
    for b in range(B):
        L = S if seqlens is None else int(np.asarray(seqlens).reshape(-1)[b])
        mask = visible_mask(S, L, causal, int(window[0]), int(window[1]))
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            s = scale * (q[b, :, h, :] @ k[b, :, g, :].T)
            z = sink_logit(softmax_type, softmax_offset, h)
            neg = np.where(mask, s, -np.inf)
            m = neg.max(axis=1)
            if z is not None:
                m = np.maximum(m, z)
            m_safe = np.where(np.isfinite(m), m, 0.0)
            e = np.where(mask, np.exp(neg - m_safe[:, None]), 0.0)
            l = e.sum(axis=1) + (0.0 if z is None else np.exp(z - m_safe))
            with np.errstate(divide="ignore"):
                lse[b, h] = np.where(l > 0, m_safe + np.log(l), -np.inf)
            codes = np.where(mask, fp8_encode(256.0 * e, E4M3), 0).astype(np.uint8)
            p8[b, h] = codes
            e_all[b, h] = e
            l_all[b, h] = l
            pq = fp8_decode(codes, E4M3) / 256.0
            with np.errstate(invalid="ignore", divide="ignore"):
                o[b, :, h, :] = np.where(l[:, None] > 0, (pq @ v[b, :, g, :]) / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return {"o": o, "lse": lse, "p8": p8, "e": e_all, "l": l_all}


def attention_fp8_rows(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, *, b, h, rows,
                       num_gqa_groups=None, causal=True, window=(-1, -1), scale_factor=None, softmax_type="vanilla",
                       softmax_offset=None, seqlens=None):
    """attention_fp8 for selected query rows of one (batch b, query head h):
    a row's output depends only on its own visible keys, so rows can be
    computed one by one at any length.  Returns o [n, Dv], lse [n]."""
    q8, k8, v8 = (np.asarray(x, dtype=np.uint8) for x in (q8, k8, v8))
    B, S, Hq, dqk = q8.shape
    Hkv = k8.shape[2] if num_gqa_groups is None else int(num_gqa_groups)
    scale = (1.0 / math.sqrt(dqk)) if not scale_factor else float(scale_factor)
    g = kv_head(h, Hq, Hkv)
    L = S if seqlens is None else int(np.asarray(seqlens).reshape(-1)[b])
    rows = np.asarray(rows, dtype=np.int64)
    mask = visible_rows(rows, S, L, causal, int(window[0]), int(window[1]))
    q = fp8_decode(q8[b, rows, h, :], E4M3) * float(descale_q)
    k = fp8_decode(k8[b, :, g, :], E4M3) * float(descale_k)
    v = fp8_decode(v8[b, :, g, :], E4M3) * float(descale_v)
    s = scale * (q @ k.T)
    z = sink_logit(softmax_type, softmax_offset, h)
    neg = np.where(mask, s, -np.inf)
    m = neg.max(axis=1)
    if z is not None:
        m = np.maximum(m, z)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(mask, np.exp(neg - m_safe[:, None]), 0.0)
    l = e.sum(axis=1) + (0.0 if z is None else np.exp(z - m_safe))
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m_safe + np.log(l), -np.inf)
    pq = fp8_decode(np.where(mask, fp8_encode(256.0 * e, E4M3), 0), E4M3) / 256.0
    o = np.where(l[:, None] > 0, (pq @ v) / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return {"o": o, "lse": lse}


def attention_fp8_bwd(q8, k8, v8, o, do8, lse, descale_q: float, descale_k: float, descale_v: float,
                      descale_do: float, scale_ds: float, *, num_gqa_groups=None, causal=True, window=(-1, -1),
                      scale_factor=None, softmax_type="vanilla", softmax_offset=None, seqlens=None):
    """FP8 attention backward (reading above).  q8 [B,S,Hq,D], k8 / v8
    [B,S,Hkv,D] E4M3 codes; do8 [B,S,Hq,Dv] E5M2 codes; o [B,S,Hq,Dv] and lse
    [B,Hq,S] from the forward (real values).  Returns dq, dk, dv (float64),
    dalpha [Hq] (None for vanilla), amax_ds, and per (b, h) the intermediates
    the tolerance bounds use: p [B,Hq,S,S], ds (unquantized dS), p8, ds8 codes,
    dp_abs (sum_d |dO_id V_jd|, the magnitude dP sums) and delta [B,Hq,S]."""
    q8, k8, v8, do8 = (np.asarray(x, dtype=np.uint8) for x in (q8, k8, v8, do8))
    B, S, Hq, dqk = q8.shape
    Hkv = k8.shape[2] if num_gqa_groups is None else int(num_gqa_groups)
    dv_dim = v8.shape[3]
    scale = (1.0 / math.sqrt(dqk)) if not scale_factor else float(scale_factor)
    q = fp8_decode(q8, E4M3) * float(descale_q)
    k = fp8_decode(k8, E4M3) * float(descale_k)
    v = fp8_decode(v8, E4M3) * float(descale_v)
    do = fp8_decode(do8, E5M2) * float(descale_do)
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    dq = np.zeros((B, S, Hq, dqk))
    dk = np.zeros((B, S, Hkv, dqk))
    dv = np.zeros((B, S, Hkv, dv_dim))
    dalpha = np.zeros(Hq)
    shape4 = (B, Hq, S, S)
    out = {"p": np.zeros(shape4), "ds": np.zeros(shape4), "p8": np.zeros(shape4, dtype=np.uint8),
           "ds8": np.zeros(shape4, dtype=np.uint8), "dp_abs": np.zeros(shape4), "delta": np.zeros((B, Hq, S))}
    amax = 0.0
    for b in range(B):
        L = S if seqlens is None else int(np.asarray(seqlens).reshape(-1)[b])
        mask = visible_mask(S, L, causal, int(window[0]), int(window[1]))
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            s = scale * (q[b, :, h, :] @ k[b, :, g, :].T)
            with np.errstate(invalid="ignore", over="ignore"):
                p = np.where(mask & np.isfinite(lse[b, h])[:, None], np.exp(s - lse[b, h][:, None]), 0.0)
            delta = np.where(np.arange(S) < L, (do[b, :, h, :] * o[b, :, h, :]).sum(axis=1), 0.0)
            dp = do[b, :, h, :] @ v[b, :, g, :].T
            ds = p * (dp - delta[:, None])
            amax = max(amax, float(np.abs(ds).max()))
            p8 = np.where(mask, fp8_encode(256.0 * p, E4M3), 0).astype(np.uint8)
            ds8 = np.where(mask, fp8_encode(float(scale_ds) * ds, E5M2), 0).astype(np.uint8)
            pq = fp8_decode(p8, E4M3) / 256.0
            dsq = fp8_decode(ds8, E5M2)
            dv[b, :, g, :] += pq.T @ do[b, :, h, :]
            dk[b, :, g, :] += scale / float(scale_ds) * (dsq.T @ q[b, :, h, :])
            dq[b, :, h, :] = scale / float(scale_ds) * (dsq @ k[b, :, g, :])
            z = sink_logit(softmax_type, softmax_offset, h)
            if z is not None:
                rows = np.isfinite(lse[b, h]) & (np.arange(S) < L)
                dalpha[h] += -float(np.sum(np.where(rows, np.exp(z - np.where(rows, lse[b, h], 0.0)) * delta, 0.0)))
            out["p"][b, h], out["ds"][b, h], out["p8"][b, h], out["ds8"][b, h] = p, ds, p8, ds8
            out["dp_abs"][b, h] = np.abs(do[b, :, h, :]) @ np.abs(v[b, :, g, :]).T
            out["delta"][b, h] = delta
    out.update(dq=dq, dk=dk, dv=dv, dalpha=None if softmax_type == "vanilla" else dalpha, amax_ds=amax)
    return out


def _bwd_rows_common(q8, k8, v8, o, do8, lse, descales, *, b, h, rows, keys, num_gqa_groups, causal, window,
                     scale_factor, seqlens):
    """Scores and gradient pieces of the FP8 backward for rows x keys of one
    (batch b, query head h): p, dp, delta of the rows, ds and the masks."""
    from .sdpa_oracle import visible_rows
    q8, k8, v8, do8 = (np.asarray(x, dtype=np.uint8) for x in (q8, k8, v8, do8))
    B, S, Hq, dqk = q8.shape
    Hkv = k8.shape[2] if num_gqa_groups is None else int(num_gqa_groups)
    scale = (1.0 / math.sqrt(dqk)) if not scale_factor else float(scale_factor)
    dq_, dk_, dv_, ddo = (float(x) for x in descales)
    g = kv_head(h, Hq, Hkv)
    L = S if seqlens is None else int(np.asarray(seqlens).reshape(-1)[b])
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    mask = visible_rows(rows, S, L, causal, int(window[0]), int(window[1]))[:, keys]
    q = fp8_decode(q8[b, rows, h, :], E4M3) * dq_
    k = fp8_decode(k8[b, keys, g, :], E4M3) * dk_
    v = fp8_decode(v8[b, keys, g, :], E4M3) * dv_
    do = fp8_decode(do8[b, rows, h, :], E5M2) * ddo
    lse_r = np.asarray(lse, dtype=np.float64)[b, h, rows]
    s = scale * (q @ k.T)
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.where(mask & np.isfinite(lse_r)[:, None], np.exp(s - lse_r[:, None]), 0.0)
    delta = np.where(rows < L, (do * np.asarray(o, dtype=np.float64)[b, rows, h, :]).sum(axis=1), 0.0)
    dp = do @ v.T
    ds = p * (dp - delta[:, None])
    return dict(q=q, k=k, do=do, p=p, ds=ds, mask=mask, scale=scale, dp_abs=np.abs(do) @ np.abs(v).T, delta=delta)


def attention_fp8_bwd_rows(q8, k8, v8, o, do8, lse, descale_q, descale_k, descale_v, descale_do, scale_ds, *, b, h,
                           rows, num_gqa_groups=None, causal=True, window=(-1, -1), scale_factor=None, seqlens=None):
    """dQ of attention_fp8_bwd for selected query rows of one (batch b, query
    head h), at any length: a row's dQ needs only its own scores against all
    keys.  Returns dq [n, D] and the row pieces p, ds, ds8, dp_abs, delta."""
    S = np.asarray(q8).shape[1]
    c = _bwd_rows_common(q8, k8, v8, o, do8, lse, (descale_q, descale_k, descale_v, descale_do), b=b, h=h,
                         rows=rows, keys=np.arange(S), num_gqa_groups=num_gqa_groups, causal=causal, window=window,
                         scale_factor=scale_factor, seqlens=seqlens)
    ds8 = np.where(c["mask"], fp8_encode(float(scale_ds) * c["ds"], E5M2), 0).astype(np.uint8)
    dq = c["scale"] / float(scale_ds) * (fp8_decode(ds8, E5M2) @ c["k"])
    return {"dq": dq, "p": c["p"], "ds": c["ds"], "ds8": ds8, "dp_abs": c["dp_abs"], "delta": c["delta"]}


def attention_fp8_bwd_keys(q8, k8, v8, o, do8, lse, descale_q, descale_k, descale_v, descale_do, scale_ds, *, b, g,
                           keys, num_gqa_groups=None, causal=True, window=(-1, -1), scale_factor=None, seqlens=None):
    """dK, dV of attention_fp8_bwd for selected keys of one (batch b, KV head
    g), summed over every row and query head of the group that sees them.
    Returns dk, dv [n, D] and, per query head of the group, the pieces
    (p, ds, p8, ds8, dp_abs, delta) as lists."""
    q8 = np.asarray(q8, dtype=np.uint8)
    B, S, Hq, dqk = q8.shape
    Hkv = np.asarray(k8).shape[2] if num_gqa_groups is None else int(num_gqa_groups)
    G = Hq // Hkv
    keys = np.asarray(keys, dtype=np.int64)
    dk = np.zeros((len(keys), dqk))
    dv = np.zeros((len(keys), np.asarray(v8).shape[3]))
    parts = {n: [] for n in ("p", "ds", "p8", "ds8", "dp_abs", "delta")}
    for h in range(g * G, (g + 1) * G):
        c = _bwd_rows_common(q8, k8, v8, o, do8, lse, (descale_q, descale_k, descale_v, descale_do), b=b, h=h,
                             rows=np.arange(S), keys=keys, num_gqa_groups=Hkv, causal=causal, window=window,
                             scale_factor=scale_factor, seqlens=seqlens)
        p8 = np.where(c["mask"], fp8_encode(256.0 * c["p"], E4M3), 0).astype(np.uint8)
        ds8 = np.where(c["mask"], fp8_encode(float(scale_ds) * c["ds"], E5M2), 0).astype(np.uint8)
        dv += (fp8_decode(p8, E4M3) / 256.0).T @ c["do"]
        dk += c["scale"] / float(scale_ds) * (fp8_decode(ds8, E5M2).T @ c["q"])
        for n, x in (("p", c["p"]), ("ds", c["ds"]), ("p8", p8), ("ds8", ds8), ("dp_abs", c["dp_abs"]),
                     ("delta", c["delta"])):
            parts[n].append(x)
    return {"dk": dk, "dv": dv, **parts}
