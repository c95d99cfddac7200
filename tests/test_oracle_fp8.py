"""Pins of the FP8 oracle (oracle/fp8.py), on the CPU.

  codec       every code decodes as torch's float8_e4m3fn / float8_e5m2 (a
              library implementation of the OFP8 formats); encoding equals
              torch's round-to-nearest-even cast on in-range values, exact ties
              included; saturation and NaN by definition; encode(decode(c)) = c
  recipe      delayed scaling on hand-worked histories
  attention   LSE equals the unquantized oracle's; O lies within the bound the
              E4M3 rounding of P allows around the unquantized oracle's O;
              scalar loops over a tiny case reproduce O and the P codes
  backward    equal to the unquantized oracle where no quantization rounds;
              the hand-worked example of tests/golden/fp8_bwd_hand.json;
              codes are nearest values (brute force) and the gradients lie
              within the E4M3 / E5M2 rounding bounds around the unquantized
              ones; the sink gradient equals the unquantized one; scalar loops
  mutants     planted mistakes in copies of the module each fail a pin
"""
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fp8.py")
TDT = {fp8.E4M3: torch.float8_e4m3fn, fp8.E5M2: torch.float8_e5m2}


def _torch_codes(x, fmt):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(TDT[fmt]).view(torch.uint8).numpy()


def pin_decode(m):
    for fmt in (m.E4M3, m.E5M2):
        codes = np.arange(256, dtype=np.uint8)
        ref = torch.tensor(codes).view(TDT[fmt]).to(torch.float64).numpy()
        got = m.fp8_decode(codes, fmt)
        assert np.array_equal(np.isnan(got), np.isnan(ref)), fmt
        ok = ~np.isnan(ref)
        assert np.array_equal(got[ok], ref[ok]), fmt
        assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok])), fmt


def pin_encode(m):
    rng = np.random.default_rng(5)
    for fmt in (m.E4M3, m.E5M2):
        mx = m.fp8_max(fmt)
        vals = np.sort(np.unique(np.abs(m.fp8_decode(np.arange(128), fmt)[:-1 if fmt == m.E4M3 else 124])))
        vals = vals[np.isfinite(vals)]
        mids = (vals[1:] + vals[:-1]) / 2  # exact ties
        x = np.concatenate([rng.uniform(-mx, mx, 4000), rng.standard_normal(4000) * 0.05,
                            rng.standard_normal(2000) * 1e-3, mids, -mids, vals, -vals])
        x = x.astype(np.float32).astype(np.float64)  # values torch sees exactly
        got = m.fp8_encode(x, fmt)
        ref = _torch_codes(x, fmt)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (fmt, x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def pin_saturation_and_nan(m):
    for fmt, top in ((m.E4M3, 0x7E), (m.E5M2, 0x7B)):
        mx = m.fp8_max(fmt)
        assert m.fp8_decode([top], fmt)[0] == mx
        big = np.array([mx * 1.01, mx * 4, 1e30, np.inf])
        assert (m.fp8_encode(big, fmt) == top).all(), fmt
        assert (m.fp8_encode(-big, fmt) == (top | 0x80)).all(), fmt
        assert np.isnan(m.fp8_decode(m.fp8_encode([np.nan], fmt), fmt)[0])
        finite = np.nonzero(np.isfinite(m.fp8_decode(np.arange(256), fmt)))[0]
        assert np.array_equal(m.fp8_encode(m.fp8_decode(finite, fmt), fmt), finite.astype(np.uint8)), fmt


def pin_recipe(m):
    h = np.array([3.0, 9.0, 2.0, 0.0])
    h2, s, d = m.delayed_scaling_update(h, 5.0, 1.0, m.E4M3)
    assert np.array_equal(h2, [5.0, 3.0, 9.0, 2.0])       # newest first, oldest dropped
    assert s == 448.0 / 9.0 and d == 1.0 / s
    _, s, _ = m.delayed_scaling_update(h, 5.0, 1.0, m.E5M2, margin=2)
    assert s == 57344.0 / 9.0 / 4.0
    _, s, _ = m.delayed_scaling_update(np.zeros(4), 0.0, 0.75, m.E4M3)
    assert s == 0.75                                       # no amax yet: keep the scale
    _, s, _ = m.delayed_scaling_update(np.zeros(4), np.inf, 0.5, m.E4M3)
    assert s == 0.5
    codes, amax = m.quantize(np.array([0.5, -3.0, 2.0]), 2.0, m.E4M3)
    assert amax == 3.0 and list(m.fp8_decode(codes, m.E4M3)) == [1.0, -6.0, 4.0]


def _case(seed, B=2, S=11, Hq=4, Hkv=2, d=8):
    rng = np.random.default_rng(seed)
    q8 = fp8.fp8_encode(rng.standard_normal((B, S, Hq, d)) * 8, fp8.E4M3)
    k8 = fp8.fp8_encode(rng.standard_normal((B, S, Hkv, d)) * 8, fp8.E4M3)
    v8 = fp8.fp8_encode(rng.standard_normal((B, S, Hkv, d)) * 8, fp8.E4M3)
    alpha = rng.standard_normal(Hq)
    return q8, k8, v8, alpha


MASKS = [(True, (-1, -1), None), (True, (3, 0), [11, 6]), (False, (2, 4), [0, 9]), (False, (-1, -1), None)]


def pin_attention_bound(m):
    """LSE is the unquantized oracle's; |O - O_exact| per element stays within
    sum_j max(2^-4 e_ij, 2^-18) |v_j| / l_i, the E4M3 rounding of 256 e_ij
    (half a unit in the last place: 2^-4 relative for normals, 2^-10 / 256
    absolute for subnormals) carried through O = sum_j e_ij v_j / l_i."""
    dq, dk, dv = 0.125, 0.25, 0.0625
    for ci, (causal, win, sl) in enumerate(MASKS):
        for st in oracle.SOFTMAX_TYPES:
            q8, k8, v8, alpha = _case(3100 + ci)
            kw = dict(num_gqa_groups=2, causal=causal, window=win, softmax_type=st, softmax_offset=alpha,
                      seqlens=None if sl is None else np.array(sl))
            r = m.attention_fp8(q8, k8, v8, dq, dk, dv, **kw)
            q, k, v = (m.fp8_decode(x, m.E4M3) * s for x, s in ((q8, dq), (k8, dk), (v8, dv)))
            ex = oracle.attention(q, k, v, None, **kw)
            fin = np.isfinite(ex["lse"])
            assert np.array_equal(np.isfinite(r["lse"]), fin)
            assert np.abs(r["lse"][fin] - ex["lse"][fin]).max() <= 1e-12
            B, S, Hq = q8.shape[:3]
            for b in range(B):
                L = S if sl is None else sl[b]
                mask = oracle.visible_mask(S, L, causal, win[0], win[1])
                for h in range(Hq):
                    g = h // 2
                    s = (q[b, :, h] @ k[b, :, g].T) / math.sqrt(q.shape[3])
                    z = oracle.sink_logit(st, alpha, h)
                    mrow = np.where(mask, s, -np.inf).max(axis=1)
                    if z is not None:
                        mrow = np.maximum(mrow, z)
                    mrow = np.where(np.isfinite(mrow), mrow, 0.0)
                    e = np.where(mask, np.exp(s - mrow[:, None]), 0.0)
                    l = e.sum(axis=1) + (0.0 if z is None else np.exp(z - mrow))
                    bound = (np.maximum(2.0 ** -4 * e, 2.0 ** -18) * mask) @ np.abs(v[b, :, g])
                    bound = np.where(l[:, None] > 0, bound / np.where(l > 0, l, 1)[:, None], 0.0)
                    err = np.abs(r["o"][b, :, h] - ex["o"][b, :, h])
                    assert (err <= bound * (1 + 1e-9) + 1e-15).all(), (ci, st, b, h, float((err - bound).max()))


def pin_attention_loops(m):
    """Scalar loops on a tiny case: scores, row max, sum, each P code and O."""
    q8, k8, v8, alpha = _case(3200, B=1, S=5, Hq=2, Hkv=1, d=4)
    dq, dk, dv = 0.5, 0.25, 2.0
    r = m.attention_fp8(q8, k8, v8, dq, dk, dv, num_gqa_groups=1, causal=True, softmax_type="off_by_one")
    S, scale = 5, 0.5  # 1/sqrt(4)
    for h in range(2):
        for i in range(S):
            s = [scale * sum(float(m.fp8_decode([q8[0, i, h, d]], m.E4M3)[0]) * dq *
                             float(m.fp8_decode([k8[0, j, 0, d]], m.E4M3)[0]) * dk for d in range(4))
                 for j in range(i + 1)]
            mx = max(max(s), 0.0)
            l = sum(math.exp(x - mx) for x in s) + math.exp(0.0 - mx)
            assert abs(r["lse"][0, h, i] - (mx + math.log(l))) <= 1e-12
            for d in range(4):
                acc = 0.0
                for j in range(i + 1):
                    c = int(m.fp8_encode([256.0 * math.exp(s[j] - mx)], m.E4M3)[0])
                    assert c == r["p8"][0, h, i, j]
                    acc += float(m.fp8_decode([c], m.E4M3)[0]) / 256.0 * float(
                        m.fp8_decode([v8[0, j, 0, d]], m.E4M3)[0]) * dv
                assert abs(r["o"][0, i, h, d] - acc / l) <= 1e-12 * (1 + abs(acc / l))


def pin_attention_rows(m):
    """The row-sampled function equals the whole-problem one."""
    for ci, (causal, win, sl) in enumerate(MASKS):
        for st in oracle.SOFTMAX_TYPES:
            q8, k8, v8, alpha = _case(3300 + ci)
            kw = dict(num_gqa_groups=2, causal=causal, window=win, softmax_type=st, softmax_offset=alpha,
                      seqlens=None if sl is None else np.array(sl))
            full = m.attention_fp8(q8, k8, v8, 0.5, 0.25, 0.125, **kw)
            for b in range(2):
                for h in (0, 1, 3):
                    rows = [10, 0, 4, 7]
                    r = m.attention_fp8_rows(q8, k8, v8, 0.5, 0.25, 0.125, b=b, h=h, rows=rows, **kw)
                    assert np.array_equal(np.isfinite(r["lse"]), np.isfinite(full["lse"][b, h, rows]))
                    fin = np.isfinite(r["lse"])
                    assert np.abs(r["lse"][fin] - full["lse"][b, h, rows][fin]).max(initial=0) <= 1e-12
                    assert np.abs(r["o"] - full["o"][b, rows, h]).max() <= 1e-12


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fp8_bwd_hand.json")


def _bwd_exact_case(m, kind, seed):
    """GQA (Hq 4, Hkv 2), S 16, d 8, no mask, where every quantization is
    exact: all scores of a row are equal (kind "q0": Q = 0; kind "krow": the
    16 keys of a KV head are one vector), so P = 1/16 and 256 P = 16; each V
    column holds eight 0s and eight 2s (mean 1); dO rows are one-hot with
    values +-1, +-2, so dS = P (dP - delta) = +-dO / 16 and with s_ds = 16 the
    E5M2 codes are exact.  Descales differ from 1 (the codes hold 2 Q, 2 K,
    2 V, 4 dO)."""
    rng = np.random.default_rng(seed)
    B, S, Hq, Hkv, d = 1, 16, 4, 2, 8
    q = np.zeros((B, S, Hq, d)) if kind == "q0" else rng.integers(-3, 4, (B, S, Hq, d)).astype(float)
    if kind == "q0":
        k = rng.integers(-3, 4, (B, S, Hkv, d)).astype(float)
    else:
        k = np.broadcast_to(rng.integers(-3, 4, (B, 1, Hkv, d)).astype(float), (B, S, Hkv, d)).copy()
    v = np.zeros((B, S, Hkv, d))
    for g in range(Hkv):
        for c in range(d):
            v[0, rng.permutation(S)[:8], g, c] = 2.0
    do = np.zeros((B, S, Hq, d))
    for i in range(S):
        for h in range(Hq):
            do[0, i, h, rng.integers(0, d)] = rng.choice([-2.0, -1.0, 1.0, 2.0])
    codes = [m.fp8_encode(2 * q, m.E4M3), m.fp8_encode(2 * k, m.E4M3), m.fp8_encode(2 * v, m.E4M3),
             m.fp8_encode(4 * do, m.E5M2)]
    return (q, k, v, do), codes


def pin_bwd_exact(m):
    """Where no quantization rounds, the FP8 backward equals the unquantized
    float64 backward (oracle.attention) on the same values."""
    for kind, seed in (("q0", 3400), ("krow", 3401)):
        (q, k, v, do), (q8, k8, v8, do8) = _bwd_exact_case(m, kind, seed)
        ex = oracle.attention(q, k, v, do, num_gqa_groups=2, causal=False)
        r = m.attention_fp8_bwd(q8, k8, v8, ex["o"], do8, ex["lse"], 0.5, 0.5, 0.5, 0.25, 16.0, num_gqa_groups=2,
                                causal=False)
        for n in ("dq", "dk", "dv"):
            err = np.abs(r[n] - ex[n]).max()
            assert err <= 1e-12 * (1 + np.abs(ex[n]).max()), (kind, n, err)
        assert np.abs(r["dq" if kind == "q0" else "dk"]).max() > 0.1  # the case exercises the product
        assert abs(r["amax_ds"] - 2.0 / 16) <= 1e-12


def pin_bwd_hand(m):
    """The hand-worked example of tests/golden/fp8_bwd_hand.json: dS rounded
    to E5M2 (1/3 -> 0.3125) and P to E4M3 (256/3 -> 88) where they enter dQ
    and dV."""
    import json
    gold = json.load(open(GOLDEN))
    S, d = 4, 4
    q8 = np.zeros((1, S, 1, d), dtype=np.uint8)
    k8 = m.fp8_encode(np.eye(S).reshape(1, S, 1, d), m.E4M3)
    v = np.zeros((1, S, 1, d))
    v[0, :, 0, 0] = np.arange(S)
    do = np.zeros((1, S, 1, d))
    do[0, :, 0, 0] = 1.0
    o = np.zeros((1, S, 1, d))
    o[0, :, 0, 0] = [0.0, 0.5, 1.0, 1.5]
    lse = np.log(np.arange(1, S + 1, dtype=float)).reshape(1, 1, S)
    r = m.attention_fp8_bwd(q8, k8, m.fp8_encode(v, m.E4M3), o, m.fp8_encode(do, m.E5M2), lse, 1.0, 1.0, 1.0, 1.0,
                            1.0, num_gqa_groups=1, causal=True)
    assert np.abs(r["dq"][0, :, 0, :] - np.array(gold["dq"])).max() <= 1e-12
    assert np.abs(r["dv"][0, :, 0, 0] - np.array(gold["dv_first_component"])).max() <= 1e-12
    assert np.abs(r["dv"][0, :, 0, 1:]).max() == 0 and np.abs(r["dk"]).max() == 0


def _nearest_ok(m, codes, x, fmt):
    """Each code's value is a nearest finite value of the format to x (brute
    force over all codes; x within the finite range)."""
    vals = m.fp8_decode(np.arange(256), fmt)
    vals = vals[np.isfinite(vals)]
    best = np.abs(x.reshape(-1, 1) - vals.reshape(1, -1)).min(axis=1)
    got = np.abs(m.fp8_decode(codes.reshape(-1), fmt) - x.reshape(-1))
    return np.all(got <= best * (1 + 1e-12) + 1e-300)


def pin_bwd_bound(m):
    """Random inputs: d_softmax_offset equals the unquantized oracle's; the P
    and dS codes are nearest values of E4M3 / E5M2 (brute force); dV, dK, dQ
    lie within the rounding bounds around the unquantized gradients:
    |P8/256 - P| <= max(2^-4 P, 2^-18) and |dS8/s - dS| <= max(2^-3 |dS|,
    2^-17 / s), carried through dV = sum P dO, dK = scale sum dS Q,
    dQ = scale sum dS K."""
    dq_, dk_, dv_, ddo = 0.125, 0.25, 0.0625, 1.0 / 64
    for ci, (causal, win, sl) in enumerate(MASKS):
        for st in oracle.SOFTMAX_TYPES:
            q8, k8, v8, alpha = _case(3500 + ci)
            rng = np.random.default_rng(3600 + ci)
            do8 = m.fp8_encode(rng.standard_normal(q8.shape) * 64, m.E5M2)
            kw = dict(num_gqa_groups=2, causal=causal, window=win, softmax_type=st, softmax_offset=alpha,
                      seqlens=None if sl is None else np.array(sl))
            q, k, v = (m.fp8_decode(x, m.E4M3) * s for x, s in ((q8, dq_), (k8, dk_), (v8, dv_)))
            do = m.fp8_decode(do8, m.E5M2) * ddo
            ex = oracle.attention(q, k, v, do, **kw)
            s_ds = 64.0
            r = m.attention_fp8_bwd(q8, k8, v8, ex["o"], do8, ex["lse"], dq_, dk_, dv_, ddo, s_ds, **kw)
            if st == "vanilla":
                assert r["dalpha"] is None
            else:
                assert np.abs(r["dalpha"] - ex["dalpha"]).max() <= 1e-12 * (1 + np.abs(ex["dalpha"]).max())
            vis = r["p"] > 0
            assert _nearest_ok(m, r["p8"][vis], 256.0 * r["p"][vis], m.E4M3)
            assert _nearest_ok(m, r["ds8"][vis], s_ds * r["ds"][vis], m.E5M2)
            scale = 1.0 / math.sqrt(q.shape[3])
            ep = np.maximum(2.0 ** -4 * r["p"], 2.0 ** -18) * vis
            eds = np.maximum(2.0 ** -3 * np.abs(r["ds"]), 2.0 ** -17 / s_ds) * vis
            B, S, Hq = q8.shape[:3]
            bdv, bdk, bdq = np.zeros(ex["dv"].shape), np.zeros(ex["dk"].shape), np.zeros(ex["dq"].shape)
            for b in range(B):
                for h in range(Hq):
                    g = h // 2
                    bdv[b, :, g] += ep[b, h].T @ np.abs(do[b, :, h])
                    bdk[b, :, g] += scale * eds[b, h].T @ np.abs(q[b, :, h])
                    bdq[b, :, h] = scale * eds[b, h] @ np.abs(k[b, :, g])
            for n, bound in (("dv", bdv), ("dk", bdk), ("dq", bdq)):
                err = np.abs(r[n] - ex[n])
                assert (err <= bound * (1 + 1e-9) + 1e-13).all(), (ci, st, n, float((err - bound).max()))
            assert abs(r["amax_ds"] - float(np.abs(r["ds"]).max())) == 0


def pin_bwd_loops(m):
    """Scalar loops on a tiny case (off-by-one sink, causal): P, delta, dP,
    dS, the codes and the three gradients element by element."""
    q8, k8, v8, alpha = _case(3700, B=1, S=4, Hq=2, Hkv=1, d=2)
    rng = np.random.default_rng(3701)
    do8 = m.fp8_encode(rng.standard_normal(q8.shape) * 8, m.E5M2)
    o = rng.standard_normal((1, 4, 2, 2))
    lse = rng.standard_normal((1, 2, 4)) + 2.0
    dq_, dk_, dv_, ddo, s_ds = 0.5, 0.25, 2.0, 0.125, 8.0
    r = m.attention_fp8_bwd(q8, k8, v8, o, do8, lse, dq_, dk_, dv_, ddo, s_ds, num_gqa_groups=1, causal=True,
                            softmax_type="off_by_one")
    e4 = lambda c: float(m.fp8_decode([c], m.E4M3)[0])  # noqa: E731
    e5 = lambda c: float(m.fp8_decode([c], m.E5M2)[0])  # noqa: E731
    S, D, scale = 4, 2, 1.0 / math.sqrt(2)
    dq = np.zeros((S, 2, D))
    dk = np.zeros((S, D))
    dv = np.zeros((S, D))
    dz = [0.0, 0.0]
    for h in range(2):
        for i in range(S):
            delta = sum(e5(do8[0, i, h, d]) * ddo * o[0, i, h, d] for d in range(D))
            dz[h] -= math.exp(0.0 - lse[0, h, i]) * delta
            for j in range(i + 1):
                s = scale * sum(e4(q8[0, i, h, d]) * dq_ * e4(k8[0, j, 0, d]) * dk_ for d in range(D))
                p = math.exp(s - lse[0, h, i])
                dp = sum(e5(do8[0, i, h, d]) * ddo * e4(v8[0, j, 0, d]) * dv_ for d in range(D))
                ds = p * (dp - delta)
                c_p = int(m.fp8_encode([256.0 * p], m.E4M3)[0])
                c_ds = int(m.fp8_encode([s_ds * ds], m.E5M2)[0])
                assert c_p == r["p8"][0, h, i, j] and c_ds == r["ds8"][0, h, i, j]
                for d in range(D):
                    dv[j, d] += e4(c_p) / 256.0 * e5(do8[0, i, h, d]) * ddo
                    dk[j, d] += scale / s_ds * e5(c_ds) * e4(q8[0, i, h, d]) * dq_
                    dq[i, h, d] += scale / s_ds * e5(c_ds) * e4(k8[0, j, 0, d]) * dk_
    assert np.abs(r["dv"][0, :, 0] - dv).max() <= 1e-12 * (1 + np.abs(dv).max())
    assert np.abs(r["dk"][0, :, 0] - dk).max() <= 1e-12 * (1 + np.abs(dk).max())
    assert np.abs(r["dq"][0] - dq).max() <= 1e-12 * (1 + np.abs(dq).max())
    assert np.abs(r["dalpha"] - np.array(dz)).max() <= 1e-12 * (1 + np.abs(dz).max())


def pin_bwd_sampled(m):
    """The row- and key-sampled backward functions equal the whole-problem one."""
    for ci, (causal, win, sl) in enumerate(MASKS):
        q8, k8, v8, alpha = _case(3800 + ci)
        rng = np.random.default_rng(3900 + ci)
        do8 = m.fp8_encode(rng.standard_normal(q8.shape) * 64, m.E5M2)
        o = rng.standard_normal(q8.shape)
        lse = rng.standard_normal((2, 4, 11)) + 3.0
        kw = dict(num_gqa_groups=2, causal=causal, window=win, seqlens=None if sl is None else np.array(sl))
        args = (q8, k8, v8, o, do8, lse, 0.125, 0.25, 0.0625, 1.0 / 64, 32.0)
        full = m.attention_fp8_bwd(*args, **kw)
        for b in range(2):
            for h in (0, 1, 3):
                rows = [10, 0, 4, 7]
                r = m.attention_fp8_bwd_rows(*args, b=b, h=h, rows=rows, **kw)
                assert np.abs(r["dq"] - full["dq"][b, rows, h]).max() <= 1e-12
                assert np.array_equal(r["ds8"], full["ds8"][b, h][rows])
            for g in (0, 1):
                keys = [9, 0, 5]
                r = m.attention_fp8_bwd_keys(*args, b=b, g=g, keys=keys, **kw)
                assert np.abs(r["dk"] - full["dk"][b, keys, g]).max() <= 1e-12
                assert np.abs(r["dv"] - full["dv"][b, keys, g]).max() <= 1e-12


PINS = [pin_decode, pin_encode, pin_saturation_and_nan, pin_recipe, pin_attention_bound, pin_attention_loops,
        pin_attention_rows, pin_bwd_exact, pin_bwd_hand, pin_bwd_bound, pin_bwd_loops, pin_bwd_sampled]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_fp8_pin(pin):
    pin(fp8)


MUTANTS = {
    "e4m3_bias_8": ("E4M3: (4, 3, 7)", "E4M3: (4, 3, 8)"),
    "ties_to_odd": ("(codes[hi] % 2 == 0)", "(codes[hi] % 2 == 1)"),
    "overflow_to_nan": ("out = np.where(np.isnan(x), 0x7F, out)",
                        "out = np.where(np.isnan(x) | (np.abs(x) > fp8_max(fmt)), 0x7F, out)"),
    "e5m2_inf_as_nan": ("val = np.where(e == emax, np.where(m == 0, np.inf, np.nan), val)",
                        "val = np.where(e == emax, np.nan, val)"),
    "p_scale_448": ("codes = np.where(mask, fp8_encode(256.0 * e, E4M3), 0).astype(np.uint8)",
                    "codes = np.where(mask, fp8_encode(448.0 * e, E4M3), 0).astype(np.uint8)"),
    "v_descale_dropped": ("v = fp8_decode(v8, E4M3) * float(descale_v)", "v = fp8_decode(v8, E4M3)", "all"),
    "history_oldest_first": ("h = np.concatenate([[float(new_amax)], np.asarray(history, dtype=np.float64)[:-1]])",
                             "h = np.concatenate([np.asarray(history, dtype=np.float64)[1:], [float(new_amax)]])"),
    "margin_ignored": ("scale = fp8_max(fmt) / amax / (2.0 ** margin)", "scale = fp8_max(fmt) / amax"),
    "sink_missing_in_sum": ("l = e.sum(axis=1) + (0.0 if z is None else np.exp(z - m_safe))", "l = e.sum(axis=1)",
                            "all"),
    "rows_wrong_kv_head": ("k = fp8_decode(k8[b, :, g, :], E4M3) * float(descale_k)",
                           "k = fp8_decode(k8[b, :, h % k8.shape[2], :], E4M3) * float(descale_k)"),
    "bwd_ds_scale_kept": ("dq[b, :, h, :] = scale / float(scale_ds) * (dsq @ k[b, :, g, :])",
                          "dq[b, :, h, :] = scale * (dsq @ k[b, :, g, :])"),
    "bwd_ds_as_e4m3": [("ds8 = np.where(mask, fp8_encode(float(scale_ds) * ds, E5M2), 0)",
                        "ds8 = np.where(mask, fp8_encode(float(scale_ds) * ds, E4M3), 0)"),
                       ("dsq = fp8_decode(ds8, E5M2)", "dsq = fp8_decode(ds8, E4M3)")],
    "bwd_p_unquantized": ("dv[b, :, g, :] += pq.T @ do[b, :, h, :]", "dv[b, :, g, :] += p.T @ do[b, :, h, :]"),
    "bwd_delta_dropped": ("ds = p * (dp - delta[:, None])", "ds = p * dp", "all"),
    "bwd_p_row_max": ("np.exp(s - lse[b, h][:, None])",
                      "np.exp(s - np.where(mask, s, -np.inf).max(axis=1)[:, None])"),
    "bwd_dk_no_group_sum": ("dk[b, :, g, :] += scale", "dk[b, :, g, :] = scale"),
    "bwd_dq_wrong_kv_head": ("dq[b, :, h, :] = scale / float(scale_ds) * (dsq @ k[b, :, g, :])",
                             "dq[b, :, h, :] = scale / float(scale_ds) * (dsq @ k[b, :, (g + 1) % Hkv, :])"),
    "bwd_do_descale_dropped": ("do = fp8_decode(do8, E5M2) * float(descale_do)", "do = fp8_decode(do8, E5M2)"),
    "bwd_dalpha_sign": ("dalpha[h] += -float(", "dalpha[h] += float("),
    "bwd_dk_takes_k": ("(dsq.T @ q[b, :, h, :])", "(dsq.T @ k[b, :, g, :])"),
    "bwd_rows_wrong_kv_head": ("    g = kv_head(h, Hq, Hkv)\n    L = S if seqlens is None else int(np.asarray(seqlens).reshape(-1)[b])\n    rows = np.asarray(rows, dtype=np.int64)\n    keys",
                               "    g = (h + 1) % Hkv\n    L = S if seqlens is None else int(np.asarray(seqlens).reshape(-1)[b])\n    rows = np.asarray(rows, dtype=np.int64)\n    keys"),
    "bwd_keys_group_off_by_one": ("for h in range(g * G, (g + 1) * G):", "for h in range(g * G, (g + 1) * G - 1):"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_mutant_is_caught(name):
    src = open(SRC).read()
    edits = MUTANTS[name] if isinstance(MUTANTS[name], list) else [MUTANTS[name]]
    for edit in edits:
        old, new = edit[:2]
        every = len(edit) > 2
        assert src.count(old) >= 1 and (every or src.count(old) == 1), name
        src = src.replace(old, new)
    mod = types.ModuleType("fp8_mutant")
    mod.__package__ = "oracle"
    exec(compile(src, "fp8_mutant.py", "exec"), mod.__dict__)
    for pin in PINS:
        try:
            pin(mod)
        except AssertionError:
            return
    pytest.fail(f"mutant {name} passed every pin")
