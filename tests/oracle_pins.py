"""Pins for the float64 oracle: checks against things other than the oracle itself.

Each pin is a function of the oracle *module*, so the same pins run against the
real oracle (test_oracle_pins.py) and against copies of it with a planted
mistake (test_oracle_mutants.py), which must fail at least one pin.

What pins what:
  brute_force      whole forward: scalar loops over the softmax definition
                   exp(s)/ (sum exp(s) [+ exp(z)]) with no max shift (PR #2225
                   sequence diagrams; codelab "How attention works")
  finite_diff      dQ, dK, dV, d(alpha): central differences of sum(dO * O)
  row_sums         sum_j P_ij = 1 (vanilla) or 1 - exp(z - LSE_i) (sink), via V = 1
  gqa_repeat       GQA equals MHA on K/V heads repeated in contiguous groups
                   (TE single-GPU page section 1; codelab section 9)
  causal_rows      first causal row attends only to itself, last row equals the
                   unmasked one (codelab section 7)
  sink_augmented   sink softmax equals vanilla softmax over one extra key whose
                   score is exactly z and whose value row is 0 (PR #2225 review
                   thread: the offset is an extra logit)
  sink_closed      closed form of the first causal row with a sink; off-by-one ==
                   learnable with alpha = 0; alpha = -1e4 == vanilla
  dalpha_forms     d(alpha) closed form == finite difference == augmented-key grad
  padding          a padded batch equals the truncated unpadded problem; padded
                   rows and keys are exactly zero
  window_limits    left >= S-1 with causal == causal; left = 0 => O_i = V_i
  scale            attn(Q, scale=c) == attn(cQ, scale=1), sink logit unscaled
  torch_sdpa       torch.nn.functional.scaled_dot_product_attention (CPU float64)
                   with autograd: O, dQ, dK, dV and, through an additive mask
                   column, d(alpha)
  golden           hand-derived closed forms stored under tests/golden/
  packed_*         packed (THD) oracle: scalar loops over each segment's
                   tokens; equality with the padded per-batch oracle (a
                   different formulation: block-diagonal mask over the token
                   axis vs one S x S problem per batch); finite differences
  philox_kat       the dropout generator (Philox4x32-10) against its published
                   known-answer vectors (tests/golden/philox4x32_10_kat.json)
  bias_*           additive post-scale bias: torch SDPA with the bias as a float
                   mask (autograd gives the bias gradient), zero / row-constant
                   bias invariants, finite differences
  dropout_*        keep rate and stream independence; scalar loops with the
                   keep mask applied by hand; p = 0 == no dropout; finite
                   differences; unbiasedness over many offsets
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_case(seed, B=2, S=9, Hq=4, Hkv=2, dqk=5, dv=3, sink=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, Hq, dqk))
    k = rng.standard_normal((B, S, Hkv, dqk))
    v = rng.standard_normal((B, S, Hkv, dv))
    do = rng.standard_normal((B, S, Hq, dv))
    alpha = rng.standard_normal(Hq)
    return q, k, v, do, alpha


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(a - b))
    bound = atol + rtol * np.maximum(np.abs(np.where(both_inf, 0, a)), np.abs(np.where(both_inf, 0, b)))
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: max err {np.nanmax(np.where(bad, err, 0))} at {np.argwhere(bad)[:3].tolist()}"


def brute_forward(q, k, v, Hkv, causal, wl, wr, scale, stype, alpha, seqlens):
    """Scalar loops over the definition, no max shift (inputs are small)."""
    B, S, Hq, dqk = q.shape
    dv = v.shape[3]
    G = Hq // Hkv
    o = np.zeros((B, S, Hq, dv))
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        L = S if seqlens is None else int(seqlens[b])
        for h in range(Hq):
            g = h // G
            for i in range(S):
                num = [0.0] * dv
                den = 0.0
                for j in range(S):
                    vis = (i < L and j < L and (not causal or j <= i)
                           and (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr))
                    if not vis:
                        continue
                    s = scale * sum(float(q[b, i, h, d]) * float(k[b, j, g, d]) for d in range(dqk))
                    e = math.exp(s)
                    den += e
                    for d in range(dv):
                        num[d] += e * float(v[b, j, g, d])
                if stype == "off_by_one":
                    den += math.exp(0.0)
                elif stype == "learnable":
                    den += math.exp(float(alpha[h]))
                for d in range(dv):
                    o[b, i, h, d] = num[d] / den if den > 0 else 0.0
                lse[b, h, i] = math.log(den) if den > 0 else -math.inf
    return o, lse


MASK_CASES = [
    # causal, (left, right), seqlens
    (True, (-1, -1), None),
    (False, (-1, -1), None),
    (True, (3, 0), [9, 5]),
    (False, (2, 1), [6, 9]),
    (True, (0, 0), None),
    (False, (-1, 2), [0, 7]),
    (True, (-1, -1), [1, 9]),
]


def pin_brute_force(orc):
    for ci, (causal, win, sl) in enumerate(MASK_CASES):
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(100 + ci)
            scale = 0.37
            sl_np = None if sl is None else np.array(sl)
            r = orc.attention(q, k, v, None, num_gqa_groups=2, causal=causal, window=win,
                              scale_factor=scale, softmax_type=st, softmax_offset=alpha,
                              seqlens=sl_np)
            o, lse = brute_forward(q, k, v, 2, causal, win[0], win[1], scale, st, alpha, sl)
            _close(r["o"], o, 1e-12, 1e-14, f"O case{ci} {st}")
            _close(r["lse"], lse, 1e-12, 1e-14, f"LSE case{ci} {st}")


def _loss(orc, q, k, v, do, alpha, **kw):
    r = orc.attention(q, k, v, None, softmax_offset=alpha, **kw)
    return float((r["o"] * do).sum())


def pin_finite_diff(orc):
    h = 1e-6
    for ci, (causal, win, sl) in enumerate([(True, (-1, -1), None), (False, (2, 1), [5, 7]),
                                            (True, (3, 0), [7, 4])]):
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(200 + ci, B=2, S=7, Hq=4, Hkv=2, dqk=3, dv=2)
            kw = dict(num_gqa_groups=2, causal=causal, window=win, scale_factor=0.6,
                      softmax_type=st, seqlens=None if sl is None else np.array(sl))
            r = orc.attention(q, k, v, do, softmax_offset=alpha, **kw)
            for name, arr, grad in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
                fd = np.zeros_like(arr)
                for idx in np.ndindex(arr.shape):
                    a0 = arr[idx]
                    arr[idx] = a0 + h
                    lp = _loss(orc, q, k, v, do, alpha, **kw)
                    arr[idx] = a0 - h
                    lm = _loss(orc, q, k, v, do, alpha, **kw)
                    arr[idx] = a0
                    fd[idx] = (lp - lm) / (2 * h)
                _close(grad, fd, 1e-6, 1e-8, f"d{name} case{ci} {st}")
            if st != "vanilla":
                fd = np.zeros(4)
                for hh in range(4):
                    a2 = alpha.copy()
                    if st == "learnable":
                        a2[hh] += h
                        lp = _loss(orc, q, k, v, do, a2, **kw)
                        a2[hh] -= 2 * h
                        lm = _loss(orc, q, k, v, do, a2, **kw)
                        fd[hh] = (lp - lm) / (2 * h)
                if st == "learnable":
                    _close(r["dalpha"], fd, 1e-6, 1e-8, f"dalpha case{ci}")
            else:
                assert r["dalpha"] is None


def pin_row_sums(orc):
    for ci, (causal, win, sl) in enumerate(MASK_CASES):
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(300 + ci, dv=1)
            ones = np.ones_like(v)
            r = orc.attention(q, k, ones, None, num_gqa_groups=2, causal=causal, window=win,
                              softmax_type=st, softmax_offset=alpha,
                              seqlens=None if sl is None else np.array(sl))
            B, S = q.shape[:2]
            for b in range(B):
                L = S if sl is None else sl[b]
                for h in range(4):
                    rs = r["o"][b, :L, h, 0]
                    if st == "vanilla":
                        expect = np.ones(L)
                    else:
                        z = 0.0 if st == "off_by_one" else alpha[h]
                        expect = 1.0 - np.exp(z - r["lse"][b, h, :L])
                        assert (rs < 1).all()
                    _close(rs, expect, 1e-12, 1e-13, f"rowsum case{ci} {st}")


def pin_gqa_repeat(orc):
    for Hq, Hkv in ((4, 2), (6, 3), (4, 1), (4, 4)):
        G = Hq // Hkv
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(400 + Hq * 10 + Hkv, Hq=Hq, Hkv=Hkv)
            alpha = np.random.default_rng(1).standard_normal(Hq)
            kw = dict(causal=True, window=(4, 0), softmax_type=st, softmax_offset=alpha,
                      seqlens=np.array([9, 6]))
            r = orc.attention(q, k, v, do, num_gqa_groups=Hkv, **kw)
            kr = np.repeat(k, G, axis=2)
            vr = np.repeat(v, G, axis=2)
            m = orc.attention(q, kr, vr, do, num_gqa_groups=Hq, **kw)
            _close(r["o"], m["o"], 1e-13, 1e-14, "O")
            _close(r["lse"], m["lse"], 1e-13, 1e-14, "LSE")
            _close(r["dq"], m["dq"], 1e-12, 1e-13, "dQ")
            B, S = q.shape[:2]
            _close(r["dk"], m["dk"].reshape(B, S, Hkv, G, -1).sum(axis=3), 1e-12, 1e-13, "dK")
            _close(r["dv"], m["dv"].reshape(B, S, Hkv, G, -1).sum(axis=3), 1e-12, 1e-13, "dV")
            if st != "vanilla":
                _close(r["dalpha"], m["dalpha"], 1e-12, 1e-13, "dalpha")


def pin_causal_rows(orc):
    q, k, v, do, alpha = rand_case(500, S=11)
    c = orc.attention(q, k, v, None, num_gqa_groups=2, causal=True)
    n = orc.attention(q, k, v, None, num_gqa_groups=2, causal=False)
    _close(c["o"][:, -1], n["o"][:, -1], 1e-13, 1e-14, "last row")
    _close(c["lse"][:, :, -1], n["lse"][:, :, -1], 1e-13, 1e-14, "last row lse")
    G = 2
    for h in range(4):
        _close(c["o"][:, 0, h], v[:, 0, h // G], 1e-13, 1e-14, "row 0 = V_0")
    assert np.abs(c["o"][:, 0] - n["o"][:, 0]).max() > 1e-3


def pin_sink_augmented(orc):
    """Sink softmax == vanilla over an extra key with score z and a zero value."""
    B, S, Hq, Hkv, dqk, dv = 2, 8, 4, 2, 5, 3
    q, k, v, do, alpha = rand_case(600, B, S, Hq, Hkv, dqk, dv)
    scale = 0.45
    G = Hq // Hkv
    for st in ("off_by_one", "learnable"):
        r = orc.attention(q, k, v, do, num_gqa_groups=Hkv, causal=False, scale_factor=scale,
                          softmax_type=st, softmax_offset=alpha)
        z = np.zeros(Hq) if st == "off_by_one" else alpha
        # MHA over S+1 positions; Q gets a constant-1 extra feature, real keys a 0,
        # the extra key (position S) has features (0.., z_h / scale) and value 0.
        qa = np.zeros((B, S + 1, Hq, dqk + 1))
        qa[:, :S, :, :dqk] = q
        qa[:, :, :, dqk] = 1.0
        ka = np.zeros((B, S + 1, Hq, dqk + 1))
        ka[:, :S, :, :dqk] = np.repeat(k, G, axis=2)
        ka[:, S, :, dqk] = z / scale
        va = np.zeros((B, S + 1, Hq, dv))
        va[:, :S] = np.repeat(v, G, axis=2)
        doa = np.zeros((B, S + 1, Hq, dv))
        doa[:, :S] = do
        a = orc.attention(qa, ka, va, doa, num_gqa_groups=Hq, causal=False, scale_factor=scale)
        _close(r["o"], a["o"][:, :S], 1e-12, 1e-14, f"O {st}")
        _close(r["lse"], a["lse"][:, :, :S], 1e-12, 1e-14, f"LSE {st}")
        _close(r["dq"], a["dq"][:, :S, :, :dqk], 1e-11, 1e-13, f"dQ {st}")
        _close(r["dk"], a["dk"][:, :S, :, :dqk].reshape(B, S, Hkv, G, dqk).sum(3), 1e-11, 1e-13, f"dK {st}")
        _close(r["dv"], a["dv"][:, :S].reshape(B, S, Hkv, G, dv).sum(3), 1e-11, 1e-13, f"dV {st}")
        # d score(extra key) = d k_extra[last] / scale, summed over batches.
        dz = a["dk"][:, S, :, dqk].sum(axis=0) / scale
        _close(r["dalpha"], dz, 1e-10, 1e-13, f"dalpha {st}")


def pin_sink_closed(orc):
    q, k, v, do, alpha = rand_case(700, S=6)
    scale = 0.5
    G = 2
    for st in ("off_by_one", "learnable"):
        r = orc.attention(q, k, v, None, num_gqa_groups=2, causal=True, scale_factor=scale,
                          softmax_type=st, softmax_offset=alpha)
        for b in range(2):
            for h in range(4):
                z = 0.0 if st == "off_by_one" else alpha[h]
                s00 = scale * float(q[b, 0, h] @ k[b, 0, h // G])
                w = math.exp(s00) / (math.exp(z) + math.exp(s00))
                _close(r["o"][b, 0, h], w * v[b, 0, h // G], 1e-13, 1e-15, f"row0 {st}")
                _close(r["lse"][b, h, 0], math.log(math.exp(z) + math.exp(s00)), 1e-13, 0, "lse0")
    kw = dict(num_gqa_groups=2, causal=True, window=(3, 0), seqlens=np.array([6, 4]))
    a = orc.attention(q, k, v, do, softmax_type="off_by_one", **kw)
    b_ = orc.attention(q, k, v, do, softmax_type="learnable", softmax_offset=np.zeros(4), **kw)
    for key in ("o", "lse", "dq", "dk", "dv", "dalpha"):
        _close(a[key], b_[key], 0, 0, f"obo==learnable(0) {key}")
    c = orc.attention(q, k, v, do, softmax_type="learnable", softmax_offset=np.full(4, -1e4), **kw)
    d = orc.attention(q, k, v, do, softmax_type="vanilla", **kw)
    for key in ("o", "dq", "dk", "dv"):
        _close(c[key], d[key], 1e-13, 1e-15, f"alpha=-1e4 == vanilla {key}")
    _close(c["lse"][:, :, :4], d["lse"][:, :, :4], 1e-13, 1e-15, "lse")


def pin_dalpha_forms(orc):
    q, k, v, do, alpha = rand_case(800, B=3, S=8)
    kw = dict(num_gqa_groups=2, causal=True, window=(4, 0), scale_factor=0.4,
              seqlens=np.array([8, 5, 3]))
    r = orc.attention(q, k, v, do, softmax_type="learnable", softmax_offset=alpha, **kw)
    h = 1e-6
    fd = np.zeros(4)
    for hh in range(4):
        ap = alpha.copy(); ap[hh] += h
        am = alpha.copy(); am[hh] -= h
        fd[hh] = (_loss(orc, q, k, v, do, ap, softmax_type="learnable", **kw)
                  - _loss(orc, q, k, v, do, am, softmax_type="learnable", **kw)) / (2 * h)
    _close(r["dalpha"], fd, 1e-6, 1e-9, "dalpha vs fd")
    # closed form from the returned O and LSE
    delta = (r["o"] * do).sum(axis=3)                    # [B,S,Hq]
    cf = -(np.exp(alpha[None, :, None] - r["lse"]) * delta.transpose(0, 2, 1)).sum(axis=(0, 2))
    _close(r["dalpha"], cf, 1e-12, 1e-14, "dalpha closed form")


def pin_padding(orc):
    q, k, v, do, alpha = rand_case(900, B=3, S=10)
    sl = np.array([10, 6, 0])
    for st in orc.SOFTMAX_TYPES:
        for causal, win in ((True, (-1, -1)), (False, (3, 2)), (True, (2, 0))):
            kw = dict(num_gqa_groups=2, causal=causal, window=win, softmax_type=st,
                      softmax_offset=alpha)
            r = orc.attention(q, k, v, do, seqlens=sl, **kw)
            for b in range(3):
                L = sl[b]
                if L > 0:
                    # same arithmetic on a smaller matrix: equal up to BLAS summation order
                    t = orc.attention(q[b:b + 1, :L], k[b:b + 1, :L], v[b:b + 1, :L],
                                      do[b:b + 1, :L], **kw)
                    _close(r["o"][b, :L], t["o"][0], 1e-13, 1e-15, "O")
                    _close(r["lse"][b, :, :L], t["lse"][0], 1e-13, 1e-15, "LSE")
                    _close(r["dq"][b, :L], t["dq"][0], 1e-13, 1e-15, "dQ")
                    _close(r["dk"][b, :L], t["dk"][0], 1e-13, 1e-15, "dK")
                    _close(r["dv"][b, :L], t["dv"][0], 1e-13, 1e-15, "dV")
                assert (r["o"][b, L:] == 0).all() and (r["dq"][b, L:] == 0).all()
                assert (r["dk"][b, L:] == 0).all() and (r["dv"][b, L:] == 0).all()
                z = -np.inf if st == "vanilla" else (0.0 if st == "off_by_one" else alpha)
                pad_lse = r["lse"][b, :, L:]
                expect = np.broadcast_to(np.reshape(z, (-1, 1)) if st == "learnable" else z, pad_lse.shape)
                _close(pad_lse, expect, 0, 0, "padded LSE")


def pin_window_limits(orc):
    S = 9
    for L in (9, 5):
        assert (orc.visible_mask(S, L, True, S - 1, 0) == orc.visible_mask(S, L, True, -1, -1)).all()
        assert (orc.visible_mask(S, L, True, S + 5, 3) == orc.visible_mask(S, L, True, -1, -1)).all()
    q, k, v, do, alpha = rand_case(1000, S=S)
    r = orc.attention(q, k, v, None, num_gqa_groups=2, causal=True, window=(0, 0))
    for h in range(4):
        _close(r["o"][:, :, h], v[:, :, h // 2], 1e-13, 1e-15, "left=0 => O=V")
    r = orc.attention(q, k, v, None, num_gqa_groups=2, causal=False, window=(0, 0))
    for h in range(4):
        _close(r["o"][:, :, h], v[:, :, h // 2], 1e-13, 1e-15, "(0,0) => O=V")
    m = orc.visible_mask(6, 6, False, 1, 2)
    expect = np.array([[abs(i - j) <= (1 if j < i else 2) for j in range(6)] for i in range(6)])
    assert (m == expect).all()
    assert orc.visible_pairs(S, S, True, -1, -1) == S * (S + 1) // 2
    for causal in (True, False):
        for wl in (-1, 0, 2, 7):
            for wr in (-1, 0, 1, 4):
                for L in (0, 3, 9):
                    assert orc.visible_pairs(S, L, causal, wl, wr) == int(orc.visible_mask(S, L, causal, wl, wr).sum())


def pin_scale(orc):
    q, k, v, do, alpha = rand_case(1100)
    c = 0.73
    for st in orc.SOFTMAX_TYPES:
        kw = dict(num_gqa_groups=2, causal=True, window=(5, 0), softmax_type=st,
                  softmax_offset=alpha, seqlens=np.array([9, 7]))
        a = orc.attention(q, k, v, do, scale_factor=c, **kw)
        b = orc.attention(c * q, k, v, do, scale_factor=1.0, **kw)
        _close(a["o"], b["o"], 1e-12, 1e-14, "O")
        _close(a["lse"], b["lse"], 1e-12, 1e-14, "LSE")
        _close(a["dq"], c * b["dq"], 1e-12, 1e-14, "dQ")
        _close(a["dk"], b["dk"], 1e-12, 1e-14, "dK")
        _close(a["dv"], b["dv"], 1e-12, 1e-14, "dV")
    d = orc.attention(q[:, :, :, :4], k[:, :, :, :4], v, None, num_gqa_groups=2, causal=False)
    e = orc.attention(0.5 * q[:, :, :, :4], k[:, :, :, :4], v, None, num_gqa_groups=2,
                      causal=False, scale_factor=1.0)
    _close(d["o"], e["o"], 1e-12, 1e-14, "default scale = 1/sqrt(d_qk)")


def pin_torch_sdpa(orc):
    import torch
    F = torch.nn.functional
    cases = [
        (2, 33, 4, 2, 16, 8, True, (-1, -1), None),
        (2, 40, 6, 3, 8, 12, True, (9, 0), [40, 23]),
        (1, 37, 4, 1, 12, 12, False, (5, 3), [30]),
        (2, 29, 2, 2, 8, 8, False, (-1, -1), [29, 1]),
    ]
    for ci, (B, S, Hq, Hkv, dqk, dv, causal, win, sl) in enumerate(cases):
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(1200 + ci, B, S, Hq, Hkv, dqk, dv)
            scale = 1.0 / math.sqrt(dqk)
            sl_np = None if sl is None else np.array(sl)
            r = orc.attention(q, k, v, do, num_gqa_groups=Hkv, causal=causal, window=win,
                              softmax_type=st, softmax_offset=alpha, seqlens=sl_np)
            G = Hq // Hkv
            tq = torch.tensor(q.transpose(0, 2, 1, 3), requires_grad=True)
            tk = torch.tensor(k.transpose(0, 2, 1, 3), requires_grad=True)
            tv = torch.tensor(v.transpose(0, 2, 1, 3), requires_grad=True)
            i = torch.arange(S)[:, None]
            j = torch.arange(S)[None, :]
            vis = torch.zeros(B, 1, S, S, dtype=torch.bool)
            dmask = torch.ones(B, 1, S, 1, dtype=torch.float64)
            for b in range(B):
                L = S if sl is None else sl[b]
                m = (i < L) & (j < L)
                if causal:
                    m &= j <= i
                if win[0] >= 0:
                    m &= j >= i - win[0]
                if win[1] >= 0:
                    m &= j <= i + win[1]
                vis[b, 0] = m
                dmask[b, 0, L:] = 0.0
            tdo = torch.tensor(do.transpose(0, 2, 1, 3)) * dmask
            kr = tk.repeat_interleave(G, dim=1)
            vr = tv.repeat_interleave(G, dim=1)
            if st == "vanilla":
                # fully masked (padded) rows see key 0 with zero upstream gradient
                vis2 = vis.clone()
                vis2[:, :, :, 0] |= ~vis.any(dim=3)
                madd = torch.where(vis2, 0.0, -torch.inf).to(torch.float64).expand(B, Hq, S, S)
                madd = madd.clone().requires_grad_(True)
                o = F.scaled_dot_product_attention(tq, kr, vr, attn_mask=madd, scale=scale)
            else:
                z = torch.zeros(Hq, dtype=torch.float64) if st == "off_by_one" else torch.tensor(alpha)
                kz = torch.cat([kr, torch.zeros(B, Hq, 1, dqk, dtype=torch.float64)], dim=2)
                vz = torch.cat([vr, torch.zeros(B, Hq, 1, dv, dtype=torch.float64)], dim=2)
                base = torch.where(vis, 0.0, -torch.inf).to(torch.float64).expand(B, Hq, S, S)
                col = z.view(1, Hq, 1, 1).expand(B, Hq, S, 1)
                madd = torch.cat([base, col], dim=3).clone().requires_grad_(True)
                o = F.scaled_dot_product_attention(tq, kz, vz, attn_mask=madd, scale=scale)
            o.backward(tdo)
            o_np = o.detach().numpy().transpose(0, 2, 1, 3)
            for b in range(B):
                L = S if sl is None else sl[b]
                _close(r["o"][b, :L], o_np[b, :L], 1e-10, 1e-12, f"O case{ci} {st}")
            _close(r["dq"], tq.grad.numpy().transpose(0, 2, 1, 3), 1e-10, 1e-12, f"dQ case{ci} {st}")
            _close(r["dk"], tk.grad.numpy().transpose(0, 2, 1, 3), 1e-10, 1e-12, f"dK case{ci} {st}")
            _close(r["dv"], tv.grad.numpy().transpose(0, 2, 1, 3), 1e-10, 1e-12, f"dV case{ci} {st}")
            if st != "vanilla":
                dz = madd.grad[:, :, :, S].sum(dim=(0, 2)).numpy()
                _close(r["dalpha"], dz, 1e-10, 1e-12, f"dalpha case{ci} {st}")


def pin_golden(orc):
    with open(os.path.join(GOLDEN, "uniform_scores.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        S = len(case["v"])
        v = np.array(case["v"], dtype=np.float64).reshape(1, S, 1, 1)
        q = np.zeros((1, S, 1, 1))
        k = np.zeros((1, S, 1, 1))
        st = case["softmax_type"]
        alpha = np.array([case.get("alpha", 0.0)])
        r = orc.attention(q, k, v, None, num_gqa_groups=1, causal=case["causal"],
                          window=tuple(case["window"]), softmax_type=st, softmax_offset=alpha)
        _close(r["o"][0, :, 0, 0], np.array(case["o"]), 1e-15, 1e-15, case["name"])
        _close(r["lse"][0, 0], np.log(np.array(case["lse_exp"], dtype=np.float64)), 1e-15, 1e-15,
               case["name"] + " lse")


def pin_sampled_rows(orc):
    """Row-sampled outputs vs brute force (O, LSE), finite differences (dQ) and
    the closed forms of delta and d(sink logit) from brute-force O and LSE."""
    h_fd = 1e-6
    for ci, (causal, win, sl) in enumerate(MASK_CASES):
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(1300 + ci)
            kw = dict(num_gqa_groups=2, causal=causal, window=win, scale_factor=0.45, softmax_type=st,
                      softmax_offset=alpha, seqlens=None if sl is None else np.array(sl))
            o_bf, lse_bf = brute_forward(q, k, v, 2, causal, win[0], win[1], 0.45, st, alpha, sl)
            for b in range(2):
                for h in (0, 3):
                    rows = [0, 4, 8, 2] if ci % 2 else [8, 1, 5]
                    r = orc.attention_rows(q, k, v, do, b=b, h=h, rows=rows, **kw)
                    _close(r["o"], o_bf[b, rows, h], 1e-12, 1e-14, f"rows O {ci} {st}")
                    _close(r["lse"], lse_bf[b, h, rows], 1e-12, 1e-14, f"rows LSE {ci} {st}")
                    delta = (o_bf[b, rows, h] * do[b, rows, h]).sum(axis=1)
                    _close(r["delta"], delta, 1e-12, 1e-14, "rows delta")
                    if st != "vanilla":
                        z = 0.0 if st == "off_by_one" else alpha[h]
                        lse_s = np.where(np.isfinite(lse_bf[b, h, rows]), lse_bf[b, h, rows], z)
                        _close(r["dz"], -np.exp(z - lse_s) * delta, 1e-12, 1e-14, "rows dz")
                    ri = rows[0]
                    for d in range(q.shape[3]):
                        q[b, ri, h, d] += h_fd
                        lp = _loss(orc, q, k, v, do, alpha, **{x: y for x, y in kw.items() if x != "softmax_offset"})
                        q[b, ri, h, d] -= 2 * h_fd
                        lm = _loss(orc, q, k, v, do, alpha, **{x: y for x, y in kw.items() if x != "softmax_offset"})
                        q[b, ri, h, d] += h_fd
                        _close(r["dq"][0, d], (lp - lm) / (2 * h_fd), 1e-6, 1e-8, f"rows dQ fd {ci} {st}")


def pin_sampled_keys(orc):
    """Key-sampled dK, dV vs finite differences of sum(dO * O)."""
    h_fd = 1e-6
    for ci, (causal, win, sl) in enumerate(MASK_CASES):
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(1400 + ci, B=2, S=8, dqk=3, dv=2)
            kw = dict(num_gqa_groups=2, causal=causal, window=win, scale_factor=0.55, softmax_type=st,
                      seqlens=None if sl is None else np.array(sl))
            for b in range(2):
                g = (b + ci) % 2
                keys = [7, 0, 3] if ci % 2 else [5, 2]
                r = orc.attention_keys(q, k, v, do, b=b, g=g, keys=keys, softmax_offset=alpha,
                                       row_block=3, **kw)
                for n, j in enumerate(keys):
                    for name, arr, got in (("k", k, r["dk"]), ("v", v, r["dv"])):
                        for d in range(arr.shape[3]):
                            arr[b, j, g, d] += h_fd
                            lp = _loss(orc, q, k, v, do, alpha, **kw)
                            arr[b, j, g, d] -= 2 * h_fd
                            lm = _loss(orc, q, k, v, do, alpha, **kw)
                            arr[b, j, g, d] += h_fd
                            _close(got[n, d], (lp - lm) / (2 * h_fd), 1e-6, 1e-8, f"keys d{name} {ci} {st}")


# ---- packed (THD) inputs ---------------------------------------------------
#
# Segments b = 0 .. B-1 occupy tokens off[b] .. off[b+1]-1 of the packed axis;
# the first seqlens[b] of them are valid.  Cases: segments of unequal size,
# one with padding inside, one empty, and tokens past the last segment.
PACKED_CASES = [
    # offsets, seqlens, T, causal, window
    ([0, 5, 12, 12, 16], [5, 4, 0, 4], 18, True, (-1, -1)),
    ([0, 7, 9], None, 9, False, (2, 1)),
    ([0, 3, 11], [3, 6], 11, True, (2, 0)),
]


def _packed_case(seed, T, B, Hq=4, Hkv=2, dqk=4, dv=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, Hq, dqk)), rng.standard_normal((T, Hkv, dqk)),
            rng.standard_normal((T, Hkv, dv)), rng.standard_normal((T, Hq, dv)), rng.standard_normal(Hq))


def pin_packed_brute_force(orc):
    """Packed forward vs scalar loops that walk each segment's tokens directly."""
    for ci, (off, sl, T, causal, (wl, wr)) in enumerate(PACKED_CASES):
        B = len(off) - 1
        S = max(off[b + 1] - off[b] for b in range(B))
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = _packed_case(1500 + ci, T, B)
            Hq, Hkv, dv = q.shape[1], k.shape[1], v.shape[2]
            r = orc.attention_packed(q, k, v, None, seq_offsets=np.array(off), max_seqlen=S,
                                     seqlens=None if sl is None else np.array(sl), num_gqa_groups=Hkv,
                                     causal=causal, window=(wl, wr), scale_factor=0.45, softmax_type=st,
                                     softmax_offset=alpha)
            o = np.zeros((T, Hq, dv))
            lse = np.zeros((B, Hq, S))
            for b in range(B):
                n = off[b + 1] - off[b]
                L = n if sl is None else min(sl[b], n)
                for h in range(Hq):
                    g = h // (Hq // Hkv)
                    for i in range(S):
                        den, num = 0.0, [0.0] * dv
                        for j in range(L if i < L else 0):
                            if (causal and j > i) or (wl >= 0 and j < i - wl) or (wr >= 0 and j > i + wr):
                                continue
                            e = math.exp(0.45 * sum(q[off[b] + i, h, d] * k[off[b] + j, g, d] for d in range(q.shape[2])))
                            den += e
                            for d in range(dv):
                                num[d] += e * v[off[b] + j, g, d]
                        if st == "off_by_one":
                            den += 1.0
                        elif st == "learnable":
                            den += math.exp(alpha[h])
                        lse[b, h, i] = math.log(den) if den > 0 else -math.inf
                        if i < n:
                            o[off[b] + i, h, :] = [x / den if den > 0 else 0.0 for x in num]
            _close(r["o"], o, 1e-12, 1e-14, f"packed O case{ci} {st}")
            _close(r["lse"], lse, 1e-12, 1e-14, f"packed LSE case{ci} {st}")


def pin_packed_equals_padded(orc):
    """Packed (block-diagonal mask over the token axis) == padded BSHD per batch.

    The two oracle paths are different formulations of the same function:
    scattering each segment into row b of a [B, S, ...] tensor with
    seqlens[b] valid rows must give identical outputs and gradients."""
    for ci, (off, sl, T, causal, win) in enumerate(PACKED_CASES):
        B = len(off) - 1
        S = max(off[b + 1] - off[b] for b in range(B))
        lens = [min(off[b + 1] - off[b], S if sl is None else sl[b]) for b in range(B)]
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = _packed_case(1600 + ci, T, B)

            def pad(x):
                y = np.zeros((B, S) + x.shape[1:])
                for b in range(B):
                    y[b, :off[b + 1] - off[b]] = x[off[b]:off[b + 1]]
                return y

            kw = dict(num_gqa_groups=k.shape[1], causal=causal, window=win, scale_factor=0.7,
                      softmax_type=st, softmax_offset=alpha)
            rp = orc.attention_packed(q, k, v, do, seq_offsets=np.array(off), max_seqlen=S,
                                      seqlens=None if sl is None else np.array(sl), **kw)
            rb = orc.attention(pad(q), pad(k), pad(v), pad(do), seqlens=np.array(lens), **kw)
            for name in ("o", "dq", "dk", "dv"):
                _close(pad(rp[name]), rb[name], 1e-12, 1e-14, f"packed vs padded {name} case{ci} {st}")
                outside = np.ones(T, dtype=bool)
                outside[off[0]:off[-1]] = False
                assert not rp[name][outside].any(), f"tokens outside segments written: {name}"
            _close(rp["lse"], rb["lse"], 1e-12, 1e-14, f"packed vs padded lse case{ci} {st}")
            if st == "vanilla":
                assert rp["dalpha"] is None
            else:
                _close(rp["dalpha"], rb["dalpha"], 1e-12, 1e-14, f"packed vs padded dalpha case{ci} {st}")


def pin_packed_finite_diff(orc):
    """Packed dQ, dK, dV, d(alpha) vs central differences of sum(dO * O)."""
    hstep = 1e-6
    off, sl, T = [0, 3, 7], [3, 3], 8
    for st in orc.SOFTMAX_TYPES:
        q, k, v, do, alpha = _packed_case(1700, T, 2, dqk=2, dv=2)
        kw = dict(seq_offsets=np.array(off), max_seqlen=4, seqlens=np.array(sl), num_gqa_groups=2,
                  causal=True, window=(1, 0), scale_factor=0.8, softmax_type=st)

        def loss(qq, kk, vv, al):
            return float((orc.attention_packed(qq, kk, vv, None, softmax_offset=al, **kw)["o"] * do).sum())

        r = orc.attention_packed(q, k, v, do, softmax_offset=alpha, **kw)
        for name, arr, grad in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                a0 = arr[idx]
                arr[idx] = a0 + hstep
                lp = loss(q, k, v, alpha)
                arr[idx] = a0 - hstep
                lm = loss(q, k, v, alpha)
                arr[idx] = a0
                fd[idx] = (lp - lm) / (2 * hstep)
            _close(grad, fd, 1e-6, 1e-8, f"packed d{name} {st}")
        if st == "learnable":
            fd = np.zeros(alpha.size)
            for hh in range(alpha.size):
                a2 = alpha.copy()
                a2[hh] += hstep
                lp = loss(q, k, v, a2)
                a2[hh] -= 2 * hstep
                lm = loss(q, k, v, a2)
                fd[hh] = (lp - lm) / (2 * hstep)
            _close(r["dalpha"], fd, 1e-6, 1e-8, "packed dalpha")


# ---- attention dropout -----------------------------------------------------

def pin_philox_kat(orc):
    """Philox4x32-10 against the generator's published known-answer vectors."""
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for vec in kat["vectors"]:
        c = [int(x, 16) for x in vec["counter"]]
        k = [int(x, 16) for x in vec["key"]]
        got = [int(x) for x in orc.philox4x32_10(*c, *k)]
        assert got == [int(x, 16) for x in vec["output"]], (vec, [hex(x) for x in got])


def pin_dropout_rate(orc):
    """Kept fraction within 5 sigma of 1 - t/256; rows, keys, heads and
    offsets draw different bytes (no repeated 4 x 4 block)."""
    for p in (0.1, 0.5, 0.9):
        t = orc.dropout_threshold(p)
        keeps = [orc.dropout_keep(b, h, np.arange(64), np.arange(64), num_heads=3, p=p, seed=0x1234567890,
                                  offset=off) for b in range(2) for h in range(3) for off in (0, 7)]
        frac = float(np.mean(keeps))
        n = sum(x.size for x in keeps)
        q = 1.0 - t / 256.0
        assert abs(frac - q) <= 5 * math.sqrt(q * (1 - q) / n), (p, frac, q)
        flat = [x.tobytes() for x in keeps]
        assert len(set(flat)) == len(flat), "two (batch, head, offset) streams coincide"
        if p == 0.5:  # 256 blocks of 16 fair bits: a few repeats at most
            blocks = {keeps[0][r:r + 4, c:c + 4].tobytes() for r in range(0, 64, 4) for c in range(0, 64, 4)}
            assert len(blocks) > 245, "4 x 4 blocks repeat"
    assert orc.dropout_threshold(0.0) == 0 and orc.dropout_threshold(0.5) == 128
    assert orc.dropout_keep(0, 0, np.arange(8), np.arange(8), num_heads=1, p=0.0, seed=5, offset=0).all()


def pin_dropout_brute(orc):
    """Dropout forward vs scalar loops over the definition with the keep mask
    applied by hand (inverted dropout on the probabilities)."""
    for ci, (causal, win, sl) in enumerate(MASK_CASES[:4]):
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(1800 + ci)
            kw = dict(num_gqa_groups=2, causal=causal, window=win, scale_factor=0.41, softmax_type=st,
                      softmax_offset=alpha, seqlens=None if sl is None else np.array(sl))
            r = orc.attention_dropout(q, k, v, None, p=0.3, seed=99, offset=3, **kw)
            base = orc.attention(q, k, v, None, **kw)
            zs = 1.0 / (1.0 - orc.dropout_threshold(0.3) / 256.0)
            B, S, Hq = q.shape[:3]
            o = np.zeros_like(r["o"])
            for b in range(B):
                for h in range(Hq):
                    keep = orc.dropout_keep(b, h, np.arange(S), np.arange(S), num_heads=Hq, p=0.3, seed=99,
                                            offset=3)
                    for i in range(S):
                        for j in range(S):
                            if not np.isfinite(base["lse"][b, h, i]):
                                continue
                            pij = math.exp(0.41 * float(q[b, i, h] @ k[b, j, h // 2]) - base["lse"][b, h, i])
                            vis = (sl is None or (i < sl[b] and j < sl[b])) and (not causal or j <= i) and \
                                (win[0] < 0 or j >= i - win[0]) and (win[1] < 0 or j <= i + win[1])
                            if vis and keep[i, j]:
                                o[b, i, h] += pij * zs * v[b, j, h // 2]
            _close(r["o"], o, 1e-12, 1e-14, f"dropout O case{ci} {st}")
            _close(r["lse"], base["lse"], 0, 0, "dropout leaves the LSE unchanged")


def pin_dropout_p0(orc):
    """p = 0 keeps every pair: identical to attention() in every output."""
    q, k, v, do, alpha = rand_case(1900)
    kw = dict(num_gqa_groups=2, causal=True, window=(3, 0), scale_factor=0.5, softmax_type="learnable",
              softmax_offset=alpha, seqlens=np.array([9, 6]))
    r = orc.attention_dropout(q, k, v, do, p=0.0, seed=1, offset=0, **kw)
    base = orc.attention(q, k, v, do, **kw)
    for n in ("o", "lse", "dq", "dk", "dv", "dalpha"):
        _close(r[n], base[n], 0, 0, f"p=0 {n}")


def pin_dropout_finite_diff(orc):
    """Dropout dQ, dK, dV, d(alpha) vs central differences (the mask is a
    fixed function of the seed, so the loss is differentiable)."""
    hstep = 1e-6
    for st in orc.SOFTMAX_TYPES:
        q, k, v, do, alpha = rand_case(2000, B=1, S=6, Hq=2, Hkv=1, dqk=2, dv=2)
        kw = dict(p=0.45, seed=0xABCDEF12345, offset=11, num_gqa_groups=1, causal=False, window=(3, 1),
                  scale_factor=0.7, softmax_type=st, seqlens=np.array([5]))

        def loss(qq, kk, vv, al):
            return float((orc.attention_dropout(qq, kk, vv, None, softmax_offset=al, **kw)["o"] * do).sum())

        r = orc.attention_dropout(q, k, v, do, softmax_offset=alpha, **kw)
        assert 0 < r["keep"].mean() < 1
        for name, arr, grad in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                a0 = arr[idx]
                arr[idx] = a0 + hstep
                lp = loss(q, k, v, alpha)
                arr[idx] = a0 - hstep
                lm = loss(q, k, v, alpha)
                arr[idx] = a0
                fd[idx] = (lp - lm) / (2 * hstep)
            _close(grad, fd, 1e-6, 1e-8, f"dropout d{name} {st}")
        if st == "learnable":
            fd = np.zeros(alpha.size)
            for hh in range(alpha.size):
                a2 = alpha.copy()
                a2[hh] += hstep
                lp = loss(q, k, v, a2)
                a2[hh] -= 2 * hstep
                lm = loss(q, k, v, a2)
                fd[hh] = (lp - lm) / (2 * hstep)
            _close(r["dalpha"], fd, 1e-6, 1e-8, "dropout dalpha")


def pin_dropout_mean(orc):
    """Inverted dropout is unbiased: O averaged over many offsets approaches
    the undropped O (200 draws; loose bound)."""
    q, k, v, do, alpha = rand_case(2100, B=1, S=8, Hq=2, Hkv=1)
    kw = dict(num_gqa_groups=1, causal=True, scale_factor=0.5)
    base = orc.attention(q, k, v, None, **kw)["o"]
    acc = np.zeros_like(base)
    n = 200
    for off in range(n):
        acc += orc.attention_dropout(q, k, v, None, p=0.25, seed=3, offset=off, **kw)["o"]
    err = np.abs(acc / n - base).max()
    assert err < 0.15 * np.abs(base).max() + 0.05, err


def pin_dropout_layout(orc):
    """The documented pair -> generator-byte layout, spelled out: pair (i, j)
    of (b, h) takes byte (i % 4) * 4 + j % 4 (word byte // 4, bits 8 (byte % 4)
    up) of the call with counter (j // 4, i // 4, b * Hq + h, offset) and the
    seed as key (low word first)."""
    seed, offset, Hq, p = 0x0123456789ABCDEF, 77, 3, 0.5
    t = orc.dropout_threshold(p)
    keep = orc.dropout_keep(1, 2, np.arange(12), np.arange(20), num_heads=Hq, p=p, seed=seed, offset=offset)
    for i in range(12):
        for j in range(20):
            words = orc.philox4x32_10(j // 4, i // 4, 1 * Hq + 2, offset, seed & 0xFFFFFFFF, seed >> 32)
            byte_no = (i % 4) * 4 + j % 4
            byte = (int(words[byte_no // 4]) >> (8 * (byte_no % 4))) & 0xFF
            assert keep[i, j] == (byte >= t), (i, j)


def pin_dropout_sampled(orc):
    """Row- and key-sampled functions with dropout equal the whole-problem
    dropout oracle on those rows and keys (different code paths: masked
    column ranges and row blocks vs full S x S matrices)."""
    for ci, (causal, win, sl) in enumerate(MASK_CASES):
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(2200 + ci, B=2, S=9)
            kw = dict(num_gqa_groups=2, causal=causal, window=win, scale_factor=0.6, softmax_type=st,
                      softmax_offset=alpha, seqlens=None if sl is None else np.array(sl))
            drop = (0.35, 0xFEED + ci, 4)
            full = orc.attention_dropout(q, k, v, do, p=drop[0], seed=drop[1], offset=drop[2], **kw)
            for b in range(2):
                h = (b + ci) % 4
                rows = np.array([0, 3, 8])
                r = orc.attention_rows(q, k, v, do, b=b, h=h, rows=rows, dropout=drop, **kw)
                _close(r["o"], full["o"][b, rows, h], 1e-12, 1e-14, f"rows O {ci} {st}")
                _close(r["dq"], full["dq"][b, rows, h], 1e-12, 1e-14, f"rows dQ {ci} {st}")
                g = h // 2
                keys = np.array([0, 4, 8])
                rk = orc.attention_keys(q, k, v, do, b=b, g=g, keys=keys, dropout=drop, row_block=2, **kw)
                _close(rk["dk"], full["dk"][b, keys, g], 1e-12, 1e-14, f"keys dK {ci} {st}")
                _close(rk["dv"], full["dv"][b, keys, g], 1e-12, 1e-14, f"keys dV {ci} {st}")


# ---- attention bias ---------------------------------------------------------

BIAS_SHAPES = [(2, 4), (1, 4), (2, 1), (1, 1)]  # [Bb, Hb] of a [Bb, Hb, S, S] bias, B = 2, Hq = 4


def pin_bias_torch(orc):
    """Bias forward and backward, every broadcast shape and softmax type, vs
    torch.nn.functional.scaled_dot_product_attention in float64 with the bias
    (plus the mask as -inf) as its additive float mask; the bias gradient is
    that mask's autograd gradient summed over the shared dimensions."""
    import torch
    F = torch.nn.functional
    B, S, Hq, Hkv, dqk, dv = 2, 21, 4, 2, 8, 6
    win, sl = (7, 0), [21, 13]
    for si, (Bb, Hb) in enumerate(BIAS_SHAPES):
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(2300 + si, B, S, Hq, Hkv, dqk, dv)
            bias = np.random.default_rng(2400 + si).standard_normal((Bb, Hb, S, S))
            r = orc.attention(q, k, v, do, num_gqa_groups=Hkv, causal=True, window=win, softmax_type=st,
                              softmax_offset=alpha, seqlens=np.array(sl), bias=bias)
            G = Hq // Hkv
            tq = torch.tensor(q.transpose(0, 2, 1, 3), requires_grad=True)
            tk = torch.tensor(k.transpose(0, 2, 1, 3), requires_grad=True)
            tv = torch.tensor(v.transpose(0, 2, 1, 3), requires_grad=True)
            i, j = torch.arange(S)[:, None], torch.arange(S)[None, :]
            vis = torch.zeros(B, 1, S, S, dtype=torch.bool)
            dmask = torch.ones(B, 1, S, 1, dtype=torch.float64)
            for b in range(B):
                L = sl[b]
                vis[b, 0] = (i < L) & (j < L) & (j <= i) & (j >= i - win[0])
                dmask[b, 0, L:] = 0.0
            vis2 = vis.clone()
            vis2[:, :, :, 0] |= ~vis.any(dim=3)  # padded rows: one dummy key, zero upstream gradient
            tb = torch.tensor(bias, requires_grad=True)
            madd = torch.where(vis2, tb.expand(B, Hq, S, S), torch.tensor(-torch.inf, dtype=torch.float64))
            kr, vr = tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1)
            if st != "vanilla":
                z = torch.zeros(Hq, dtype=torch.float64) if st == "off_by_one" else torch.tensor(alpha)
                kr = torch.cat([kr, torch.zeros(B, Hq, 1, dqk, dtype=torch.float64)], dim=2)
                vr = torch.cat([vr, torch.zeros(B, Hq, 1, dv, dtype=torch.float64)], dim=2)
                madd = torch.cat([madd, z.view(1, Hq, 1, 1).expand(B, Hq, S, 1)], dim=3)
            o = F.scaled_dot_product_attention(tq, kr, vr, attn_mask=madd, scale=1.0 / math.sqrt(dqk))
            o.backward(torch.tensor(do.transpose(0, 2, 1, 3)) * dmask)
            o_np = o.detach().numpy().transpose(0, 2, 1, 3)
            for b in range(B):
                _close(r["o"][b, :sl[b]], o_np[b, :sl[b]], 1e-10, 1e-12, f"bias O {Bb}x{Hb} {st}")
            _close(r["dq"], tq.grad.numpy().transpose(0, 2, 1, 3), 1e-10, 1e-12, f"bias dQ {Bb}x{Hb} {st}")
            _close(r["dk"], tk.grad.numpy().transpose(0, 2, 1, 3), 1e-10, 1e-12, f"bias dK {Bb}x{Hb} {st}")
            _close(r["dv"], tv.grad.numpy().transpose(0, 2, 1, 3), 1e-10, 1e-12, f"bias dV {Bb}x{Hb} {st}")
            _close(r["dbias"], tb.grad.numpy(), 1e-10, 1e-12, f"dbias {Bb}x{Hb} {st}")


def pin_bias_invariants(orc):
    """Zero bias == no bias; a bias constant along each row changes nothing
    for vanilla softmax (shift invariance) and its gradient's rows sum to 0;
    the bias gradient vanishes on pairs the mask hides."""
    q, k, v, do, alpha = rand_case(2500)
    kw = dict(num_gqa_groups=2, causal=True, window=(4, 0), scale_factor=0.5, seqlens=np.array([9, 6]))
    for st in orc.SOFTMAX_TYPES:
        base = orc.attention(q, k, v, do, softmax_type=st, softmax_offset=alpha, **kw)
        r0 = orc.attention(q, k, v, do, softmax_type=st, softmax_offset=alpha, bias=np.zeros((1, 1, 9, 9)), **kw)
        for n in ("o", "lse", "dq", "dk", "dv"):
            _close(r0[n], base[n], 0, 0, f"zero bias {n} {st}")
    base = orc.attention(q, k, v, do, **kw)
    rowc = np.random.default_rng(2501).standard_normal((2, 4, 9, 1)) * np.ones((1, 1, 1, 9))
    r = orc.attention(q, k, v, do, bias=rowc, **kw)
    for n in ("o", "dq", "dk", "dv"):
        _close(r[n], base[n], 1e-12, 1e-14, f"row-constant bias {n}")
    _close(r["dbias"].sum(axis=3), np.zeros((2, 4, 9)), 0, 1e-12, "dbias row sums")
    for b, L in enumerate([9, 6]):
        vis = orc.visible_mask(9, L, True, 4, 0)
        assert not r["dbias"][b][:, ~vis].any(), "dbias on hidden pairs"


def pin_bias_finite_diff(orc):
    """The bias gradient (shared over the batch) vs central differences."""
    hstep = 1e-6
    for st in orc.SOFTMAX_TYPES:
        q, k, v, do, alpha = rand_case(2600, B=2, S=5, Hq=2, Hkv=1, dqk=3, dv=2)
        bias = np.random.default_rng(2601).standard_normal((1, 2, 5, 5))
        kw = dict(num_gqa_groups=1, causal=False, window=(2, 1), scale_factor=0.7, softmax_type=st,
                  softmax_offset=alpha, seqlens=np.array([5, 4]))
        r = orc.attention(q, k, v, do, bias=bias, **kw)
        fd = np.zeros_like(bias)
        for idx in np.ndindex(bias.shape):
            b0 = bias[idx]
            bias[idx] = b0 + hstep
            lp = float((orc.attention(q, k, v, None, bias=bias, **kw)["o"] * do).sum())
            bias[idx] = b0 - hstep
            lm = float((orc.attention(q, k, v, None, bias=bias, **kw)["o"] * do).sum())
            bias[idx] = b0
            fd[idx] = (lp - lm) / (2 * hstep)
        _close(r["dbias"], fd, 1e-6, 1e-8, f"dbias finite differences {st}")


def pin_bias_sampled(orc):
    """Row- and key-sampled functions with a bias equal the whole-problem bias
    oracle (itself pinned against torch SDPA above): O, LSE, dQ and the rows'
    dS (the bias gradient of a full-shape bias) per row; dK, dV per key."""
    for ci, (causal, win, sl) in enumerate(MASK_CASES):
        for st in orc.SOFTMAX_TYPES:
            q, k, v, do, alpha = rand_case(2700 + ci)
            for si, (Bb, Hb) in enumerate(BIAS_SHAPES):
                bias = np.random.default_rng(2750 + 4 * ci + si).standard_normal((Bb, Hb, 9, 9))
                kw = dict(num_gqa_groups=2, causal=causal, window=win, scale_factor=0.45, softmax_type=st,
                          softmax_offset=alpha, seqlens=None if sl is None else np.array(sl), bias=bias)
                full = orc.attention(q, k, v, do, **kw)
                for b in range(2):
                    for h in (1, 2):
                        rows = [0, 4, 8, 2] if ci % 2 else [8, 1, 5]
                        r = orc.attention_rows(q, k, v, do, b=b, h=h, rows=rows, **kw)
                        _close(r["o"], full["o"][b, rows, h], 1e-12, 1e-14, f"bias rows O {ci} {st}")
                        _close(r["lse"], full["lse"][b, h, rows], 1e-12, 1e-14, f"bias rows LSE {ci} {st}")
                        _close(r["dq"], full["dq"][b, rows, h], 1e-12, 1e-14, f"bias rows dQ {ci} {st}")
                        if (Bb, Hb) == (2, 4):
                            ds = np.zeros((len(rows), 9))
                            ds[:, r["cols"][0]:r["cols"][1]] = r["ds"]
                            _close(ds, full["dbias"][b, h, rows], 1e-12, 1e-14, f"bias rows dS {ci} {st}")
                    g = (b + ci) % 2
                    keys = [7, 0, 3] if ci % 2 else [5, 2]
                    rk = orc.attention_keys(q, k, v, do, b=b, g=g, keys=keys, row_block=2, **kw)
                    _close(rk["dk"], full["dk"][b, keys, g], 1e-12, 1e-14, f"bias keys dK {ci} {st}")
                    _close(rk["dv"], full["dv"][b, keys, g], 1e-12, 1e-14, f"bias keys dV {ci} {st}")


ALL_PINS = [pin_brute_force, pin_finite_diff, pin_row_sums, pin_gqa_repeat, pin_causal_rows,
            pin_sink_augmented, pin_sink_closed, pin_dalpha_forms, pin_padding,
            pin_window_limits, pin_scale, pin_torch_sdpa, pin_golden, pin_sampled_rows,
            pin_sampled_keys, pin_packed_brute_force, pin_packed_equals_padded, pin_packed_finite_diff,
            pin_philox_kat, pin_dropout_rate, pin_dropout_brute, pin_dropout_p0, pin_dropout_finite_diff,
            pin_dropout_mean, pin_dropout_layout,
            pin_dropout_sampled, pin_bias_torch, pin_bias_invariants, pin_bias_finite_diff, pin_bias_sampled]
