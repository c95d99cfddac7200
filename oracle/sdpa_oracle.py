"""Float64 CPU oracle for fused scaled dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  This module is the independent reference that the
HIP kernels are checked against.  Only the test suite, the smoke entry point
and the CPU-baseline leg of the benchmark may import or call it; the library's
product path never does.  It shares no code, constant or helper with the HIP
path and imports nothing from it.

What it computes (plain definitions, written out; one (batch, head) at a time,
materialising the whole S x S score matrix exactly as the naive attention of
the codelab "Speed up attention on GPU with cuDNN and TransformerEngine",
section 4 "Implement attention from scratch", does):

  * scores  s_ij = scale * q_i . k_j                 (codelab, "How attention works",
                                                      steps 1-2; scale defaults to
                                                      1/sqrt(d_qk): TransformerEngine
                                                      "JAX: Single-GPU Attention",
                                                      "Other attention knobs", score scaling)
  * mask    causal / sliding window / padding        (TE single-GPU page, sections 1-2;
                                                      codelab section 7)
  * softmax vanilla, off-by-one or learnable sink     (PR "[JAX] Add support for sink
                                                      attention in JAX" #2225, the
                                                      softmax formulas in the review
                                                      summaries' sequence diagrams)
  * output  O = P V                                  (codelab, "How attention works", step 3)
  * LSE     natural-log log-sum-exp of each row, sink term included
  * grads   dQ, dK, dV of L = sum(dO * O), and the gradient of the sink logit
            (PR #2225: the backward returns grad_q, grad_k, grad_v and
            grad_softmax_offset)
  * packed  sequences back to back on one token axis (attention_packed: one
            block-diagonal mask over the axis; TE single-GPU page, section 1)
  * dropout inverted dropout on the probabilities with a Philox4x32-10 keep
            mask (attention_dropout; TE single-GPU page, "Other attention
            knobs"; the generator and its layout are readings, stated below)

Readings taken where the pages are silent or disagree (each also listed in the
design notes):
  * off-by-one softmax = one extra logit of value 0 (denominator 1 + sum exp);
    PR #2225 review thread on the Softmax module offset settles 0, not 1.
  * learnable softmax: softmax_offset holds the raw logit alpha_h per query head;
    denominator adds exp(alpha_h), unscaled by scale_factor.
  * GQA: query head h reads kv head floor(h / (Hq/Hkv)) (K/V heads repeated, TE
    single-GPU page section 1; codelab section 9 "each shared by 4 query heads").
  * window (left, right) is inclusive: key j is visible from row i iff
    i-left <= j <= i+right; -1 means unbounded.
  * seqlens[b] right-pads both queries and keys; rows and keys at or beyond it
    are invisible.  Empty rows give O = 0, LSE = -inf (vanilla) or the sink logit.
"""
from __future__ import annotations

import math

import numpy as np

VANILLA = "vanilla"
OFF_BY_ONE = "off_by_one"
LEARNABLE = "learnable"
SOFTMAX_TYPES = (VANILLA, OFF_BY_ONE, LEARNABLE)


def kv_head(h: int, num_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h: contiguous groups of Hq/Hkv query heads.

    TE single-GPU page, section 1 (the baseline repeats K/V heads for GQA) and
    section 2 (num_gqa_groups = number of KV heads); codelab section 9.
    """
    return h // (num_heads // num_kv_heads)


def visible_mask(S: int, L: int, causal: bool, window_left: int, window_right: int) -> np.ndarray:
    """Boolean [S, S] matrix: True where query row i may attend to key j.

    Intersection of padding (i < L and j < L), the causal lower triangle
    (codelab section 7, j <= i) and the sliding window (TE single-GPU page
    section 2, window_size = (left, right), -1 unbounded).
    """
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = (i < L) & (j < L)
    if causal:
        m &= j <= i
    if window_left >= 0:
        m &= j >= i - window_left
    if window_right >= 0:
        m &= j <= i + window_right
    return m


def sink_logit(softmax_type: str, softmax_offset, h: int):
    """The extra softmax logit z for query head h, or None for vanilla.

    PR #2225 sequence diagrams: off-by-one adds 1 = exp(0) to the denominator,
    learnable adds exp(alpha[h]).
    """
    if softmax_type == VANILLA:
        return None
    if softmax_type == OFF_BY_ONE:
        return 0.0
    if softmax_type == LEARNABLE:
        return float(np.asarray(softmax_offset, dtype=np.float64).reshape(-1)[h])
    raise ValueError(f"unknown softmax_type {softmax_type!r}")


def _softmax_rows(s: np.ndarray, mask: np.ndarray, z):
    """Masked row softmax with optional sink logit z (a logit with no value row).

    Returns (P, LSE): P_ij = exp(s_ij - LSE_i) on visible entries, 0 elsewhere;
    LSE_i = log(sum_visible exp(s_ij) + [sink] exp(z)).
    """
    neg = np.where(mask, s, -np.inf)
    m = neg.max(axis=1)
    if z is not None:
        m = np.maximum(m, z)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(mask, np.exp(neg - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    if z is not None:
        l = l + np.exp(z - m_safe)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m_safe + np.log(l), -np.inf)
    lse_safe = np.where(np.isfinite(lse), lse, 0.0)
    p = np.where(mask, np.exp(neg - lse_safe[:, None]), 0.0)
    return p, lse


def _resolve(q, k, v, num_gqa_groups, scale_factor):
    B, S, Hq, dqk = q.shape
    Hkv = k.shape[2] if num_gqa_groups is None else int(num_gqa_groups)
    if k.shape != (B, S, Hkv, dqk) or v.shape[:3] != (B, S, Hkv):
        raise ValueError("K/V shapes do not match Q and num_gqa_groups")
    if Hq % Hkv:
        raise ValueError("num_heads must be a multiple of num_gqa_groups")
    scale = (1.0 / math.sqrt(dqk)) if not scale_factor else float(scale_factor)
    return B, S, Hq, Hkv, dqk, v.shape[3], scale


def _bias_index(bias, b, h):
    """Indices of batch b, query head h into a [Bb, Hb, S, S] bias (Bb, Hb = 1 broadcast)."""
    return (b if bias.shape[0] > 1 else 0), (h if bias.shape[1] > 1 else 0)


def attention_group(q, k, v, d_o, *, b, g, num_gqa_groups=None, causal=True,
                    window=(-1, -1), scale_factor=None, softmax_type=VANILLA,
                    softmax_offset=None, seqlens=None, want_grads=True, bias=None):
    """Forward (and backward) for one batch b and one KV head g, in float64.

    Computes every query head of the group.  Returns a dict with
      o    [S, G, dv]   lse [G, S]   (forward)
      dq   [S, G, dqk]  dk  [S, dqk]  dv [S, dv]
      dz   [G]          this batch's share of d(sink logit) per query head
      ds   [G, S, S]    dS per query head (with bias, for its gradient)
    Inputs may be any float dtype; they are upcast to float64 exactly.  bias:
    an additive post-scale bias [Bb, Hb, S, S] (Bb in {1, B}, Hb in {1, Hq};
    see attention()).
    """
    B, S, Hq, Hkv, dqk, dv_dim, scale = _resolve(q, k, v, num_gqa_groups, scale_factor)
    G = Hq // Hkv
    L = S if seqlens is None else int(np.asarray(seqlens).reshape(-1)[b])
    mask = visible_mask(S, L, causal, int(window[0]), int(window[1]))
    kb = np.asarray(k[b, :, g, :], dtype=np.float64)
    vb = np.asarray(v[b, :, g, :], dtype=np.float64)
    out = {"o": np.zeros((S, G, dv_dim)), "lse": np.zeros((G, S))}
    if want_grads:
        out.update(dq=np.zeros((S, G, dqk)), dk=np.zeros((S, dqk)),
                   dv=np.zeros((S, dv_dim)), dz=np.zeros(G))
    for gi in range(G):
        h = g * G + gi
        assert kv_head(h, Hq, Hkv) == g
        qh = np.asarray(q[b, :, h, :], dtype=np.float64)
        z = sink_logit(softmax_type, softmax_offset, h)
        s = scale * (qh @ kb.T)                       # score + scale
        if bias is not None:
            s = s + np.asarray(bias[_bias_index(bias, b, h)], dtype=np.float64)
        p, lse = _softmax_rows(s, mask, z)            # softmax (+ sink)
        o = p @ vb                                    # attend
        out["o"][:, gi, :] = o
        out["lse"][gi] = lse
        if not want_grads:
            continue
        doh = np.asarray(d_o[b, :, h, :], dtype=np.float64)
        dp = doh @ vb.T                               # dL/dP
        delta = (doh * o).sum(axis=1)                 # rowsum(dO * O) = sum_j P_ij dP_ij
        ds = p * (dp - delta[:, None])                # softmax Jacobian applied to dP
        if bias is not None:
            out.setdefault("ds", np.zeros((G, S, S)))[gi] = ds
        out["dq"][:, gi, :] = scale * (ds @ kb)
        out["dk"] += scale * (ds.T @ qh)
        out["dv"] += p.T @ doh
        if z is not None:
            # dL/dz_i = -p_sink,i * delta_i with p_sink,i = exp(z - LSE_i):
            # the sink enters only the denominator and carries a zero value row.
            lse_safe = np.where(np.isfinite(lse), lse, z)
            out["dz"][gi] = -(np.exp(z - lse_safe) * delta).sum()
    return out


def attention(q, k, v, d_o=None, *, num_gqa_groups=None, causal=True, window=(-1, -1),
              scale_factor=None, softmax_type=VANILLA, softmax_offset=None, seqlens=None, bias=None):
    """Whole-problem oracle (small shapes): assembles every (batch, kv head) group.

    Returns dict o [B,S,Hq,dv], lse [B,Hq,S] and, when d_o is given,
    dq [B,S,Hq,dqk], dk [B,S,Hkv,dqk], dv [B,S,Hkv,dv], dalpha [Hq]
    (dalpha is None for vanilla softmax) and dbias (None without bias).

    bias: attention bias, read as an additive post-scale bias on the visible
    scores, s_ij = scale q_i.k_j + bias[b, h, i, j], of shape [Bb, Hb, S, S]
    with Bb in {1, B} and Hb in {1, Hq} (1 = shared, broadcast).  The TE
    single-GPU page ("Other attention knobs") passes a bias with a bias type,
    and the PR #2225 backward returns grad_bias; the reading: the gradient is
    dS = P (dP - delta), summed over the dimensions the bias is shared along,
    and zero on pairs the mask hides.
    """
    B, S, Hq, Hkv, dqk, dv_dim, _ = _resolve(q, k, v, num_gqa_groups, scale_factor)
    G = Hq // Hkv
    grads = d_o is not None
    res = {"o": np.zeros((B, S, Hq, dv_dim)), "lse": np.zeros((B, Hq, S))}
    if grads:
        res.update(dq=np.zeros((B, S, Hq, dqk)), dk=np.zeros((B, S, Hkv, dqk)),
                   dv=np.zeros((B, S, Hkv, dv_dim)), dalpha=np.zeros(Hq),
                   dbias=None if bias is None else np.zeros(np.shape(bias)))
    if bias is not None and (np.ndim(bias) != 4 or np.shape(bias)[0] not in (1, B) or
                             np.shape(bias)[1] not in (1, Hq) or np.shape(bias)[2:] != (S, S)):
        raise ValueError("bias must have shape [1 or B, 1 or Hq, S, S]")
    for b in range(B):
        for g in range(Hkv):
            r = attention_group(q, k, v, d_o, b=b, g=g, num_gqa_groups=Hkv, causal=causal,
                                window=window, scale_factor=scale_factor,
                                softmax_type=softmax_type, softmax_offset=softmax_offset,
                                seqlens=seqlens, want_grads=grads, bias=bias)
            hs = slice(g * G, (g + 1) * G)
            res["o"][b, :, hs, :] = r["o"]
            res["lse"][b, hs, :] = r["lse"]
            if grads:
                res["dq"][b, :, hs, :] = r["dq"]
                res["dk"][b, :, g, :] = r["dk"]
                res["dv"][b, :, g, :] = r["dv"]
                res["dalpha"][hs] += r["dz"]
                if bias is not None:
                    for gi in range(G):
                        res["dbias"][_bias_index(bias, b, g * G + gi)] += r["ds"][gi]
    if grads and softmax_type == VANILLA:
        res["dalpha"] = None
    return res


def visible_pairs(S: int, L: int, causal: bool, window_left: int, window_right: int) -> int:
    """Number of visible (query, key) pairs of one (batch, head), in closed form.

    Row i < L sees keys max(0, i-left) .. min(L-1, i [causal], i+right).
    """
    total = 0
    for i in range(min(L, S)):
        hi = L - 1
        if causal:
            hi = min(hi, i)
        if window_right >= 0:
            hi = min(hi, i + window_right)
        lo = max(0, i - window_left) if window_left >= 0 else 0
        total += max(0, hi - lo + 1)
    return total


def visible_rows(rows, S: int, L: int, causal: bool, window_left: int, window_right: int,
                 cols=None) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: the visible_mask definition for selected
    query rows and keys (all S keys when cols is None)."""
    i = np.asarray(rows)[:, None]
    j = (np.arange(S) if cols is None else np.asarray(cols))[None, :]
    m = (i < L) & (j < L)
    if causal:
        m = m & (j <= i)
    if window_left >= 0:
        m = m & (j >= i - window_left)
    if window_right >= 0:
        m = m & (j <= i + window_right)
    return m


def attention_rows(q, k, v, d_o, *, b, h, rows, num_gqa_groups=None, causal=True, window=(-1, -1),
                   scale_factor=None, softmax_type=VANILLA, softmax_offset=None, seqlens=None, dropout=None,
                   bias=None):
    """Outputs of selected query rows of one (batch b, query head h), in float64.

    A row's output, LSE, delta and dQ depend only on that row's visible keys,
    so rows can be computed one by one at any sequence length.  Columns where
    the row mask is zero for every selected row are left out: they contribute
    exactly zero.  Returns o [n, dv], lse [n], delta [n], dq [n, dqk] and
    dz [n] = -exp(z - LSE_i) * delta_i (0 for vanilla).  dropout = (p, seed,
    offset) applies attention dropout as attention_dropout does.  bias: the
    additive post-scale bias of attention() ([Bb, Hb, S, S]); with it, ds
    [n, c1 - c0] holds the rows' dS on keys c0 .. c1-1 (cols = (c0, c1)), zero
    on every other key.
    """
    B, S, Hq, Hkv, dqk, dv_dim, scale = _resolve(q, k, v, num_gqa_groups, scale_factor)
    g = kv_head(h, Hq, Hkv)
    L = S if seqlens is None else int(np.asarray(seqlens).reshape(-1)[b])
    rows = np.asarray(rows, dtype=np.int64)
    # keys outside [min row - left, max row + right] fail the window rule for
    # every selected row; the mask definition is evaluated on the rest
    lo = max(0, int(rows.min()) - int(window[0])) if window[0] >= 0 and rows.size else 0
    hi = min(S, int(rows.max()) + int(window[1]) + 1) if window[1] >= 0 and rows.size else S
    lo, hi = (lo, hi) if lo < hi else (0, 1)
    mask = visible_rows(rows, S, L, causal, int(window[0]), int(window[1]), cols=np.arange(lo, hi))
    cols = np.nonzero(mask.any(axis=0))[0]
    c0, c1 = (int(cols[0]), int(cols[-1]) + 1) if cols.size else (0, 1)  # one fully masked column
    mask = mask[:, c0:c1]
    c0, c1 = c0 + lo, c1 + lo
    kb = np.asarray(k[b, c0:c1, g, :], dtype=np.float64)
    vb = np.asarray(v[b, c0:c1, g, :], dtype=np.float64)
    qh = np.asarray(q[b, rows, h, :], dtype=np.float64)
    doh = np.asarray(d_o[b, rows, h, :], dtype=np.float64)
    z = sink_logit(softmax_type, softmax_offset, h)
    s = scale * (qh @ kb.T)
    if bias is not None:
        s = s + np.asarray(bias[_bias_index(bias, b, h)][rows][:, c0:c1], dtype=np.float64)
    p, lse = _softmax_rows(s, mask, z)
    zmat = _dropout_factors(dropout, b, h, Hq, rows, np.arange(c0, c1))
    o = (p * zmat) @ vb
    delta = (doh * o).sum(axis=1)
    ds = p * (zmat * (doh @ vb.T) - delta[:, None])
    dq = scale * (ds @ kb)
    if z is None:
        dz = np.zeros(len(rows))
    else:
        dz = -np.exp(z - np.where(np.isfinite(lse), lse, z)) * delta
    return {"o": o, "lse": lse, "delta": delta, "dq": dq, "dz": dz, "ds": ds, "cols": (c0, c1)}


def attention_keys(q, k, v, d_o, *, b, g, keys, num_gqa_groups=None, causal=True, window=(-1, -1),
                   scale_factor=None, softmax_type=VANILLA, softmax_offset=None, seqlens=None,
                   row_block=1024, dropout=None, bias=None):
    """dK, dV of selected keys of one (batch b, KV head g), in float64.

    dK_j = scale * sum_h sum_i dS_ij Q_i and dV_j = sum_h sum_i P_ij dO_i over
    the query heads h of the group and every row i that sees key j; each such
    row's LSE and delta come from attention_rows.  Returns dk [n, dqk], dv [n, dv].
    bias: the additive post-scale bias of attention().
    """
    B, S, Hq, Hkv, dqk, dv_dim, scale = _resolve(q, k, v, num_gqa_groups, scale_factor)
    G = Hq // Hkv
    L = S if seqlens is None else int(np.asarray(seqlens).reshape(-1)[b])
    keys = np.asarray(keys, dtype=np.int64)
    # rows that see any selected key: the mask definition on those key columns
    sees = visible_rows(np.arange(S), S, L, causal, int(window[0]), int(window[1]), cols=keys)
    rows_all = np.nonzero(sees.any(axis=1))[0]
    kk = np.asarray(k[b, keys, g, :], dtype=np.float64)
    vk = np.asarray(v[b, keys, g, :], dtype=np.float64)
    dk = np.zeros((len(keys), dqk))
    dvv = np.zeros((len(keys), dv_dim))
    kw = dict(num_gqa_groups=Hkv, causal=causal, window=window, scale_factor=scale_factor,
              softmax_type=softmax_type, softmax_offset=softmax_offset, seqlens=seqlens, dropout=dropout,
              bias=bias)
    # row blocks never straddle a gap in rows_all, so each block's key range
    # stays as narrow as the mask allows
    cuts = np.nonzero(np.diff(rows_all) > 1)[0] + 1
    blocks = [run[r0:r0 + row_block] for run in np.split(rows_all, cuts) for r0 in range(0, len(run), row_block)]
    for gi in range(G):
        h = g * G + gi
        for rows in blocks:
            rr = attention_rows(q, k, v, d_o, b=b, h=h, rows=rows, **kw)
            m = sees[rows]
            qh = np.asarray(q[b, rows, h, :], dtype=np.float64)
            doh = np.asarray(d_o[b, rows, h, :], dtype=np.float64)
            s = scale * (qh @ kk.T)
            if bias is not None:
                s = s + np.asarray(bias[_bias_index(bias, b, h)][rows][:, keys], dtype=np.float64)
            lse = np.where(np.isfinite(rr["lse"]), rr["lse"], 0.0)
            p = np.where(m, np.exp(np.where(m, s, 0.0) - lse[:, None]), 0.0)
            zmat = _dropout_factors(dropout, b, h, Hq, rows, keys)
            ds = p * (zmat * (doh @ vk.T) - rr["delta"][:, None])
            dk += scale * (ds.T @ qh)
            dvv += (p * zmat).T @ doh
    return {"dk": dk, "dv": dvv}


def packed_visible_mask(seq_offsets, seqlens, T: int, causal: bool, window_left: int,
                        window_right: int) -> np.ndarray:
    """Boolean [T, T] over the packed token axis: True where token t may attend to token u.

    Packed (THD) inputs: in the TE single-GPU page, section 1, the sequence
    descriptor tells the library, besides lengths, where packed sequences
    start and which of their tokens pad them.  Reading taken: segment b holds tokens seq_offsets[b] ..
    seq_offsets[b+1]-1, of which the first seqlens[b] are valid (all of them
    when seqlens is None) and the rest padding.  Token t may attend to token u
    iff both lie in the same segment, both are valid, and their positions
    inside the segment satisfy the causal and window rules.  Tokens outside
    every segment see nothing and are seen by nothing.
    """
    off = np.asarray(seq_offsets, dtype=np.int64).reshape(-1)
    B = off.size - 1
    seg = np.full(T, -1, dtype=np.int64)
    pos = np.zeros(T, dtype=np.int64)
    valid = np.zeros(T, dtype=bool)
    for b in range(B):
        n = int(off[b + 1] - off[b])
        L = n if seqlens is None else min(int(np.asarray(seqlens).reshape(-1)[b]), n)
        seg[off[b]:off[b + 1]] = b
        pos[off[b]:off[b + 1]] = np.arange(n)
        valid[off[b]:off[b] + L] = True
    same = (seg[:, None] == seg[None, :]) & (seg[:, None] >= 0)
    m = same & valid[:, None] & valid[None, :]
    pi, pj = pos[:, None], pos[None, :]
    if causal:
        m &= pj <= pi
    if window_left >= 0:
        m &= pj >= pi - window_left
    if window_right >= 0:
        m &= pj <= pi + window_right
    return m


def attention_packed(q, k, v, d_o=None, *, seq_offsets, max_seqlen, seqlens=None,
                     num_gqa_groups=None, causal=True, window=(-1, -1), scale_factor=None,
                     softmax_type=VANILLA, softmax_offset=None):
    """Oracle for packed (THD) inputs: one attention over the whole token axis.

    q [T,Hq,dqk], k [T,Hkv,dqk], v [T,Hkv,dv], d_o [T,Hq,dv]; the segments
    and their valid lengths come from seq_offsets [B+1] and seqlens [B] (see
    packed_visible_mask).  The T x T score matrix of each head is masked
    block-diagonally, then softmax (+ sink), attend and the gradients follow
    the same definitions as attention_group.  Returns o [T,Hq,dv],
    lse [B,Hq,max_seqlen] (row i of segment b; rows past the segment or its
    valid length are empty: -inf for vanilla, the sink logit otherwise), and
    with d_o: dq, dk, dv on the token axis and dalpha [Hq] (None for vanilla).
    Tokens outside every segment get zeros.
    """
    T, Hq, dqk = q.shape
    Hkv = k.shape[1] if num_gqa_groups is None else int(num_gqa_groups)
    if k.shape != (T, Hkv, dqk) or v.shape[:2] != (T, Hkv) or Hq % Hkv:
        raise ValueError("K/V shapes do not match Q and num_gqa_groups")
    dv_dim = v.shape[2]
    scale = (1.0 / math.sqrt(dqk)) if not scale_factor else float(scale_factor)
    off = np.asarray(seq_offsets, dtype=np.int64).reshape(-1)
    B = off.size - 1
    mask = packed_visible_mask(off, seqlens, T, causal, int(window[0]), int(window[1]))
    grads = d_o is not None
    res = {"o": np.zeros((T, Hq, dv_dim)), "lse": np.zeros((B, Hq, max_seqlen))}
    if grads:
        res.update(dq=np.zeros((T, Hq, dqk)), dk=np.zeros((T, Hkv, dqk)),
                   dv=np.zeros((T, Hkv, dv_dim)), dalpha=np.zeros(Hq))
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        z = sink_logit(softmax_type, softmax_offset, h)
        qh = np.asarray(q[:, h, :], dtype=np.float64)
        kg = np.asarray(k[:, g, :], dtype=np.float64)
        vg = np.asarray(v[:, g, :], dtype=np.float64)
        s = scale * (qh @ kg.T)
        p, lse_t = _softmax_rows(s, mask, z)
        o = p @ vg
        res["o"][:, h, :] = o
        empty = -np.inf if z is None else z
        res["lse"][:, h, :] = empty
        for b in range(B):
            n = min(int(off[b + 1] - off[b]), max_seqlen)
            res["lse"][b, h, :n] = lse_t[off[b]:off[b] + n]
        if not grads:
            continue
        doh = np.asarray(d_o[:, h, :], dtype=np.float64)
        delta = (doh * o).sum(axis=1)
        ds = p * (doh @ vg.T - delta[:, None])
        res["dq"][:, h, :] = scale * (ds @ kg)
        res["dk"][:, g, :] += scale * (ds.T @ qh)
        res["dv"][:, g, :] += p.T @ doh
        if z is not None:
            lse_safe = np.where(np.isfinite(lse_t), lse_t, z)
            res["dalpha"][h] = -(np.exp(z - lse_safe) * delta).sum()
    if grads and softmax_type == VANILLA:
        res["dalpha"] = None
    return res


# ---- attention dropout ------------------------------------------------------
#
# The TE single-GPU page ("Other attention knobs") enables attention dropout
# with a rate and an RNG, and the PR #2225 sequence diagrams show the fused
# forward returning an rng_state next to the output and softmax_aux.  The
# pages fix neither the generator nor where the rate applies; readings taken:
#   * inverted dropout on the softmax probabilities: O = (P * Z) V with
#     Z_ij = keep_ij / (1 - p_eff); the LSE and the softmax normalisation use
#     the undropped P;
#   * keep_ij comes from the counter-based generator Philox4x32-10 (Salmon,
#     Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
#     SC 2011), with the 64-bit seed as key and the 32-bit offset (the rng
#     state advanced between calls) in the counter.  One generator call
#     covers a 4 x 4 block of (query row, key) pairs of one (batch, query
#     head): counter = (j >> 2, i >> 2, b * Hq + h, offset); the 16 output
#     bytes (word w, byte k = bits 8k .. 8k+7) are the pairs' random bytes,
#     byte (i & 3) * 4 + (j & 3);
#   * a pair is kept iff its byte >= t with t = round(256 p), so the drop
#     rate is p_eff = t / 256 (the rate is quantised to 1/256).

PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on arrays of counter words and a key.

    One round multiplies counter words 0 and 2 by the round constants, keeps
    each 64-bit product's high and low halves, and mixes the high halves with
    counter words 1 and 3 and the round key; the key grows by the Weyl
    constants between rounds.  All words are uint32 (held in uint64 arrays).
    """
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & MASK32)
    k1 = np.uint64(int(k1) & MASK32)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for r in range(10):
        if r:
            k0 = np.uint64((int(k0) + PHILOX_W0) & MASK32)
            k1 = np.uint64((int(k1) + PHILOX_W1) & MASK32)
        p0 = m0 * c0
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def dropout_threshold(p: float) -> int:
    """Byte threshold t = round(256 p), clamped to [0, 255]."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must lie in [0, 1)")
    return min(255, int(math.floor(256.0 * p + 0.5)))


def dropout_keep(b: int, h: int, rows, keys, *, num_heads: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Boolean [len(rows), len(keys)]: True where pair (row, key) of batch b,
    query head h is kept."""
    t = dropout_threshold(p)
    i = np.asarray(rows, dtype=np.uint64)[:, None]
    j = np.asarray(keys, dtype=np.uint64)[None, :]
    i, j = np.broadcast_arrays(i, j)
    out = philox4x32_10(j >> np.uint64(2), i >> np.uint64(2), np.full(i.shape, b * num_heads + h, np.uint64),
                        np.full(i.shape, offset, np.uint64), seed & MASK32, (seed >> 32) & MASK32)
    byte_idx = (i & np.uint64(3)) * np.uint64(4) + (j & np.uint64(3))
    words = np.stack(out)                                         # [4, rows, keys]
    w = np.take_along_axis(words, (byte_idx >> np.uint64(2)).astype(np.int64)[None], axis=0)[0]
    byte = (w >> ((byte_idx & np.uint64(3)) * np.uint64(8))) & np.uint64(0xFF)
    return byte >= np.uint64(t)


def _dropout_factors(dropout, b, h, num_heads, rows, keys):
    """Z = keep / (1 - p_eff) for the pairs rows x keys, or 1 without dropout."""
    if dropout is None:
        return np.ones((len(rows), len(keys)))
    p, seed, offset = dropout
    keep = dropout_keep(b, h, rows, keys, num_heads=num_heads, p=p, seed=seed, offset=offset)
    return np.where(keep, 1.0 / (1.0 - dropout_threshold(p) / 256.0), 0.0)


def attention_dropout(q, k, v, d_o=None, *, p: float, seed: int, offset: int, num_gqa_groups=None,
                      causal=True, window=(-1, -1), scale_factor=None, softmax_type=VANILLA,
                      softmax_offset=None, seqlens=None):
    """attention() with inverted dropout on the probabilities (readings above).

    Per (batch, query head): P and LSE as without dropout; Z = keep / (1 - p_eff);
    O = (P Z) V;  dV = (P Z)^T dO;  dP = Z (dO V^T);  delta = rowsum(dO O);
    dS = P (dP - delta);  dQ = scale dS K;  dK = scale dS^T Q;  dz = -p_sink delta.
    Returns the same dict as attention() plus keep [B, Hq, S, S].
    """
    B, S, Hq, Hkv, dqk, dv_dim, scale = _resolve(q, k, v, num_gqa_groups, scale_factor)
    G = Hq // Hkv
    zscale = 1.0 / (1.0 - dropout_threshold(p) / 256.0)
    grads = d_o is not None
    res = {"o": np.zeros((B, S, Hq, dv_dim)), "lse": np.zeros((B, Hq, S)),
           "keep": np.zeros((B, Hq, S, S), dtype=bool)}
    if grads:
        res.update(dq=np.zeros((B, S, Hq, dqk)), dk=np.zeros((B, S, Hkv, dqk)),
                   dv=np.zeros((B, S, Hkv, dv_dim)), dalpha=np.zeros(Hq))
    for b in range(B):
        L = S if seqlens is None else int(np.asarray(seqlens).reshape(-1)[b])
        mask = visible_mask(S, L, causal, int(window[0]), int(window[1]))
        for h in range(Hq):
            g = h // G
            keep = dropout_keep(b, h, np.arange(S), np.arange(S), num_heads=Hq, p=p, seed=seed, offset=offset)
            res["keep"][b, h] = keep
            z = sink_logit(softmax_type, softmax_offset, h)
            qh = np.asarray(q[b, :, h, :], dtype=np.float64)
            kg = np.asarray(k[b, :, g, :], dtype=np.float64)
            vg = np.asarray(v[b, :, g, :], dtype=np.float64)
            s = scale * (qh @ kg.T)
            pr, lse = _softmax_rows(s, mask, z)
            zmat = np.where(keep, zscale, 0.0)
            o = (pr * zmat) @ vg
            res["o"][b, :, h, :] = o
            res["lse"][b, h] = lse
            if not grads:
                continue
            doh = np.asarray(d_o[b, :, h, :], dtype=np.float64)
            dp = zmat * (doh @ vg.T)
            delta = (doh * o).sum(axis=1)
            ds = pr * (dp - delta[:, None])
            res["dq"][b, :, h, :] = scale * (ds @ kg)
            res["dk"][b, :, g, :] += scale * (ds.T @ qh)
            res["dv"][b, :, g, :] += (pr * zmat).T @ doh
            if z is not None:
                lse_safe = np.where(np.isfinite(lse), lse, z)
                res["dalpha"][h] += -(np.exp(z - lse_safe) * delta).sum()
    if grads and softmax_type == VANILLA:
        res["dalpha"] = None
    return res
