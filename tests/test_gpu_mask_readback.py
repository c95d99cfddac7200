"""Exact read-back of the plain kernels' per-element visibility decisions, and
full coverage of every output row by the grids' work items.

Inputs built so that each output element isolates one (query, key) pair:
Q and K are one-hot in disjoint halves of the head dims (every score is
exactly 0, so every visible key of row i gets P = 1/n_i with n_i its visible
count), V and dO are one-hot by position modulo d_v, K and Q by position
modulo d_qk/2.  With windows no wider than those moduli, column c of

    O[i]  holds P for the key j of row i's window with j = c (mod d_v),
    dV[j] holds P for the row i of key j's window with i = c (mod d_v),
    dQ[i] holds scale * dS for the key j with j = c (mod d_qk/2),
    dK[j] holds scale * dS for the row i with i = c (mod d_qk/2), in the upper half,

and dS_ij = P_ij ([i = j] - delta_i) with delta_i = O[i, i mod d_v] = 1/n_i.  A
pair the forward, dQ or dK/dV kernel wrongly keeps or drops makes a zero
nonzero (or the reverse) or changes n_i, and so the value; both are checked
exactly against the oracle's mask (windows at tile edges, diagonals, padding
that ends inside a tile, windows spanning several tiles).

Outputs are pre-filled with NaN, so a row or key tile that no workgroup
writes fails as well.
"""
import math

import numpy as np
import pytest

import oracle
from scaled_dot_product_15_amd import binding
from tests import gpu_cases as gc

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gc.gpu_available(), reason="needs a GPU and the built library")]

# (d_qk, d_v, causal, window, S, lengths)
CASES = [
    (128, 128, True, (0, 0), 333, (333, 200, 77)),
    (128, 128, True, (1, 0), 333, (333, 129, 64)),
    (128, 128, True, (17, 0), 333, (333, 256, 1)),
    (128, 128, True, (62, 0), 700, (700, 513, 300)),
    (128, 128, False, (20, 9), 333, (333, 200, 77)),
    (128, 128, False, (31, 30), 400, (400, 257, 33)),
    (128, 128, False, (0, 0), 300, (300, 65, 2)),
    (64, 64, True, (30, 0), 333, (333, 200, 77)),
    (64, 64, False, (11, 19), 333, (333, 100, 31)),
    (192, 128, True, (94, 0), 500, (500, 321, 96)),
    (192, 128, False, (40, 50), 333, (333, 190, 7)),
]


def _inputs(B, S, Hq, Hkv, dqk, dv):
    import torch
    mk = dqk // 2
    i = torch.arange(S, device="cuda")
    q = torch.zeros(B, S, Hq, dqk, device="cuda", dtype=torch.bfloat16)
    k = torch.zeros(B, S, Hkv, dqk, device="cuda", dtype=torch.bfloat16)
    v = torch.zeros(B, S, Hkv, dv, device="cuda", dtype=torch.bfloat16)
    do = torch.zeros(B, S, Hq, dv, device="cuda", dtype=torch.bfloat16)
    q[:, i, :, mk + i % mk] = 1
    k[:, i, :, i % mk] = 1
    v[:, i, :, i % dv] = 1
    do[:, i, :, i % dv] = 1
    return q, k, v, do


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"d{c[0]}_{c[1]}_{'c' if c[2] else 'nc'}_w{c[3][0]}_{c[3][1]}_S{c[4]}")
def test_visibility_readback(case):
    import torch
    dqk, dv, causal, win, S, lens = case
    mk = dqk // 2
    span = win[0] + (0 if causal else win[1]) + 1  # keys a row sees at most (rows a key is seen by)
    assert span <= min(dv, mk)  # so every column holds at most one pair
    B, Hq, Hkv = len(lens), 4, 2
    scale = 1.0 / math.sqrt(dqk)
    q, k, v, do = _inputs(B, S, Hq, Hkv, dqk, dv)
    seqlens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    nan = float("nan")
    o = torch.full((B, S, Hq, dv), nan, device="cuda", dtype=torch.bfloat16)
    lse = torch.full((B, Hq, S), nan, device="cuda")
    outs = (torch.full_like(q, nan), torch.full_like(k, nan), torch.full_like(v, nan), None)
    kw = dict(num_gqa_groups=Hkv, attn_mask_type="causal" if causal else "no_mask", window_size=win,
              seqlens=seqlens)
    gc.log(f"readback d={dqk}/{dv} causal={causal} window={win} S={S} lengths={lens}")
    binding.attn_fwd(q, k, v, out=o, lse=lse, **kw)
    dq, dk, dvv, _ = binding.attn_bwd(q, k, v, o, lse, do, outs=outs, **kw)
    torch.cuda.synchronize()
    o, dq, dk, dvv = (x.float().cpu().numpy() for x in (o, dq, dk, dvv))
    for b, L in enumerate(lens):
        vis = oracle.visible_mask(S, L, causal, win[0], win[1])      # [S, S], rows i, keys j
        n = vis.sum(axis=1).astype(np.float64)                        # visible keys per row
        inv = np.where(n > 0, 1.0 / np.maximum(n, 1), 0.0)
        ii, jj = np.nonzero(vis)
        # expected values, one (row, key) pair per output element
        e_o = np.zeros((S, dv))
        e_o[ii, jj % dv] = inv[ii]
        e_dv = np.zeros((S, dv))
        e_dv[jj, ii % dv] = inv[ii]
        ds = inv[ii] * ((ii == jj).astype(np.float64) - inv[ii])
        e_dq = np.zeros((S, dqk))
        e_dq[ii, jj % mk] = scale * ds
        e_dk = np.zeros((S, dqk))
        e_dk[jj, mk + ii % mk] = scale * ds
        # GQA sums dK / dV over the group's query heads (all alike here)
        G = Hq // Hkv
        for h in range(Hq):
            for name, got, want, rtol in (("O", o[b, :, h], e_o, 2.0 ** -8), ("dQ", dq[b, :, h], e_dq, 2.0 ** -6)):
                _check(got, want, rtol, f"{name} b={b} h={h}")
        for g in range(Hkv):
            _check(dvv[b, :, g], G * e_dv, 2.0 ** -7, f"dV b={b} g={g}")
            _check(dk[b, :, g], G * e_dk, 2.0 ** -6, f"dK b={b} g={g}")


def _check(got, want, rtol, tag):
    assert np.isfinite(got).all(), f"{tag}: unwritten (NaN) elements at {np.argwhere(~np.isfinite(got))[:4]}"
    zero = want == 0
    bad = np.argwhere(zero & (got != 0))
    assert bad.size == 0, f"{tag}: invisible pairs contribute at (row, col) {bad[:6].tolist()}"
    nz = ~zero
    err = np.abs(got[nz] - want[nz]) / np.abs(want[nz])
    if err.size:
        worst = int(np.argmax(err))
        assert err[worst] <= rtol, (f"{tag}: visible pair value off by {err[worst]:.3g} at "
                                    f"{np.argwhere(nz)[worst].tolist()} (got {got[nz][worst]}, want {want[nz][worst]})")


# Grid coverage: causal masks with and without windows whose light leading
# query tiles and trailing key tiles come in odd and even counts, ragged S and
# a padded batch: every output element is written (NaN pre-fill) and matches
# the oracle.
ITEMS = [(True, (-1, -1), 1000), (True, (-1, -1), 1024), (True, (300, 0), 1000), (True, (128, 0), 1300),
         (True, (1023, 0), 2100), (False, (-1, -1), 900)]


@pytest.mark.parametrize("causal,win,S", ITEMS, ids=lambda x: str(x))
def test_grids_cover_every_row(causal, win, S):
    import torch
    from scaled_dot_product_15_amd import inputs
    p = inputs.Problem(B=2, S=S, Hq=4, Hkv=2, d_qk=128, d_v=128, dtype="bf16", causal=causal, window=win,
                       softmax_type="learnable")
    arr = inputs.draw(p, 61_000 + ITEMS.index((causal, win, S)))
    arr["seqlens"] = np.array([S, S - 37], dtype=np.int32)
    t = inputs.to_torch(arr, "bf16", "cuda")
    nan = float("nan")
    o = torch.full((p.B, S, p.Hq, 128), nan, device="cuda", dtype=torch.bfloat16)
    lse = torch.full((p.B, p.Hq, S), nan, device="cuda")
    outs = (torch.full_like(t["q"], nan), torch.full_like(t["k"], nan), torch.full_like(t["v"], nan),
            torch.full((p.Hq,), nan, device="cuda"))
    kw = dict(num_gqa_groups=p.Hkv, attn_mask_type="causal" if causal else "no_mask", window_size=win,
              softmax_type="learnable", softmax_offset=t["alpha"], seqlens=t["seqlens"])
    gc.log(f"grid coverage causal={causal} window={win} S={S}")
    binding.attn_fwd(t["q"], t["k"], t["v"], out=o, lse=lse, **kw)
    dq, dk, dv, doff = binding.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], outs=outs, **kw)
    torch.cuda.synchronize()
    for name, x in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv), ("doff", doff)):
        assert torch.isfinite(x).all(), f"{name} has unwritten elements"
    gc.compare_full(p, t, (o, lse, dq, dk, dv, doff), gc.oracle_full(p, t), tag=f"grid {causal} {win} {S}")
