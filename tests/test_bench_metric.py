"""Pins of the benchmark's metric: visible-pair counts and effective FLOPs.

The metric (fwd+bwd effective TFLOP/s) counts only visible (query, key) pairs,
with forward 2 * pairs * (d_qk + d_v) and backward 2 * pairs * (3 d_qk + 2 d_v)
FLOPs.  bench.py computes both itself (closed form per row); these CPU tests
check the counts against brute force over the oracle's boolean mask and
against the per-workload values worked out by hand for the five workloads, and
show that plausible slips in either function fail a pin.
"""
import os
import types

import numpy as np
import pytest

import bench
import oracle

BENCH_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py")


def _per_head_cases():
    """(S, L, causal, wl, wr) -> visible pairs of one (batch, head), each
    derived by hand: causal rows i < left see i + 1 keys, later rows left + 1."""
    return [
        ((128, 128, True, -1, -1), 128 * 129 // 2),                         # tiny fp32 workload
        ((4096, 4096, True, 1024, 0), 1024 * 1025 // 2 + 3072 * 1025),    # GQA+SWA S=4096
        ((512, 512, True, -1, -1), 512 * 513 // 2),                         # sweep, S=512
        ((16384, 16384, True, -1, -1), 16384 * 16385 // 2),                 # sweep, S=16384
        ((4096, 4096, True, -1, -1), 4096 * 4097 // 2),                     # MLA dims
        ((8192, 6000, True, 4096, 0), 8390656 + 4097 * (6000 - 4096)),     # sink + padding
        ((8192, 4096, True, 4096, 0), 8390656),
        ((64, 64, False, -1, -1), 64 * 64),                                 # no mask
        ((64, 40, False, 3, 5), sum(min(39, i + 5) - max(0, i - 3) + 1 for i in range(40))),
        ((10, 0, True, -1, -1), 0),                                         # empty batch
    ]


def _check_pairs(vp):
    for args, want in _per_head_cases():
        assert vp(*args) == want, (args, vp(*args), want)


def _check_workload_totals(vp, ef):
    # GQA+SWA S=4096: B=4, Hq=32, d=128.
    pairs = vp(4096, 4096, True, 1024, 0) * 4 * 32
    assert pairs == 470_220_800
    assert ef(pairs, 128, 128) == (240_753_049_600, 601_882_624_000)
    # tiny fp32 workload: B=1, Hq=4, d=64.
    assert vp(128, 128, True, -1, -1) * 4 == 33_024
    # MHA/GQA/MQA sweep: Hq=16, B*S = 16384, doubling per step of S.
    sweep = [vp(S, S, True, -1, -1) * (16384 // S) * 16 for S in (512, 1024, 2048, 4096, 8192, 16384)]
    assert sweep == [67_239_936, 134_348_800, 268_566_528, 537_001_984, 1_073_872_896, 2_147_614_720]
    # MLA dims: B=2, Hq=128, d_qk=192, d_v=128.
    pairs = vp(4096, 4096, True, -1, -1) * 2 * 128
    assert pairs == 2_148_007_936
    f, b = ef(pairs, 192, 128)
    assert f == 2 * pairs * 320 and b == 2 * pairs * 832


def _check_flops_by_products(ef):
    # Each contraction of a visible pair costs 2 * (its reduced dimension):
    # forward S = QK^T (d_qk), O = PV (d_v); backward S again (d_qk),
    # dP = dO V^T (d_v), dV = P^T dO (d_v), dK = dS^T Q (d_qk), dQ = dS K (d_qk).
    for d_qk, d_v in ((64, 64), (128, 128), (192, 128), (7, 11)):
        fwd = 2 * d_qk + 2 * d_v
        bwd = 2 * d_qk + 2 * d_v + 2 * d_v + 2 * d_qk + 2 * d_qk
        assert ef(1, d_qk, d_v) == (fwd, bwd)
        assert ef(1000, d_qk, d_v) == (1000 * fwd, 1000 * bwd)


def test_pairs_hand_derived():
    _check_pairs(bench.visible_pairs)


def test_pairs_match_mask_brute_force():
    rng = np.random.default_rng(7)
    for _ in range(300):
        S = int(rng.integers(1, 70))
        L = int(rng.integers(0, S + 1))
        causal = bool(rng.integers(0, 2))
        wl = int(rng.integers(-1, S + 3))
        wr = int(rng.integers(-1, S + 3))
        want = int(oracle.visible_mask(S, L, causal, wl, wr).sum())
        assert bench.visible_pairs(S, L, causal, wl, wr) == want, (S, L, causal, wl, wr)


def test_workload_totals():
    _check_workload_totals(bench.visible_pairs, bench.effective_flops)


def test_flops_by_products():
    _check_flops_by_products(bench.effective_flops)


def test_workload_pairs_sums_batches():
    p = types.SimpleNamespace(S=300, B=3, Hq=6, causal=True, window=(50, 0))
    seq = np.array([300, 120, 0], dtype=np.int32)
    want = sum(int(oracle.visible_mask(300, int(L), True, 50, 0).sum()) for L in seq) * 6
    assert bench.workload_pairs(p, seq) == want
    assert bench.workload_pairs(p, None) == int(oracle.visible_mask(300, 300, True, 50, 0).sum()) * 18


MUTANTS = {
    "bwd_two_dqk": ("2 * pairs * (3 * d_qk + 2 * d_v)", "2 * pairs * (2 * d_qk + 2 * d_v)"),
    "bwd_dv_once": ("2 * pairs * (3 * d_qk + 2 * d_v)", "2 * pairs * (3 * d_qk + d_v)"),
    "fwd_qk_only": ("return 2 * pairs * (d_qk + d_v)", "return 2 * pairs * (2 * d_qk)"),
    "fwd_no_factor_two": ("return 2 * pairs * (d_qk + d_v)", "return pairs * (d_qk + d_v)"),
    "window_exclusive": ("lo = np.maximum(0, i - window_left)", "lo = np.maximum(0, i - window_left + 1)"),
    "right_window_ignored": ("        hi = np.minimum(hi, i + window_right)\n", "        pass\n"),
    "causal_ignored": ("        hi = np.minimum(hi, i)\n", "        pass\n"),
    "padding_ignored": ("hi = np.full(L, L - 1, dtype=np.int64)", "hi = np.full(L, S - 1, dtype=np.int64)"),
    "count_off_by_one": ("np.maximum(0, hi - lo + 1)", "np.maximum(0, hi - lo)"),
}


def _mutant(name):
    src = open(BENCH_SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"bench_mutant_{name}")
    mod.__file__ = BENCH_SRC
    exec(compile(src.replace(old, new), BENCH_SRC, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_metric_mistakes_fail_a_pin(name):
    m = _mutant(name)
    caught = False
    for check in (lambda: _check_pairs(m.visible_pairs),
                  lambda: _check_workload_totals(m.visible_pairs, m.effective_flops),
                  lambda: _check_flops_by_products(m.effective_flops)):
        try:
            check()
        except AssertionError:
            caught = True
    assert caught, f"mutant {name} passed every metric pin"
