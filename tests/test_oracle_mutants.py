"""Planted mistakes in copies of the oracle must each fail at least one pin.

Every mutant is the oracle's source with one textual change, executed as a
fresh module on the CPU; the real oracle module is never modified.  This shows
the pins would notice a dropped term, a wrong sign, index or operand, or the
off-by-one constant bug discussed in PR #2225 (offset 1.0 instead of 0.0).
"""
import os
import types

import pytest

from tests import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "sdpa_oracle.py")

MUTANTS = {
    "off_by_one_logit_1": [("    if softmax_type == OFF_BY_ONE:\n        return 0.0",
                            "    if softmax_type == OFF_BY_ONE:\n        return 1.0")],
    "gqa_strided_heads": [("return h // (num_heads // num_kv_heads)", "return h % num_kv_heads"),
                          ("h = g * G + gi", "h = gi * Hkv + g", "all")],
    "dk_missing_scale": [('out["dk"] += scale * (ds.T @ qh)', 'out["dk"] += (ds.T @ qh)')],
    "dv_untransposed_p": [('out["dv"] += p.T @ doh', 'out["dv"] += p @ doh')],
    "dq_wrong_operand": [('out["dq"][:, gi, :] = scale * (ds @ kb)', 'out["dq"][:, gi, :] = scale * (ds.T @ kb)')],
    "ds_dropped_delta": [("ds = p * (dp - delta[:, None])", "ds = p * dp")],
    "window_left_exclusive": [("m &= j >= i - window_left", "m &= j > i - window_left")],
    "window_right_off_by_one": [("m &= j <= i + window_right", "m &= j <= i + window_right + 1")],
    "causal_reversed": [("m &= j <= i\n", "m &= j >= i\n")],
    "padding_rows_only": [("    m = (i < L) & (j < L)\n    if causal:\n        m &= j <= i",
                           "    m = (i < L)\n    if causal:\n        m &= j <= i")],
    "sink_not_in_denominator": [("l = l + np.exp(z - m_safe)", "l = l")],
    "lse_missing_max": [("lse = np.where(l > 0, m_safe + np.log(l), -np.inf)",
                         "lse = np.where(l > 0, np.log(l), -np.inf)")],
    "dz_sign_flip": [('out["dz"][gi] = -(np.exp(z - lse_safe) * delta).sum()',
                      'out["dz"][gi] = (np.exp(z - lse_safe) * delta).sum()')],
    "default_scale_uses_dv": [("scale = (1.0 / math.sqrt(dqk))", "scale = (1.0 / math.sqrt(v.shape[-1]))", "all")],
    "sink_logit_scaled": [("z = sink_logit(softmax_type, softmax_offset, h)\n        s = scale * (qh @ kb.T)",
                           "z = sink_logit(softmax_type, softmax_offset, h)\n"
                           "        z = None if z is None else z * scale\n        s = scale * (qh @ kb.T)")],
    "rows_dq_missing_scale": [("dq = scale * (ds @ kb)\n", "dq = ds @ kb\n")],
    "rows_window_off_by_one": [("m = m & (j >= i - window_left)", "m = m & (j > i - window_left)")],
    "keys_dk_missing_scale": [("dk += scale * (ds.T @ qh)", "dk += ds.T @ qh")],
    "packed_segments_leak": [("same = (seg[:, None] == seg[None, :]) & (seg[:, None] >= 0)",
                              "same = (seg[:, None] >= 0) & (seg[None, :] >= 0)")],
    "packed_padding_ignored": [("valid[off[b]:off[b] + L] = True", "valid[off[b]:off[b + 1]] = True")],
    "packed_lse_shifted_rows": [('res["lse"][b, h, :n] = lse_t[off[b]:off[b] + n]',
                                 'res["lse"][b, h, :n] = lse_t[b:b + n]')],
    "philox_round_constant": [("PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57",
                               "PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D59")],
    "dropout_rows_keys_swapped": [("out = philox4x32_10(j >> np.uint64(2), i >> np.uint64(2),",
                                   "out = philox4x32_10(i >> np.uint64(2), j >> np.uint64(2),")],
    "dropout_byte_order": [("byte_idx = (i & np.uint64(3)) * np.uint64(4) + (j & np.uint64(3))",
                            "byte_idx = (j & np.uint64(3)) * np.uint64(4) + (i & np.uint64(3))")],
    "dropout_no_rescale": [("zmat = np.where(keep, zscale, 0.0)", "zmat = np.where(keep, 1.0, 0.0)")],
    "dropout_dp_unmasked": [("dp = zmat * (doh @ vg.T)", "dp = doh @ vg.T")],
    "dropout_dv_unmasked": [('res["dv"][b, :, g, :] += (pr * zmat).T @ doh', 'res["dv"][b, :, g, :] += pr.T @ doh')],
    "rows_dropout_dp_unmasked": [("ds = p * (zmat * (doh @ vb.T) - delta[:, None])",
                                  "ds = p * (doh @ vb.T - delta[:, None])")],
    "keys_dropout_dv_unmasked": [("dvv += (p * zmat).T @ doh", "dvv += p.T @ doh")],
    "rows_bias_transposed": [("bias[_bias_index(bias, b, h)][rows][:, c0:c1]", "bias[_bias_index(bias, b, h)].T[rows][:, c0:c1]")],
    "keys_bias_wrong_head": [("s = s + np.asarray(bias[_bias_index(bias, b, h)][rows][:, keys], dtype=np.float64)",
                              "s = s + np.asarray(bias[_bias_index(bias, b, g)][rows][:, keys], dtype=np.float64)")],
    "bias_pre_scale": [("            s = s + np.asarray(bias[_bias_index(bias, b, h)], dtype=np.float64)",
                        "            s = s + scale * np.asarray(bias[_bias_index(bias, b, h)], dtype=np.float64)")],
    "bias_transposed": [("            s = s + np.asarray(bias[_bias_index(bias, b, h)], dtype=np.float64)",
                         "            s = s + np.asarray(bias[_bias_index(bias, b, h)], dtype=np.float64).T")],
    "dbias_not_summed": [('res["dbias"][_bias_index(bias, b, g * G + gi)] += r["ds"][gi]',
                          'res["dbias"][_bias_index(bias, b, g * G + gi)] = r["ds"][gi]')],
    "keys_rows_subset": [("rows_all = np.nonzero(sees.any(axis=1))[0]",
                          "rows_all = np.nonzero(sees.any(axis=1))[0][1:]")],
}

# cheap pins first: a mutant stops at its first failing pin
ORDER = [oracle_pins.pin_golden, oracle_pins.pin_brute_force, oracle_pins.pin_causal_rows,
         oracle_pins.pin_window_limits, oracle_pins.pin_row_sums, oracle_pins.pin_sink_closed,
         oracle_pins.pin_gqa_repeat, oracle_pins.pin_padding, oracle_pins.pin_scale,
         oracle_pins.pin_dalpha_forms, oracle_pins.pin_sink_augmented,
         oracle_pins.pin_torch_sdpa, oracle_pins.pin_finite_diff, oracle_pins.pin_sampled_rows,
         oracle_pins.pin_sampled_keys, oracle_pins.pin_packed_brute_force,
         oracle_pins.pin_packed_equals_padded, oracle_pins.pin_packed_finite_diff,
         oracle_pins.pin_philox_kat, oracle_pins.pin_dropout_rate, oracle_pins.pin_dropout_p0,
         oracle_pins.pin_dropout_brute, oracle_pins.pin_dropout_finite_diff, oracle_pins.pin_dropout_mean,
         oracle_pins.pin_dropout_layout, oracle_pins.pin_dropout_sampled,
         oracle_pins.pin_bias_invariants, oracle_pins.pin_bias_torch, oracle_pins.pin_bias_finite_diff,
         oracle_pins.pin_bias_sampled]


def _mutant(edits):
    with open(SRC) as f:
        src = f.read()
    for edit in edits:
        old, new = edit[0], edit[1]
        every = len(edit) > 2 and edit[2] == "all"
        n = src.count(old)
        assert n >= 1 and (every or n == 1), f"mutation anchor not unique/present: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant.py", "exec"), mod.__dict__)
    return mod


def test_pin_order_covers_all():
    assert set(ORDER) == set(oracle_pins.ALL_PINS)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(MUTANTS[name])
    for pin in ORDER:
        try:
            pin(mod)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            return
    pytest.fail(f"no pin caught mutant {name}")
