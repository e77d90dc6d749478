"""The fp64 oracle against its pins, and the pins against planted mistakes.

A planted mistake lives only in a temporary copy of the oracle's C source;
each one must make at least one pin fail.
"""
import pytest

import oracle
import pins

MUTATIONS = {
    # name: (text in oracle.c, replacement)
    "sin_sign_first": ("y[a] = xa * c - xb * s;", "y[a] = xa * c + xb * s;"),
    "sin_sign_second": ("y[b] = xa * s + xb * c;", "y[b] = -xa * s + xb * c;"),
    "second_uses_cos_twice": ("y[b] = xa * s + xb * c;", "y[b] = xa * c + xb * c;"),
    "frequency_denominator": ("-2.0 * (double)i / (double)rot_dim", "-2.0 * (double)i / (double)(rot_dim + 2)"),
    "frequency_no_factor_two": ("-2.0 * (double)i / (double)rot_dim", "-1.0 * (double)i / (double)rot_dim"),
    "layouts_swapped": ("if (layout == OR_GPTJ) {", "if (layout != OR_GPTJ) {"),
    "neox_partner_off_by_one": ("*b = i + rot_dim / 2;", "*b = (i + rot_dim / 2 + 1) % rot_dim;"),
    "tail_dropped": ("        y[d] = x[d];", "        y[d] = 0.0;"),
    "row_index_as_position": ("positions[r], base, layout);", "(double)r, base, layout);"),
    "query_offset_ignored": ("(double)(q_off + r % Sq)", "(double)(r % Sq)"),
    "key_offset_ignored": ("(double)(k_off + r % Sk)", "(double)(r % Sk)"),
    "mask_off_by_one": ("int64_t last = q_off + i - k_off;", "int64_t last = q_off + i - k_off - 1;"),
    "mask_sees_future": ("int64_t last = q_off + i - k_off;", "int64_t last = q_off + i - k_off + 1;"),
    "scale_uses_d": ("scale = 1.0 / sqrt((double)D);", "scale = 1.0 / (double)D;"),
    "dot_index": ("s += qr[d] * kr[j * D + d];", "s += qr[d] * kr[j + d];"),
    "pv_index": ("out[e] += scores[j] * v[j * Dv + e];", "out[e] += scores[j] * v[j * Dv];"),
    "not_normalised": ("for (int e = 0; e < Dv; ++e) out[e] /= l;", ""),
    "query_rotated_at_key_offset": ("(double)(q_off + r % Sq)", "(double)(k_off + r % Sq)"),
    "kv_heads_interleaved": ("int64_t kvh = bh / group;", "int64_t kvh = (bh / H) * Hkv + (bh % H) % Hkv;"),
    "kv_heads_interleaved_rows": ("kvh = b * Hkv + h / (H / Hkv);", "kvh = b * Hkv + h % Hkv;"),
    "pos_div_multiplies": ("((double)p / pos_div)", "((double)p * pos_div)"),
    "pos_div_ignored_for_queries": ("(double)(q_off + r % Sq) / pos_div", "(double)(q_off + r % Sq)"),
    "pos_div_ignored_for_row_keys": ("(double)(k_off + j) / pos_div", "(double)(k_off + j)"),
    "bwd_q_unrotated_forward": ("-(double)(q_off + i) / pos_div", "(double)(q_off + i) / pos_div"),
    "bwd_k_unrotated_forward": ("-(double)(k_off + j) / pos_div", "(double)(k_off + j) / pos_div"),
    "bwd_no_row_correction": ("p[j] * (dp[j] - pdp)", "p[j] * dp[j]"),
    "bwd_no_row_correction_keys": ("pij * (dpij - row_c[r])", "pij * dpij"),
    "bwd_dk_unscaled": ("dkr[d] += scale * ds * qri[d];", "dkr[d] += ds * qri[d];"),
    "bwd_dq_uses_query": ("dqr[d] += scale * ds * krh[j * D + d];", "dqr[d] += scale * ds * qri[d];"),
    "bwd_unnormalised_p": ("                    p[j] /= l;\n", ""),
    "bwd_keys_unnormalised_p": ("exp(s * scale - row_m[r]) / row_l[r]", "exp(s * scale - row_m[r])"),
    "bwd_keys_unscaled_scores": ("exp(s * scale - row_m[r])", "exp(s - row_m[r])"),
    "bwd_dv_from_dp": ("dvj[e] += pij * doi[e];", "dvj[e] += dpij * doi[e];"),
    "bwd_heads_interleaved": ("(kvh % Hkv) * group + g;", "(kvh % Hkv) + g * Hkv;"),
    "bwd_rows_heads_interleaved": ("const int64_t kvh = bh / group;   /* (b * H + h)",
                                   "const int64_t kvh = (bh / H) * Hkv + (bh % H) % Hkv;   /* (b * H + h)"),
    "bwd_keys_mask_off_by_one": ("if (j >= visible_keys(i, Sk, q_off, k_off, causal)) continue;",
                                 "if (j > visible_keys(i, Sk, q_off, k_off, causal)) continue;"),
    "lse_without_log": ("lse[r] = m + log(l);", "lse[r] = m + l;"),
    "kv_head_count_unchecked": ("if (Hkv <= 0 || H % Hkv != 0) return 0;", "if (Hkv <= 0) return 0;"),
}


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    src = oracle.SOURCE.read_text()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found in oracle.c"
    mutant = oracle.load_variant(src.replace(old, new), name)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, oracle.OracleError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
