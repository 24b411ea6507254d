"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins catch each one.

Each mutant is one textual edit of oracle/ka_oracle.c -- a dropped term, a wrong
sign, a wrong index, an off-by-one window, a swapped operand.  The edited source
is compiled to a temporary library and the full pin set runs against it; at
least one pin must fail.  This is evidence that the pins constrain every part
of the oracle, not only its happy path.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS, bound_oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "ka_oracle.c")

MUTANTS = {
    "rope_sign_first_half": ("y[i] = x[i] * c - x[i + half] * s;", "y[i] = x[i] * c + x[i + half] * s;"),
    "rope_opposite_direction": ("y[i] = x[i] * c - x[i + half] * s;\n    y[i + half] = x[i + half] * c + x[i] * s;",
                                "y[i] = x[i] * c + x[i + half] * s;\n    y[i + half] = x[i + half] * c - x[i] * s;"),
    "rope_frequency_exponent": ("-2.0 * (double)i / (double)D", "-1.0 * (double)i / (double)D"),
    "rope_pairs_adjacent_dims": ("y[i + half] = x[i + half] * c + x[i] * s;",
                                 "y[i + half] = x[i + half] * c + x[(i + 1) % half] * s;"),
    "dyt_drops_beta": ("y[d] = gamma[d] * tanh(alpha * x[d]) + beta[d];", "y[d] = gamma[d] * tanh(alpha * x[d]);"),
    "dyt_drops_alpha": ("++d) y[d] = gamma[d] * tanh(alpha * x[d])", "++d) y[d] = gamma[d] * tanh(x[d])"),
    "dyt_drops_gamma": ("++d) y[d] = gamma[d] * tanh(alpha * x[d])", "++d) y[d] = tanh(alpha * x[d])"),
    "softmax_no_max_shift": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "scale_dropped": ("s[j] = scale * acc;", "s[j] = acc;"),
    "no_normalisation": ("out[d] /= z;", "out[d] /= 1.0;"),
    "pv_uses_first_value_row": ("out[d] += s[j] * vals[j][d];", "out[d] += s[j] * vals[0][d];"),
    "score_dot_misindexed": ("acc += q[d] * keys[j][d];", "acc += q[d] * keys[j][(d + 1) % D];"),
    "window_low_off_by_one": ("long lo = p - window, hi = p + window;", "long lo = p - window + 1, hi = p + window;"),
    "window_high_off_by_one": ("long lo = p - window, hi = p + window;", "long lo = p - window, hi = p + window - 1;"),
    "window_clamp_high": ("if (hi > S - 1) hi = S - 1;", "if (hi > S - 2) hi = S - 2;"),
    "lambda_sign": ("out[flat * D + d] = o1[d] - lam[h] * o2[d];", "out[flat * D + d] = o1[d] + lam[h] * o2[d];"),
    "lambda_wrong_head": ("out[flat * D + d] = o1[d] - lam[h] * o2[d];", "out[flat * D + d] = o1[d] - lam[0] * o2[d];"),
    "branch2_uses_branch1_keys": ("attend_row(qh2 + p * D, kr2, vr, nk", "attend_row(qh2 + p * D, kr1, vr, nk"),
    "branch2_uses_branch1_query": ("attend_row(qh2 + p * D, kr2", "attend_row(qh1 + p * D, kr2"),
    "one_param_set_for_all": ("dyt ? alpha[t] : 0.0, dyt ? gamma + (int64_t)t * D : NULL,\n"
                              "                 dyt ? beta + (int64_t)t * D : NULL",
                              "dyt ? alpha[0] : 0.0, dyt ? gamma : NULL,\n                 dyt ? beta : NULL"),
    "rms_drops_eps": ("1.0 / sqrt(ss / (double)D + eps);", "1.0 / sqrt(ss / (double)D);"),
    "rms_sum_not_mean": ("1.0 / sqrt(ss / (double)D + eps);", "1.0 / sqrt(ss + eps);"),
    "rms_eps_outside_root": ("1.0 / sqrt(ss / (double)D + eps);", "1.0 / (sqrt(ss / (double)D) + eps);"),
    "rms_drops_weight": ("y[d] = w[d] * (x[d] * inv);", "y[d] = x[d] * inv;"),
    "rms_one_weight_set": ("dyt ? NULL : rms_w + (int64_t)t * D", "dyt ? NULL : rms_w"),
    "rope_partial_sign": ("y[i] = x[i] * c - x[h + i] * s;", "y[i] = x[i] * c + x[h + i] * s;"),
    "rope_partial_pairs_half_head": ("y[i] = x[i] * c - x[h + i] * s;\n    y[h + i] = x[h + i] * c + x[i] * s;",
                                     "y[i] = x[i] * c - x[D / 2 + i] * s;\n    y[D / 2 + i] = x[D / 2 + i] * c + x[i] * s;"),
    "rope_partial_frequency_over_head": ("-2.0 * (double)i / (double)rot", "-2.0 * (double)i / (double)D"),
    "rope_partial_tail_dropped": ("for (int d = rot; d < D; ++d) y[d] = x[d];", "for (int d = rot; d < D; ++d) y[d] = 0.0;"),
    "rope_width_ignored": ("if (m.rot == D)", "if (1)"),
    "v_keep_ignored": ("vr[j] = (keep && !keep[j0 + j]) ? zero_row : vb", "vr[j] = vb"),
    "v_keep_inverted": ("vr[j] = (keep && !keep[j0 + j]) ? zero_row : vb", "vr[j] = (keep && keep[j0 + j]) ? zero_row : vb"),
    "v_keep_wrong_batch": ("v_keep + (bh / H) * (int64_t)S", "v_keep + (bh % H) * (int64_t)S"),
    "rope_position_ignored": ("ora_rope_row(tmp, D, p, base, y + (int64_t)p * D);",
                              "ora_rope_row(tmp, D, 0, base, y + (int64_t)p * D);"),
    "dense_wrong_head_kv": ("int64_t bh = flat / Sq;", "int64_t bh = (flat / Sq) % (B * H > 1 ? B * H - 1 : 1);"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique in ka_oracle.c"
    src = tmp_path / f"mut_{name}.c"
    src.write_text(source.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / f"libmut_{name}.so")))
    ora = bound_oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(ora)
        except Exception:  # an assertion, a NaN check or a crash-free error return all count
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
