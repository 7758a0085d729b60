"""The pins must reject plausible mistakes in the oracle.

Each case below alters one spot of a copy of the oracle source (on the CPU, in
a temporary directory), compiles it with gcc and runs the pin battery against
it; at least one pin has to fail.  This checks that the pins constrain every
step: acceptance test, residual, bonus row, transforms, draw and output.
"""
import pytest

import test_oracle_pins as pins
import test_oracle_stats as stats_pins

MUTANTS = {
    "accept_transposed": ("if (!(u * qy < py))", "if (!(u * py < qy))"),
    "accept_not_strict": ("if (!(u * qy < py))", "if (!(u * qy <= py))"),
    "residual_sign": ("double d = P[A][x] - qx;", "double d = qx - P[A][x];"),
    "residual_wrong_row": ("double d = P[A][x] - qx;", "double d = P[g][x] - qx;"),
    "bonus_wrong_row": ("            w[x] = P[g][x];", "            w[x] = P[0][x];"),
    "zero_residual_fallback_row": ("                w[x] = P[A][x];", "                w[x] = P[g][x];"),
    "null_q_keeps_draft_cell": ("(x == r->ids[A] ? 1.0 : 0.0)", "0.0"),
    "draft_not_renormalised": ("q_out[x] = keep[x] ? r[x] / z : 0.0;", "q_out[x] = keep[x] ? r[x] : 0.0;"),
    "temperature_multiplies": ("s[x] = l / T;", "s[x] = l * T;"),
    "draft_temperature_inverted": ("pow((double)f, 1.0 / T)", "pow((double)f, T)"),
    "top_k_drops_ties": ("keep[x] = order[x] >= kth;", "keep[x] = order[x] > kth;"),
    "top_k_off_by_one": ("double kth = sorted[top_k - 1];", "double kth = sorted[top_k];"),
    "top_p_unnormalised": ("double target = top_p * zk;", "double target = top_p;"),
    "cdf_ignores_mass": ("double tau = u * S,", "double tau = u,"),
    "greedy_highest_id_on_ties": ("if (l > best) {", "if (l >= best) {"),
    "num_accepted_is_advance": ("*r->num_accepted = A;\n}", "*r->num_accepted = A + 1;\n}"),
}


def battery(o):
    """Run the pins against oracle-like object o; return the names that fail."""
    fails = []
    checks = [
        ("worked_example", lambda: pins.test_worked_example_two_token(o)),
        ("exercise", lambda: pins.test_exercise_three_token(o)),
        ("strict", lambda: pins.test_accept_is_strict(o)),
        ("greedy", lambda: pins.test_greedy_example(o)),
        ("greedy_ties", lambda: pins.test_greedy_ties_lowest_id(o)),
        ("reject_third", lambda: pins.test_exercise_reject_third(o)),
        ("top_k_ties", lambda: pins.test_top_k_keeps_ties(o)),
        ("top_p", lambda: pins.test_top_p_cut_is_smallest_tie_group_prefix(o)),
        ("transform_np", lambda: [pins.test_target_transform_matches_numpy(o, s) for s in (0, 1)]),
        ("draft_np", lambda: [pins.test_draft_transform_matches_numpy(o, s) for s in (0, 1)]),
        ("cdf", lambda: pins.test_inverse_cdf_matches_searchsorted(o)),
        ("law", lambda: [pins.test_enumerated_law_equals_closed_form(o, *c) for c in pins.LAW_CASES]),
        ("top_k_one", lambda: pins.test_top_k_one_is_greedy(o)),
        ("one_hot", lambda: pins.test_one_hot_q_equals_null_q(o)),
        ("exercise_stats", lambda: stats_pins.test_first_token_marginal_and_expected_advance(
            o, *stats_pins.CASES[1])),
    ]
    for name, f in checks:
        try:
            f()
        except (AssertionError, ValueError, IndexError, ZeroDivisionError, FloatingPointError):
            fails.append(name)
    return fails


def test_unaltered_source_passes_battery(oracle_mod, tmp_path):
    import oracle
    v = oracle.build_variant(oracle.source_text(), str(tmp_path))
    assert battery(v) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(oracle_mod, tmp_path, name):
    import oracle
    old, new = MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, "mutation site must be unique: " + name
    v = oracle.build_variant(src.replace(old, new), str(tmp_path))
    failed = battery(v)
    assert failed, name + " survived every pin"
