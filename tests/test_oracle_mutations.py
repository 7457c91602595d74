"""The pins catch plausible mistakes in the oracles.

Each case plants one mistake in a copy of oracle/sv_oracle.c or
oracle/kd_oracle.c (a dropped term, a wrong sign, a non-strict comparison, a
wrong uniform slot, an index off by one row, a reversed tie order, ...),
builds the copy with gcc on the CPU, and runs the pins of
test_oracle_pins.py and test_kd_pins.py against it, cheapest first: at least
one pin must fail.  The unaltered sources must pass the same pins, so a
failure is the planted mistake's doing.
"""
import os
import shutil

import pytest

import oracle
import golden_cases
import test_kd_pins as KP
import test_oracle_pins as OP

SRC = os.path.dirname(oracle.__file__)

# (name, file, original text, planted text)
MUTATIONS = [
    ("accept_not_strict", "sv_oracle.c", "if (!(u < a)) { j = i; break; }", "if (!(u <= a)) { j = i; break; }"),
    ("chain_keeps_going", "sv_oracle.c", "if (!(u < a)) { j = i; break; }", "if (!(u < a)) { j = i; }"),
    ("residual_sign", "sv_oracle.c", "return p > q ? p - q : 0.0;", "return q > p ? q - p : 0.0;"),
    ("cdf_not_strict", "sv_oracle.c", "if (C > tau) {", "if (C >= tau) {"),
    ("residual_uniform_slot", "sv_oracle.c", "V, R, (double)ub[k], &margin)", "V, R, (double)ub[k + 1], &margin)"),
    ("bonus_uniform_slot", "sv_oracle.c", "st[k].s, (double)ub[k + 1], &margin)", "st[k].s, (double)ub[k], &margin)"),
    ("normaliser_without_T", "sv_oracle.c", "r.s += exp((elem(row, dtype, x) - r.m) / T);",
     "r.s += exp((elem(row, dtype, x) - r.m));"),
    ("prob_without_max", "sv_oracle.c", "return exp((elem(row, dtype, x) - st.m) / T) / st.s;",
     "return exp((elem(row, dtype, x)) / T) / st.s;"),
    ("top32_tie_order", "sv_oracle.c", "return (p->x > q->x) - (p->x < q->x);", "return (p->x < q->x) - (p->x > q->x);"),
    ("argmax_last_of_ties", "sv_oracle.c", "if (v > bv) { bv = v; best = x; }", "if (v >= bv) { bv = v; best = x; }"),
    ("zero_q_rejects", "sv_oracle.c", "(p > 0.0 ? INFINITY : 0.0)", "(p > 0.0 ? 0.0 : 0.0)"),
    ("no_zero_mass_fallback", "sv_oracle.c", "if (R == 0.0) {", "if (0) {"),
    ("bonus_from_row_0", "sv_oracle.c", "bonus_ctx c = { tb + (size_t)k * V * e, dtype, T, st[k].m };",
     "bonus_ctx c = { tb, dtype, T, st[k].m };"),
    ("greedy_compares_next_row", "sv_oracle.c", "if (xb[i] != argmax_row(tb + (size_t)i * V * e, dtype, V))",
     "if (xb[i] != argmax_row(tb + (size_t)(i + 1) * V * e, dtype, V))"),
    ("lse_without_log", "sv_oracle.c", "lse_target[(size_t)b * K1 + i] = st[i].m / T + log(st[i].s);",
     "lse_target[(size_t)b * K1 + i] = st[i].m / T + st[i].s;"),
    ("nan_not_detected", "sv_oracle.c", "if (isnan(v)) r.has_nan = 1;", "if (0) r.has_nan = 1;"),
    ("kd_grad_sign", "kd_oracle.c", "w * (exp(kd_elem(row, dtype, x[j]) - lse) - exp((double)v[j] - mv) / sv)",
     "w * (exp(kd_elem(row, dtype, x[j]) - lse) + exp((double)v[j] - mv) / sv)"),
    ("kd_weight_not_normalised", "kd_oracle.c", "double w = sum > 0.0 ? (double)rewards[s] / sum : 0.0;",
     "double w = sum > 0.0 ? (double)rewards[s] : 0.0;"),
    ("kd_kl_sign", "kd_oracle.c", "d += pt * (lpt - lq);", "d += pt * (lpt + lq);"),
    ("kd_no_clip", "kd_oracle.c", "if (w > w_max) w = w_max;", "if (0) w = w_max;"),
    ("kd_repeats_allowed", "kd_oracle.c", "est |= KD_DUP_INDEX;", "est |= 0;"),
]


def _pins():
    """The pins, cheapest first, as zero-argument calls on the loaded oracle."""
    P = []
    for case in golden_cases.load():
        P.append((f"hand {case['name']}", lambda c=case: OP.test_hand_exact(oracle, c)))
    P += [
        ("top32 V=40", lambda: OP.test_top32_brute_force_with_ties(oracle, 53, 40)),
        ("lse closed forms", lambda: OP.test_lse_closed_forms(oracle)),
        ("power-of-two T", lambda: OP.test_temperature_power_of_two_scaling(oracle)),
        ("greedy limit", lambda: OP.test_greedy_is_the_zero_temperature_limit(oracle, 21)),
        ("kd single sample", lambda: KP.test_single_sample_worked_example(oracle)),
        ("kd grpo group", lambda: KP.test_grpo_group_worked_example(oracle)),
        ("kd clip", lambda: KP.test_clip_and_empty_group(oracle)),
        ("kd error rows", lambda: KP.test_error_rows(oracle)),
        ("kd scipy", lambda: KP.test_kl_matches_scipy_relative_entropy(oracle, 0)),
        ("kd derivative", lambda: KP.test_gradient_is_the_derivative_of_the_loss(oracle)),
        ("top32 V=5000", lambda: OP.test_top32_brute_force_with_ties(oracle, 51, 5000)),
        ("lse fsum", lambda: OP.test_lse_against_exact_summation(oracle)),
        ("lossless V=8", lambda: OP.test_lossless_marginal_and_closed_forms(oracle, 8, 1.0, 11)),
    ]
    return P


def _first_failing_pin(lib_path):
    saved = oracle._lib
    oracle._lib = oracle.bind(lib_path)
    try:
        for name, pin in _pins():
            try:
                pin()
            except AssertionError:
                return name
        return None
    finally:
        oracle._lib = saved


def _build_copy(tmp_path, name, fname=None, old=None, new=None):
    d = tmp_path / name
    d.mkdir()
    srcs = []
    for f in ("sv_oracle.c", "kd_oracle.c"):
        text = open(os.path.join(SRC, f)).read()
        if f == fname:
            assert text.count(old) == 1, (name, "the original text must occur exactly once")
            text = text.replace(old, new)
        (d / f).write_text(text)
        srcs.append(str(d / f))
    return oracle.build(srcs=srcs, out=str(d / "liborc.so"))


def test_unaltered_oracle_passes_every_pin(tmp_path):
    assert _first_failing_pin(_build_copy(tmp_path, "unaltered")) is None


@pytest.mark.parametrize("name,fname,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, fname, old, new):
    caught = _first_failing_pin(_build_copy(tmp_path, name, fname, old, new))
    assert caught is not None, f"no pin fails with the mistake {name!r} planted"
    shutil.rmtree(tmp_path / name, ignore_errors=True)
