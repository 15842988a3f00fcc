"""Each planted mistake in a copy of the oracle must fail at least one pin.

The mistakes are the plausible ones: a dropped factor, a wrong sign, an
off-by-one index, a transposed or swapped operand, a wrong normaliser. The
copies are built from the oracle source on the CPU; the real oracle is not
touched.
"""
import importlib.util
import os
import sys
import types

import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "oracle.py")

MUTANTS = {
    "weight_rows_reversed": ("out += g[:, vrows].T @ as_f64(student.hidden[r])",
                             "out += g[:, vrows[::-1]].T @ as_f64(student.hidden[r])"),
    "weight_rows_teacher_hidden": ("out += g[:, vrows].T @ as_f64(student.hidden[r])",
                                   "out += g[:, vrows].T @ as_f64(student.hidden[r][::-1])"),
    "reverse_as_forward": ("return (T * T) * (np.exp(lp_s) * (lp_s - lp_t)).sum(axis=-1)",
                           "return (T * T) * (np.exp(lp_t) * (lp_t - lp_s)).sum(axis=-1)"),
    "reverse_grad_missing_kl": ("return T * p * (lp_s - lp_t - kl)", "return T * p * (lp_s - lp_t)"),
    "reverse_grad_missing_T": ("return T * p * (lp_s - lp_t - kl)", "return p * (lp_s - lp_t - kl)"),
    "jeffreys_twice_forward": ("""        return (forward_kl(student_logits, teacher_logits, T, Tt)
                + reverse_kl(student_logits, teacher_logits, T, Tt))""",
                               """        return (forward_kl(student_logits, teacher_logits, T, Tt)
                + forward_kl(student_logits, teacher_logits, T, Tt))"""),
    "kl_without_T2": ("return (T * T) * (q * np.where", "return (q * np.where"),
    "kl_scaled_by_teacher_T": ("return (T * T) * (q * np.where", "return (Tt * Tt) * (q * np.where"),
    "kl_teacher_not_tempered": ("lp_t = log_softmax(teacher_logits / Tt)\n    q = np.exp(lp_t)",
                                "lp_t = log_softmax(teacher_logits)\n    q = np.exp(lp_t)"),
    "kl_teacher_at_student_T": ("lp_t = log_softmax(teacher_logits / Tt)\n    q = np.exp(lp_t)",
                                "lp_t = log_softmax(teacher_logits / T)\n    q = np.exp(lp_t)"),
    "reverse_teacher_at_student_T": (
        "lp_t = log_softmax(teacher_logits / Tt)\n    return (T * T) * (np.exp(lp_s)",
        "lp_t = log_softmax(teacher_logits / T)\n    return (T * T) * (np.exp(lp_s)"),
    "dkl_teacher_at_student_T": ("return T * (softmax(student_logits / T) - softmax(teacher_logits / Tt))",
                                 "return T * (softmax(student_logits / T) - softmax(teacher_logits / T))"),
    "dreverse_teacher_at_student_T": ("lp_t = log_softmax(teacher_logits / Tt)\n    p = np.exp(lp_s)",
                                      "lp_t = log_softmax(teacher_logits / T)\n    p = np.exp(lp_s)"),
    "teacher_temperature_ignored": (
        "return p.temperature if p.teacher_temperature is None else p.teacher_temperature",
        "return p.temperature"),
    "zero_teacher_probability_nan": ("(q * np.where(q > 0, lp_t - lp_s, 0.0))", "(q * (lp_t - lp_s))"),
    "logits_teacher_columns_reversed": ("return as_f64(t.logits[rows])",
                                        "return as_f64(t.logits[rows][:, ::-1])"),
    "zero_weight_term_multiplied": ("        if w_term != 0.0:\n            contrib = contrib + w_term * term",
                                    "        contrib = contrib + w_term * term"),
    "compact_keeps_ignored_kl": ("np.where(vb, kl, 0.0) if p.compact_valid else kl",
                                 "kl if p.compact_valid else kl"),
    "teacher_grad_missing_weight": ("g = p.teacher_ce_weight * dce_dlogits(t, lab, valid)",
                                    "g = dce_dlogits(t, lab, valid)"),
    "teacher_grad_loss_ignored": ("# 0 on invalid rows\n    return g * (grad_loss / den)",
                                  "# 0 on invalid rows\n    return g * (1.0 / den)"),
    "teacher_dW_uses_student_hidden": ("dWt += g.T @ as_f64(teacher.hidden[r])",
                                       "dWt += g.T @ as_f64(student.hidden[r])"),
    "teacher_dH_uses_teacher_weight_when_tied": (
        "Wt = as_f64(student.weight if teacher.kind == \"tied\" else teacher.weight)",
        "Wt = as_f64(teacher.weight if teacher.weight is not None else student.weight[::-1])"),
    "kl_reversed": ("(q * np.where(q > 0, lp_t - lp_s, 0.0))", "(np.exp(lp_s) * (lp_s - lp_t))"),
    "ce_label_off_by_one": ("picked = np.take_along_axis(logits, y[:, None], axis=1)",
                            "picked = np.take_along_axis(logits, (y[:, None] + 1) % logits.shape[1], axis=1)"),
    "ce_ignored_not_zeroed": ("return np.where(valid, logsumexp(logits) - picked, 0.0)",
                              "return logsumexp(logits) - picked"),
    "lse_missing_shift": ("return m + np.log(np.exp(x - m[..., None]).sum(axis=-1))",
                          "return np.log(np.exp(x - m[..., None]).sum(axis=-1))"),
    "topk_mass_dropped": ("return entropy_term - cross_term + mass * logsumexp(student_logits)",
                          "return entropy_term - cross_term + logsumexp(student_logits)"),
    "topk_entropy_sign": ("return entropy_term - cross_term + mass",
                          "return -entropy_term - cross_term + mass"),
    "dkl_missing_T": ("return T * (softmax(student_logits / T) - softmax(teacher_logits / Tt))",
                      "return (softmax(student_logits / T) - softmax(teacher_logits / Tt))"),
    "dtopk_plus_p": ("np.subtract.at(g,", "np.add.at(g,"),
    "dce_label_not_subtracted": ("g[rows, np.asarray(labels, dtype=np.int64)[rows]] -= 1.0",
                                 "pass"),
    "den_counts_all_rows": ("return float(max(n_valid, 1))", "return float(max(n_valid + 1, 1))"),
    "grad_not_masked": ("    g[~valid] = 0.0\n    return g * (grad_loss / den)",
                        "    return g * (grad_loss / den)"),
    "dW_uses_teacher_hidden": ("dW += g.T @ as_f64(student.hidden[r])",
                               "dW += g.T @ as_f64((teacher.hidden if teacher.hidden is not None and teacher.hidden.shape == student.hidden.shape else student.hidden)[r])"),
    "dH_transposed_weight_rows": ("dH[r] = g @ W", "dH[r] = g @ W[::-1]"),
    "grad_loss_ignored": ("    g[~valid] = 0.0\n    return g * (grad_loss / den)",
                          "    g[~valid] = 0.0\n    return g * (1.0 / den)"),
    "out_of_range_label_valid": ("return (y != ignore_index) & (y >= 0) & (y < vocab)",
                                 "return (y != ignore_index)"),
}


def _load_mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: anchor not found exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = SRC
    sys.modules[mod.__name__] = mod
    exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    mod = _load_mutant(name, old, new)
    failures = []
    for check in pins.ALL:
        try:
            check(mod)
        except Exception as e:  # AssertionError, or an error the mistake provokes
            failures.append((check.__name__, type(e).__name__))
    assert failures, f"planted mistake {name} passed every pin"
