"""Plant plausible mistakes in a copy of the oracle's recurrence (on the CPU)
and check that the pins catch every one of them.

Each mutant differs from the NumPy oracle's gated delta rule in one place:
a dropped term, a wrong sign, a wrong index or a transposed operand.
"""
import numpy as np
import pytest

from tests import pins


def _make(mutation):
    def f(q, k, v, g, beta, S0=None):
        T, DK = q.shape
        DV = v.shape[1]
        S = np.zeros((DK, DV)) if S0 is None else np.array(S0, dtype=np.float64)
        o = np.zeros((T, DV))
        gg = np.asarray(g, np.float64)
        if mutation != "no_clamp":
            gg = np.clip(gg, -5.0, 0.0)
        a = np.exp(-gg) if mutation == "decay_sign" else np.exp(gg)
        for t in range(T):
            if mutation == "decay_on_columns" and DK == DV:
                Sbar = S * a[t][None, :]
            elif mutation == "no_decay_in_probe":
                Sbar = S
            else:
                Sbar = a[t][:, None] * S
            if mutation == "no_probe":
                e = v[t].copy()
            elif mutation == "correct_sign":
                e = v[t] + Sbar.T @ k[t]
            elif mutation == "probe_transposed" and DK == DV:
                e = v[t] - Sbar @ k[t]
            else:
                e = v[t] - Sbar.T @ k[t]
            wstr = 1.0 if mutation == "no_beta" else beta[t]
            S_new = Sbar + wstr * np.outer(k[t], e)
            if mutation == "no_decay_in_probe":
                S_new = a[t][:, None] * S + wstr * np.outer(k[t], e)
            if mutation == "read_before_write":
                o[t] = Sbar.T @ q[t]
            elif mutation == "read_transposed" and DK == DV:
                o[t] = S_new @ q[t]
            else:
                o[t] = S_new.T @ q[t]
            S = S_new
        return o, S
    return f


MUTANTS = ["no_clamp", "decay_sign", "decay_on_columns", "no_decay_in_probe", "no_probe",
           "correct_sign", "probe_transposed", "no_beta", "read_before_write",
           "read_transposed"]


def test_unmutated_copy_passes(np_oracle):
    errs = pins.run_all(_make(None), np_oracle.gated_delta_rule_bruteforce)
    assert max(errs.values()) < pins.TOL, errs


@pytest.mark.parametrize("mutation", MUTANTS)
def test_pins_catch_mutant(np_oracle, mutation):
    errs = pins.run_all(_make(mutation), np_oracle.gated_delta_rule_bruteforce)
    caught = [k for k, e in errs.items() if not e < pins.TOL]
    assert caught, f"mutation {mutation} passed every pin: {errs}"
