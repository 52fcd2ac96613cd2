"""Pins of the oracle's tolerance check, oracle.compare (CPU only).

The bound every floating-point parity test applies: a GPU result G of one
shard product passes iff every element's error is at most 1e-2 times its
magnitude scale S = |A|.|B| and the relative Frobenius error is at most
5e-3. The pins feed compare hand-built (G, O, S) triples whose verdict
follows from that definition alone: values on and just past each bound, a
result that only the Frobenius criterion rejects, zero scales, an all-zero
exact value, and non-finite results. The planted-mistake test then checks
that plausible wrong versions of the check (either criterion alone, a scale
taken from |O|, a loosened bound, NaN slipping through) each fail a pin.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

ELEM, FRO = 1e-2, 5e-3


def _base(n: int = 100):
    """O = 1 everywhere (||O|| = n), S = 4 everywhere: elementwise bound 0.04."""
    O = np.ones((n, n), dtype=np.float64)
    S = np.full((n, n), 4.0)
    return O, S


def case_exact_match(cmp):
    O, S = _base()
    r = cmp(O.copy(), O, S)
    return r["pass"] and r["max_err_ratio"] == 0.0 and r["rel_fro"] == 0.0


def case_error_on_the_elementwise_bound(cmp):
    # one element off by exactly 1e-2 * S (0.04; its exact value is 0, so the
    # error is the bound itself, with no rounding): ratio 1, Frobenius 4e-4
    O, S = _base()
    O[3, 7] = 0.0
    G = O.copy()
    G[3, 7] = ELEM * S[3, 7]
    r = cmp(G, O, S)
    return r["pass"] and r["max_err_ratio"] == 1.0


def case_error_just_past_the_elementwise_bound(cmp):
    # the same element one ulp further: rejected by the elementwise criterion
    # alone (Frobenius stays at 4e-4)
    O, S = _base()
    O[3, 7] = 0.0
    G = O.copy()
    G[3, 7] = np.nextafter(ELEM * S[3, 7], np.inf)
    r = cmp(G, O, S)
    return (not r["pass"]) and r["max_err_ratio"] > 1.0 and r["rel_fro"] < FRO


def case_frobenius_only_violation(cmp):
    # every element 0.9 of its bound (error 0.009 with S = O): elementwise
    # fine, relative Frobenius 9e-3 > 5e-3
    O = np.ones((64, 64))
    S = O.copy()
    G = O * (1.0 + 0.9 * ELEM)
    r = cmp(G, O, S)
    return (not r["pass"]) and r["max_err_ratio"] <= 1.0 and r["rel_fro"] == pytest.approx(0.009, rel=1e-9)


def case_frobenius_within_bound(cmp):
    # every element off by 4e-3 relative: both criteria hold
    O = np.ones((64, 64))
    S = O.copy()
    G = O * (1.0 + 4e-3)
    r = cmp(G, O, S)
    return r["pass"] and r["rel_fro"] == pytest.approx(4e-3, rel=1e-9)


def case_frobenius_uses_the_exact_norm(cmp):
    # ||G - O|| / ||O||, not / ||G||: O = 1, G = 1.0049 in one half and 0.9951
    # in the other gives 4.9e-3 over ||O|| (pass); a mixed-up normaliser
    # gives a different figure
    O = np.ones((10, 10))
    S = np.full_like(O, 10.0)
    G = O.copy()
    G[:5] += 4.9e-3
    G[5:] -= 4.9e-3
    r = cmp(G, O, S)
    return r["pass"] and r["rel_fro"] == pytest.approx(4.9e-3, rel=1e-9)


def case_scale_from_S_not_from_O(cmp):
    # O near zero through cancellation, S large: an error of 0.5 is within
    # 1e-2 * S = 1 although it is far beyond 1e-2 * |O|
    O = np.array([[1e-3, 100.0]])
    S = np.array([[100.0, 100.0]])
    G = O + np.array([[0.5, 0.0]])
    r = cmp(G, O, S)
    return r["pass"] and r["max_err_ratio"] == pytest.approx(0.5)


def case_zero_scale_demands_exact(cmp):
    O, S = _base(8)
    S[2, 2] = 0.0
    O[2, 2] = 0.0
    ok = cmp(O.copy(), O, S)["pass"]
    G = O.copy()
    G[2, 2] = 1e-300  # any error where S = 0
    bad = cmp(G, O, S)
    return ok and (not bad["pass"]) and bad["max_err_ratio"] == np.inf


def case_all_zero_exact_value(cmp):
    Z = np.zeros((4, 5))
    ok = cmp(Z.copy(), Z, Z)
    # O = 0 everywhere with a scale (cancellation): a nonzero result is an
    # infinite relative error, whatever its size
    S = np.ones((4, 5))
    G = Z.copy()
    G[0, 0] = 1e-6
    bad = cmp(G, Z, S)
    return ok["pass"] and ok["rel_fro"] == 0.0 and (not bad["pass"]) and bad["rel_fro"] == np.inf


def case_nan_rejected(cmp):
    O, S = _base(8)
    G = O.copy()
    G[1, 1] = np.nan
    r1 = cmp(G, O, S)
    # a NaN where the scale is zero must not hide behind the exact-match rule
    S2 = S.copy()
    S2[1, 1] = 0.0
    r2 = cmp(G, O, S2)
    return (not r1["pass"]) and (not r2["pass"])


def case_inf_rejected(cmp):
    O, S = _base(8)
    G = O.copy()
    G[0, 5] = np.inf
    G2 = O.copy()
    G2[0, 5] = -np.inf
    return (not cmp(G, O, S)["pass"]) and (not cmp(G2, O, S)["pass"])


def case_custom_tolerances(cmp):
    # the bounds are the arguments: error 0.02 with S = 1 fails at 1e-2 and
    # passes at 3e-2 (Frobenius loosened alike)
    O = np.ones((2, 2))
    S = O.copy()
    G = O + 0.02
    return (not cmp(G, O, S)["pass"]) and cmp(G, O, S, 3e-2, 3e-2)["pass"]


def case_shape_mismatch_raises(cmp):
    O, S = _base(4)
    try:
        cmp(np.ones((4, 5)), O, S)
    except ValueError:
        return True
    return False


CASES = [case_exact_match, case_error_on_the_elementwise_bound, case_error_just_past_the_elementwise_bound,
         case_frobenius_only_violation, case_frobenius_within_bound, case_frobenius_uses_the_exact_norm,
         case_scale_from_S_not_from_O, case_zero_scale_demands_exact, case_all_zero_exact_value,
         case_nan_rejected, case_inf_rejected, case_custom_tolerances, case_shape_mismatch_raises]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.__name__[5:])
def test_compare_pin(case):
    assert case(oracle.compare)


# ---------------------------------------------------------- planted mistakes

def _ratio(G, O, S, elem):
    err = np.abs(G - O)
    b = elem * S
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(b > 0, err / np.where(b > 0, b, 1.0), np.where(err > 0, np.inf, 0.0))


def _fro(G, O):
    on = np.linalg.norm(O)
    d = np.linalg.norm(G - O)
    return d / on if on > 0 else (0.0 if d == 0 else np.inf)


def _mutant(kind):
    def cmp(G, O, S, elem=ELEM, fro=FRO):
        G = np.asarray(G, dtype=np.float64)
        if G.shape != O.shape:
            raise ValueError("shape")
        if kind == "scale_from_O":
            S = np.abs(O)
        if kind == "loose_elem":
            elem = 2 * elem
        r = _ratio(G, O, S, elem)
        mr = float(np.nanmax(r)) if kind == "nan_slips" else float(r.max())
        rf = float(_fro(G, O))
        if kind == "fro_over_G":
            rf = float(np.linalg.norm(G - O) / np.linalg.norm(G))
        if kind == "nan_slips":
            rf = float(np.nan_to_num(rf))
        if kind == "or":
            ok = mr <= 1.0 or rf <= fro
        elif kind == "elem_only":
            ok = mr <= 1.0
        elif kind == "fro_only":
            ok = rf <= fro
        elif kind == "strict_lt":
            ok = mr < 1.0 and rf <= fro
        elif kind == "zero_scale_free":
            r = np.where(S > 0, r, 0.0)
            ok = float(r.max()) <= 1.0 and rf <= fro
        elif kind == "abs_fro_when_O_zero":
            rf = float(np.linalg.norm(G - O)) if np.linalg.norm(O) == 0 else rf
            ok = mr <= 1.0 and rf <= fro
        else:
            ok = mr <= 1.0 and rf <= fro
        return {"max_err_ratio": mr, "rel_fro": rf, "pass": bool(ok)}
    return cmp


MUTANTS = ["or", "elem_only", "fro_only", "scale_from_O", "loose_elem", "strict_lt", "fro_over_G", "nan_slips",
           "zero_scale_free", "abs_fro_when_O_zero"]


def _all_pins_hold(cmp) -> bool:
    for case in CASES:
        try:
            if not case(cmp):
                return False
        except Exception:
            return False
    return True


def test_pins_hold_for_the_oracle():
    assert _all_pins_hold(oracle.compare)


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_reject_planted_mistake(kind):
    assert not _all_pins_hold(_mutant(kind)), f"the mutant '{kind}' passes every pin"
