"""The parity checker (``oracle.tolerance_violations``) against hand-worked cases, and
planted slips: copies of the checker's source, each with one plausible mistake, must each
fail at least one case.  Every GPU parity test goes through this function, so it is pinned
here on its own, independently of any kernel."""
import inspect
import textwrap

import numpy as np
import pytest

import oracle

INF, NAN = np.inf, np.nan


def _count(chk, y, r, atol=1e-3, rtol=1.6e-2, extra=None):
    return chk(np.asarray(y, dtype=np.float64), np.asarray(r, dtype=np.float64), atol, rtol, extra)[0]


# (name, y, ref, atol, rtol, extra, expected violation count).  With atol = 0.25 and
# rtol = 0.5 every bound below is exact in binary, so the edge cases sit exactly on it.
CASES = [
    ("finite against +inf", [5.0], [INF], 1e-3, 1.6e-2, None, 1),
    ("finite against -inf", [-1e300], [-INF], 1e-3, 1.6e-2, None, 1),
    ("-inf against +inf", [-INF], [INF], 1e-3, 1.6e-2, None, 1),
    ("+inf against -inf", [INF], [-INF], 1e-3, 1.6e-2, None, 1),
    ("+inf against finite", [INF], [3.0], 1e-3, 1.6e-2, None, 1),
    ("nan against finite", [NAN], [1.0], 1e-3, 1.6e-2, None, 1),
    ("finite against nan", [1.0], [NAN], 1e-3, 1.6e-2, None, 1),
    ("nan against inf", [NAN], [INF], 1e-3, 1.6e-2, None, 1),
    ("both nan", [NAN], [NAN], 1e-3, 1.6e-2, None, 0),
    ("equal +inf", [INF], [INF], 1e-3, 1.6e-2, None, 0),
    ("equal -inf", [-INF], [-INF], 1e-3, 1.6e-2, None, 0),
    ("mixed specials and finite", [1.0, NAN, INF, -INF, 2.0], [1.0, NAN, INF, -INF, 2.0], 1e-3, 1.6e-2, None, 0),
    ("on the bound above", [3.25], [2.0], 0.25, 0.5, None, 0),
    ("on the bound below", [0.75], [2.0], 0.25, 0.5, None, 0),
    ("just past the bound above", [3.25 + 2.0 ** -40], [2.0], 0.25, 0.5, None, 1),
    ("just past the bound below", [0.75 - 2.0 ** -40], [2.0], 0.25, 0.5, None, 1),
    ("bound scales with the reference, not the result", [10.0], [0.0], 0.25, 0.5, None, 1),
    ("absolute term alone near zero", [0.2], [0.0], 0.25, 0.5, None, 0),
    ("absolute term is needed near zero", [0.2], [0.0], 0.25, 0.0, None, 0),
    ("extra widens the bound", [1.0], [0.0], 0.25, 0.0, [1.0], 0),
    ("extra too small", [1.0], [0.0], 0.25, 0.0, [0.5], 1),
    ("extra is elementwise", [1.0, 1.0], [0.0, 0.0], 0.25, 0.0, [1.0, 0.5], 1),
    ("infinite extra admits only equality", [1.0, 2.0], [1.0, 1.0], 0.25, 0.0, [INF, INF], 1),
    ("violations are counted", [0.0, 2.0, -3.0, 0.1], [0.0, 0.0, 0.0, 0.0], 1.0, 0.0, None, 2),
]


def _check_cases(chk):
    """Names of the cases a checker gets wrong."""
    wrong = []
    for name, y, r, atol, rtol, extra, want in CASES:
        try:
            got = _count(chk, y, r, atol, rtol, extra)
        except Exception:   # a slip that breaks the function counts as caught
            got = None
        if got != want:
            wrong.append(name)
    return wrong


def test_checker_cases():
    assert _check_cases(oracle.tolerance_violations) == []


def test_checker_excess():
    n, ex = oracle.tolerance_violations(np.array([0.0, 2.0, 0.5]), np.zeros(3), 1.0, 0.0)
    assert (n, ex) == (1, 1.0)
    n, ex = oracle.tolerance_violations(np.array([5.0]), np.array([INF]))
    assert n == 1 and ex == INF
    assert oracle.tolerance_violations(np.zeros(0), np.zeros(0)) == (0, 0.0)


def test_checker_shape_mismatch():
    with pytest.raises(ValueError):
        oracle.tolerance_violations(np.zeros(3), np.zeros(4))


def test_checker_default_bar():
    """The defaults are the LCE parity bar 1e-3 + 1.6e-2*|ref|."""
    r = np.array([0.0, 1.0, -100.0])
    y = r + np.array([1e-3, 1e-3 + 1.6e-2, -(1e-3 + 1.6)])
    assert oracle.tolerance_violations(y * (1 - 1e-12) + r * 1e-12, r)[0] == 0
    assert oracle.tolerance_violations(r + np.array([1.1e-3, 0.0, 0.0]), r)[0] == 1


# Planted slips: (description, text in the checker's source, replacement).
SLIPS = [
    ("infinite reference bound admits anything", "fin_ok = fin & np.isfinite(bound) & (err <= bound)",
     "fin_ok = ~np.isnan(Y_gpu) & ~np.isnan(Y_ref) & (err <= bound)"),
    ("sign of an infinity ignored", "| (Y_gpu == Y_ref))", "| (np.abs(Y_gpu) == np.abs(Y_ref)))"),
    ("one NaN side accepted", "(np.isnan(Y_gpu) & np.isnan(Y_ref))", "(np.isnan(Y_gpu) | np.isnan(Y_ref))"),
    ("bound relative to the result", "rtol * np.abs(Y_ref)", "rtol * np.abs(Y_gpu)"),
    ("strict inequality", "(err <= bound)", "(err < bound)"),
    ("extra ignored", "bound = bound + np.asarray(extra, dtype=np.float64)", "bound = bound"),
    ("absolute term dropped", "bound = atol + rtol * np.abs(Y_ref)", "bound = rtol * np.abs(Y_ref)"),
    ("signed error", "err = np.abs(Y_gpu - Y_ref)", "err = Y_gpu - Y_ref"),
    ("infinite bound admits anything", "fin & ~np.isfinite(bound) & (Y_gpu == Y_ref)", "fin & ~np.isfinite(bound)"),
    ("presence instead of count", "int(bad.sum())", "int(bad.any())"),
]


def _mutant(old: str, new: str):
    src = textwrap.dedent(inspect.getsource(oracle.tolerance_violations))
    assert src.count(old) == 1, f"slip anchor not found once: {old!r}"
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    return ns["tolerance_violations"]


@pytest.mark.parametrize("desc,old,new", SLIPS, ids=[s[0] for s in SLIPS])
def test_checker_slip_is_caught(desc, old, new):
    assert _check_cases(_mutant(old, new)), f"planted slip not caught: {desc}"
