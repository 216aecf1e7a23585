"""Mutation check of the oracle's pins (CPU only).

Each case below plants one plausible mistake in a copy of the oracle's
source (a dropped term, a wrong sign, exponent, index or operand, a wrong
momentum or update rule, a wrong norm), loads the copy as a module of its
own and runs every pin of tests/test_oracle_pins.py against it.  The case
passes when at least one pin fails on the mutant: the pins would catch that
mistake in the oracle.  The oracle itself is never modified.

Rewrites that leave the result unchanged are not listed, since no pin can or
should catch them: iterating on the tall orientation (the right-hand form
X (X^T X) equals (X X^T) X), and Q^T for the symmetric Q of Gram NS.
"""

import inspect
import itertools
import os
import types

import pytest

import test_oracle_pins as P

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "msign_oracle.py")

# (name, text in the oracle, replacement)
MUTATIONS = [
    ("Keller c misprinted", "KELLER_ABC = (3.4445, -4.7750, 2.0315)", "KELLER_ABC = (3.4445, -4.7750, 2.0351)"),
    ("cubic term exponent", "return a * x + b * x ** 3 + c * x ** 5", "return a * x + b * x ** 2 + c * x ** 5"),
    ("quintic term dropped", "return a * x + b * x ** 3 + c * x ** 5", "return a * x + b * x ** 3"),
    ("Theorem 1: r updated by z, not z^2", "r = r * z * z", "r = r * z"),
    ("Theorem 1: q not multiplied", "q = q * z", "q = z"),
    ("inverse square root without the root", "return (v * (1.0 / np.sqrt(w))) @ v.T @ m",
     "return (v * (1.0 / w)) @ v.T @ m"),
    ("SVD msign keeps the singular values", "return u[:, :r] @ vt[:r, :]", "return (u[:, :r] * s[:r]) @ vt[:r, :]"),
    ("normalisation by the entry-wise 1-norm", "return x / math.sqrt(float(np.sum(x * x)) + eps)",
     "return x / (float(np.sum(np.abs(x))) + eps)"),
    ("A A term dropped", "B = b * A + c * (A @ A)", "B = b * A + c * A"),
    ("update sign", "x = a * x + B @ x", "x = a * x - B @ x"),
    ("update from the previous-step B only", "x = a * x + B @ x", "x = a * x + B"),
    ("Gram: Q update adds a Z", "Q = Q @ Z + a * Q", "Q = Q @ Z + a * Z"),
    ("Gram: RZ update adds a Z", "RZ = R @ Z + a * R", "RZ = R @ Z + a * Z"),
    ("Gram: R update adds a R", "R = Z @ RZ + a * RZ", "R = Z @ RZ + a * R"),
    ("Gram: Q not reset at a restart", "            Q = eye.copy()\n    y = Q @ x", "            Q = Q\n    y = Q @ x"),
    ("Gram: output X without Q", "    y = Q @ x\n    return y.T if tall else y", "    y = x\n    return y.T if tall else y"),
    ("spectral form normalised by sigma_1", "scale = math.sqrt(float(np.sum(s * s)) + eps)", "scale = float(s[0]) + eps"),
    ("improved init: fourth instead of eighth root", "s = (float(np.sum(lam ** 4)) + eps) ** 0.125",
     "s = (float(np.sum(lam ** 4)) + eps) ** 0.25"),
    ("improved init: squares instead of fourth powers", "s = (float(np.sum(lam ** 4)) + eps) ** 0.125",
     "s = (float(np.sum(lam ** 2)) + eps) ** 0.125"),
    ("per-step table applied in reverse", "return [tuple(float(v) for v in row) for row in arr]",
     "return [tuple(float(v) for v in row) for row in arr[::-1]]"),
    ("Muon: momentum mu (M + G)", "m_new = mu * np.asarray(m, dtype=np.float64) + np.asarray(g, dtype=np.float64)",
     "m_new = mu * (np.asarray(m, dtype=np.float64) + np.asarray(g, dtype=np.float64))"),
    ("Muon: momentum M + mu G", "m_new = mu * np.asarray(m, dtype=np.float64) + np.asarray(g, dtype=np.float64)",
     "m_new = np.asarray(m, dtype=np.float64) + mu * np.asarray(g, dtype=np.float64)"),
    ("Muon: EMA momentum", "m_new = mu * np.asarray(m, dtype=np.float64) + np.asarray(g, dtype=np.float64)",
     "m_new = mu * np.asarray(m, dtype=np.float64) + (1.0 - mu) * np.asarray(g, dtype=np.float64)"),
    ("Muon: update sign", "return w - lr * o, m_new", "return w + lr * o, m_new"),
    ("Muon: msign of the gradient", "o = (ns if msign is None else msign)(m_new)",
     "o = (ns if msign is None else msign)(np.asarray(g, dtype=np.float64))"),
    ("Muon: msign of the old momentum", "o = (ns if msign is None else msign)(m_new)",
     "o = (ns if msign is None else msign)(np.asarray(m, dtype=np.float64))"),
    ("Muon: Nesterov-style direction", "o = (ns if msign is None else msign)(m_new)",
     "o = (ns if msign is None else msign)(mu * m_new + np.asarray(g, dtype=np.float64))"),
    ("error measure without the denominator", "worst = max(worst, num / den if den > 0 else num)",
     "worst = max(worst, num)"),
    ("FLOP model: A^2 counted once", "return steps * (2.0 * m * n * n + 2.0 * n ** 3 + 2.0 * m * n * n)",
     "return steps * (2.0 * m * n * n + 1.0 * n ** 3 + 2.0 * m * n * n)"),
]


def _pin_cases():
    """(name, function, kwargs) for every parametrised case of every pin."""
    cases = []
    for name, fn in sorted(inspect.getmembers(P, inspect.isfunction)):
        if not name.startswith("test_"):
            continue
        grids = []
        for mark in getattr(fn, "pytestmark", []):
            if mark.name != "parametrize":
                continue
            names = [a.strip() for a in mark.args[0].split(",")]
            values = [v if len(names) > 1 else (v,) for v in mark.args[1]]
            grids.append([dict(zip(names, v)) for v in values])
        for combo in itertools.product(*grids) if grids else [()]:
            kw = {}
            for part in combo:
                kw.update(part)
            cases.append((name, fn, kw))
    return cases


PIN_CASES = _pin_cases()


def _mutant(src):
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_pin_cases_are_collected():
    assert len(PIN_CASES) >= 60, len(PIN_CASES)
    params = {n for n, fn, kw in PIN_CASES for _ in [fn] if set(inspect.signature(fn).parameters) - set(kw)}
    assert not params, f"pins with unfilled arguments: {params}"


def test_unmutated_copy_passes_every_pin(monkeypatch):
    with open(SRC_PATH) as f:
        src = f.read()
    monkeypatch.setattr(P, "O", _mutant(src))
    for name, fn, kw in PIN_CASES:
        fn(**kw)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(monkeypatch, name, old, new):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    monkeypatch.setattr(P, "O", _mutant(src.replace(old, new)))
    for pin, fn, kw in PIN_CASES:
        try:
            fn(**kw)
        except Exception:  # an assertion or a crash: the mistake is caught
            return
    pytest.fail(f"no pin fails when the oracle has: {name}")
