"""Mutation check of the oracle's pins (CPU).

Each plausible mistake below is planted in a copy of the oracle's source
(never in the oracle itself), and the pins of tests/test_oracle_pins.py,
run against that copy, must reject it: at least one pin fails or raises.
The unmutated copy must pass every pin, which checks the harness."""
import importlib.util
import itertools
import os
import sys

import pytest

import tests.test_oracle_pins as PINS

# the mutants overflow or divide by zero on the way to failing a pin
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

ORACLE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "muon_oracle.py")

# (what the mistake is, source text, replacement)
MUTATIONS = [
    ("sign of b in eq. (2)", "X = hp.a * X + hp.b * (A @ X)", "X = hp.a * X - hp.b * (A @ X)"),
    ("dropped c term", " + hp.c * ((A @ A) @ X)", ""),
    ("transposed Gram operand", "        A = X @ X.T\n", "        A = X.T @ X\n"),
    ("one iteration short", "    for _ in range(hp.ns_steps):", "    for _ in range(hp.ns_steps - 1):"),
    ("no Frobenius normalisation", "    X = X / nrm\n", ""),
    ("Nesterov weight mu dropped", "    return mu * M_new + _f64(G)", "    return M_new + _f64(G)"),
    ("Nesterov on the old momentum", "    U = nesterov_input(M_new, G, hp.momentum, hp.nesterov)\n    X, tr = orient(U)\n    ns",
     "    U = nesterov_input(_f64(M), G, hp.momentum, hp.nesterov)\n    X, tr = orient(U)\n    ns"),
    ("dampened momentum", "    return mu * _f64(M) + _f64(G)", "    return mu * _f64(M) + (1.0 - mu) * _f64(G)"),
    ("min instead of max in the scale", "coeff * math.sqrt(max(m, n))", "coeff * math.sqrt(min(m, n))"),
    ("square matrices transposed", "    if m <= n:\n        return U, False", "    if m < n:\n        return U, False"),
    ("eps added instead of max", "den = eps if nrm < eps else nrm", "den = nrm + eps"),
    ("decay without the learning rate", "(1.0 - lr * wd) * _f64(W)", "(1.0 - wd) * _f64(W)"),
    ("update sign", "- lr * scale * _f64(D)", "+ lr * scale * _f64(D)"),
    ("Gram update missing one P", "            A = P @ A @ P", "            A = P @ A"),
    ("RowNorm on the unoriented matrix", "    R = unorient(rownorm(X, hp.rownorm_eps), tr)",
     "    R = rownorm(unorient(X, tr), hp.rownorm_eps)"),
]


def _load(src: str, name: str):
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod  # dataclasses resolve the module by name
    try:
        exec(compile(src, ORACLE, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


def _pin_calls():
    """Every non-slow pin with its parametrize arguments expanded."""
    for name, fn in sorted(vars(PINS).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = getattr(fn, "pytestmark", [])
        if any(m.name == "slow" for m in marks):
            continue
        grids = []
        for m in marks:
            if m.name != "parametrize":
                continue
            argnames, values = m.args[0], m.args[1]
            names = [a.strip() for a in argnames.split(",")] if isinstance(argnames, str) else list(argnames)
            opts = []
            for v in values:
                v = v.values if hasattr(v, "values") else v
                v = tuple(v) if len(names) > 1 else (v,)
                opts.append(dict(zip(names, v)))
            grids.append(opts)
        for combo in itertools.product(*grids):
            kw = {}
            for d in combo:
                kw.update(d)
            yield f"{name}{kw if kw else ''}", fn, kw


def _failures(mod, monkeypatch):
    monkeypatch.setattr(PINS, "O", mod)
    failed = []
    for label, fn, kw in _pin_calls():
        try:
            fn(**kw)
        except Exception:  # an assertion, or the mistake breaking a shape
            failed.append(label)
    return failed


SRC = open(ORACLE).read()


def test_unmutated_copy_passes_every_pin(monkeypatch):
    assert _failures(_load(SRC, "oracle_copy"), monkeypatch) == []


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_mutation(what, old, new, monkeypatch):
    assert SRC.count(old) == 1, f"mutation site not unique: {what}"
    mutant = _load(SRC.replace(old, new), "oracle_mutant")
    failed = _failures(mutant, monkeypatch)
    assert failed, f"no pin rejects the mutation: {what}"
