import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Mutation testing of the oracle's pins (tests/test_oracle_mutants.py): when
# FP4_ORACLE_MUTATION holds a JSON [module, text, replacement], that oracle
# module is loaded from its source with the one replacement before any test
# imports the oracle, so the CPU pins run against a deliberately wrong oracle.
_MUTATION = os.environ.get("FP4_ORACLE_MUTATION")
if _MUTATION:
    import importlib
    import importlib.util
    import json

    _mod, _old, _new = json.loads(_MUTATION)
    importlib.import_module("oracle")
    _spec = importlib.util.find_spec(_mod)
    with open(_spec.origin) as _f:
        _src = _f.read()
    if _src.count(_old) != 1:
        raise RuntimeError(f"mutation text does not occur exactly once in {_mod}")
    _m = importlib.util.module_from_spec(_spec)
    sys.modules[_mod] = _m
    exec(compile(_src.replace(_old, _new), _spec.origin, "exec"), _m.__dict__)
    setattr(sys.modules["oracle"], _mod.rsplit(".", 1)[1], _m)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """key -> list of tokens, from a golden fixture (comments start with #)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            out[k] = v
    return out


def read_golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows
