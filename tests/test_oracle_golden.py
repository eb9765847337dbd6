"""The oracle still reproduces its stored tiny-case results exactly (CPU)."""
import importlib.util
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _load_fixture():
    out = {}
    with open(os.path.join(HERE, "golden", "tiny_oracle.txt")) as f:
        lines = [ln for ln in f.read().splitlines() if not ln.startswith("#")]
    for head, body in zip(lines[0::2], lines[1::2]):
        name, dt, *shape = head.split()
        shape = tuple(int(s) for s in shape)
        if np.dtype(dt).kind == "f":
            vals = np.array([float.fromhex(v) for v in body.split()], np.float64)
        else:
            vals = np.array([int(v) for v in body.split()], dt)
        out[name] = vals.reshape(shape)
    return out


def test_oracle_matches_stored_tiny_results():
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    now = mg.tiny_results()
    ref = _load_fixture()
    assert set(now) == set(ref)
    for name in ref:
        a = np.asarray(now[name])
        if a.dtype.kind == "f":
            assert np.array_equal(a.astype(np.float64), ref[name], equal_nan=True), name
        else:
            assert np.array_equal(a, ref[name]), name
