"""Reading the oracle regression fixtures in tests/golden (no method arithmetic here)."""

import importlib.util
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fixture(name):
    """{key: np.ndarray} from tests/golden/<name>: hex values as int64, others as float64."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":", 1)
            toks = vals.split()
            if toks and toks[0].startswith("0x"):
                out[key.strip()] = np.array([int(t, 16) for t in toks], dtype=np.int64)
            else:
                out[key.strip()] = np.array([float(t) for t in toks], dtype=np.float64)
    return out


def generator_module():
    """tests/golden/make_golden.py as a module (its item functions regenerate every fixture)."""
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(GOLDEN, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod
