"""The oracle against its stored regression fixtures (tests/golden, written by make_golden.py).

The fixtures hold what the oracle computed when they were written: codes and scale bytes must
come out identical, floats within 1e-12 relative (BLAS may order a sum differently).  A failure
means the oracle's arithmetic changed; such a change is made on purpose, with the fixtures
regenerated in the same commit.  These are drift guards, not pins against the pages (the oracle's
pins are in the test_oracle_*.py files).
"""

import numpy as np
import pytest

from golden_io import generator_module, read_fixture

MG = generator_module()


def _stored_equals_recomputed(name):
    stored = read_fixture(name)
    header, fn = MG.FIXTURES[name]
    fresh = {}
    for key, text in fn():
        toks = text.split()
        fresh[key] = (np.array([int(t, 16) for t in toks], dtype=np.int64) if toks[0].startswith("0x")
                      else np.array([float(t) for t in toks]))
    assert sorted(stored) == sorted(fresh), name + ": keys differ"
    for key, want in stored.items():
        got = fresh[key]
        assert got.shape == want.shape, key
        if want.dtype == np.int64:
            assert np.array_equal(got, want), "%s %s: codes differ" % (name, key)
        else:
            tol = 1e-12 * max(1.0, float(np.abs(want).max()))
            assert np.max(np.abs(got - want)) <= tol, "%s %s: %.3e" % (name, key, np.max(np.abs(got - want)))
    return stored


@pytest.mark.parametrize("name", ["mx_quantize_tiny.txt", "attn_fwd_tiny.txt", "attn_bwd_tiny.txt"])
def test_oracle_reproduces_fixture(name):
    _stored_equals_recomputed(name)


def test_fixture_shapes_and_ranges():
    q = read_fixture("mx_quantize_tiny.txt")
    for r in range(4):
        assert q["q_row%d_codes" % r].shape == (64,) and q["q_row%d_scales" % r].shape == (2,)
        assert np.all(q["q_row%d_codes" % r] < 16) and np.all(q["q_row%d_scales" % r] < 255)
    f = read_fixture("attn_fwd_tiny.txt")
    for key, val in f.items():
        if key.endswith("_o"):
            assert val.shape == (64,)
        if key.endswith("_l"):
            assert val[0] >= 1.0        # the row's own maximum contributes P~ = 1
    b = read_fixture("attn_bwd_tiny.txt")
    assert all(v.shape == (64,) and np.all(np.isfinite(v)) for v in b.values())
