"""The oracle against its own stored outputs (tests/golden/oracle_regression.json):
a regression record, not a pin (the pages print no worked example; see
tests/golden/README.md). Integers must match exactly, floats to 1e-12."""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_oracle_matches_its_regression_record():
    want = json.load(open(os.path.join(HERE, "golden", "oracle_regression.json")))
    got = make_golden.compute()
    assert set(want) == set(got)
    for key in want:
        a = np.asarray(got[key])
        b = np.asarray(want[key])
        assert a.shape == b.shape, key
        if np.issubdtype(b.dtype, np.integer):
            assert np.array_equal(a, b), key
        else:
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14, err_msg=key)
