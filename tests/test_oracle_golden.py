"""The oracle still reproduces its committed regression fixtures (CPU only)."""
import json
import os

import numpy as np
import pytest

from golden import make_golden

DATA = json.load(open(os.path.join(os.path.dirname(make_golden.__file__),
                                   "oracle_regression.json")))


@pytest.mark.parametrize("name", sorted(make_golden.CASES))
def test_oracle_matches_fixture(name):
    out, lse = make_golden.compute(make_golden.CASES[name])
    ref = DATA[name]
    assert list(out.shape) == ref["shape"]
    np.testing.assert_allclose(out.reshape(-1), ref["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse.reshape(-1), ref["lse"], rtol=0, atol=1e-12)
