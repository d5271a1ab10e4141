"""The oracle reproduces its own committed outputs (tests/golden/oracle_regression.json,
written by tests/golden/make_oracle_golden.py): any change to its arithmetic shows here."""
import json
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
import make_oracle_golden as g  # noqa: E402

GOLD = json.load(open(g.OUT))


@pytest.mark.parametrize("name", sorted(g.CASES))
def test_oracle_matches_its_golden(name):
    w, path = g.CASES[name]
    ys, final = g.run(w, path)
    ref = GOLD[name]
    np.testing.assert_allclose(ys[0, 0, :8], ref["y_first_step_head0"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ys[-1, 1, :8], ref["y_last_step_head1"], rtol=1e-12, atol=1e-14)
    assert ys.sum() == pytest.approx(ref["y_sum"], rel=1e-12, abs=1e-12)
    assert np.abs(ys).sum() == pytest.approx(ref["y_abs_sum"], rel=1e-12)
    assert final.sum() == pytest.approx(ref["final_state_sum"], rel=1e-12, abs=1e-12)
    assert np.abs(final).sum() == pytest.approx(ref["final_state_abs_sum"], rel=1e-12)
