"""The oracle still reproduces the committed snapshots in tests/golden/ (CPU).

The pages print no worked example, so the snapshots hold the oracle's own
values on small seeded inputs (see tests/golden/make_fixtures.py): a change to
the oracle's arithmetic must come with a regenerated, reviewed fixture."""
import importlib.util
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_spec = importlib.util.spec_from_file_location("make_fixtures", os.path.join(GOLDEN, "make_fixtures.py"))
mf = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(mf)


@pytest.mark.parametrize("case", mf.CASES, ids=[c[0] for c in mf.CASES])
def test_oracle_reproduces_the_snapshot(case):
    name, base, kw, rows = case
    w = mf.workload(name, base, kw)
    with open(os.path.join(GOLDEN, name + ".txt")) as f:
        stored = f.read()
    assert mf.render(name, w, rows, mf.compute(w, rows)) == stored
