"""The oracle against its stored regression digests (tests/golden/, written
by tests/golden/make_golden.py from the oracle alone).  A failure means the
oracle's arithmetic changed: regenerate the file only together with the
reading of the pages that justifies the change."""

import importlib.util
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _maker():
    spec = importlib.util.spec_from_file_location("make_golden",
                                                  os.path.join(HERE, "golden", "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_oracle_matches_stored_digests():
    mk = _maker()
    with open(mk.OUT) as f:
        stored = json.load(f)
    now = mk.cases()
    assert set(now) == set(stored)
    for case, outs in stored.items():
        assert set(now[case]) == set(outs), case
        for key, d in outs.items():
            got = now[case][key]
            assert got["dtype"] == d["dtype"] and got["shape"] == d["shape"], f"{case}.{key}"
            assert got["sha256"] == d["sha256"], f"{case}.{key}: oracle output changed"
