"""The oracle's outputs on the small fixtures still hash to the committed
manifest (written by tests/golden/make_golden.py from the oracle alone)."""
import json
from pathlib import Path

import pytest

from golden.make_golden import OUT, manifest


def test_oracle_matches_golden_manifest():
    want = json.loads(Path(OUT).read_text())
    got = manifest()
    for case, fields in want.items():
        for name, h in fields["inputs"].items():
            assert got[case]["inputs"][name] == h, f"input drift: {case}.{name}"
        for name, h in fields.items():
            if name != "inputs":
                assert got[case][name] == h, f"oracle drift: {case}.{name}"
