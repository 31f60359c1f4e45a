"""The oracle still produces the locked tiny-workload fixture (tests/golden/)."""
import json
import os

from tests.golden.make_golden import tiny_fixture

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_locked_tiny_fixture():
    with open(os.path.join(HERE, "golden", "tiny_oracle.json")) as f:
        locked = json.load(f)
    assert tiny_fixture() == locked
