"""The seeded tiny layer and the oracle's answer on it have not drifted."""
import os

from tests.golden import make_golden


def test_tiny_layer_golden():
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    assert make_golden.serialise(make_golden.compute()) == open(os.path.join(here, "tiny_T16.txt")).read()
