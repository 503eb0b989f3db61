"""The fp64 oracle against closed forms, brute force, torch fp64 and invariants (CPU)."""
import json
import os

import pytest

import oracle
from tests import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_retention_counts_from_pages():
    """Keeping one indexer in four (FSSS) removes 75% of indexer runs."""
    with open(os.path.join(GOLDEN, "indexcache_retention.json")) as f:
        g = json.load(f)
    P.pin_stack_counts(oracle, g["cases"])
    for c in g["cases"]:
        assert 1 - c["expected_indexer_calls"] / c["n_layers"] == pytest.approx(
            g["indexer_compute_removed"])


@pytest.mark.parametrize("bad", ["SFFF", "FSX", "FSS"])
def test_pattern_validation(bad):
    with pytest.raises(ValueError):
        oracle.validate_pattern(bad, 4)
