"""Planted mistakes in the oracle (built on the CPU into a temporary
directory) must each fail at least one pin.  Mutations: 1 previous packed node
as parent; 2 decay dropped; 3 sign of the delta correction; 4 transposed
state; 5 conv tap from the previous packed row; 6 conv taps reversed; 7 commit
drops the frontier step; 8 the q/k normalisation floor added outside the
square root; 9 the published conv history stored newest first; 10 the
stored delta correction taken before the write strength beta."""
import pytest

import oracle
from oracle_pins import failing_pins


@pytest.mark.parametrize("mutation", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
def test_planted_mistake_is_caught(mutation, tmp_path):
    path = oracle.build(force=True, mutation=mutation, outdir=str(tmp_path))
    lib = oracle.load(path)
    assert failing_pins(lib), f"mutation {mutation} passed every pin"


def test_clean_build_passes_every_pin():
    assert failing_pins(oracle.load()) == []
