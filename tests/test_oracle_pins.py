"""The CPU oracle against its pins (no GPU), and evidence that the pins are
sharp: each planted mistake in a rebuilt oracle is caught by the expected pins."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("name", sorted(P.ALL_PINS))
def test_pin(oracle_mod, name):
    P.ALL_PINS[name](oracle_mod, 0)


@pytest.mark.parametrize("mutation", sorted(P.MUTATIONS))
def test_planted_mistake_is_caught(oracle_mod, mutation):
    what, expected = P.MUTATIONS[mutation]
    oracle_mod.build(mutation)
    failed = set()
    for name, fn in P.ALL_PINS.items():
        try:
            fn(oracle_mod, mutation)
        except AssertionError:
            failed.add(name)
    assert expected <= failed, f"mutation {mutation} ({what}): expected {sorted(expected)} to fail, got {sorted(failed)}"
