"""The oracle against its pins, and the pins against planted mistakes."""
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("pin", P.ORACLE_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)


MUTANTS = {
    1: "scale dropped",
    2: "query head mapped to KV head h % H_kv",
    3: "in-block offset off by one",
    4: "softmax without max subtraction",
    5: "newest token left out of the normaliser",
    6: "keys used in place of values",
    7: "pool head and slot axes swapped",
    8: "slot split into block/offset the wrong way round",
    9: "block copy skips the value pool",
    10: "sign of the exponent flipped",
    11: "E4M3 exponent bias 8",
    12: "values scaled by the key scale",
    13: "E4M3 ties rounded away from zero",
    14: "E4M3 encode without saturation",
    15: "key scale taken from the logical block",
    16: "a query token does not attend to itself",
    17: "query positions shifted by one",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_planted_mistake_is_caught(mutant):
    m = oracle.build_mutant(mutant)
    caught = []
    for pin in P.ORACLE_PINS:
        try:
            pin(m)
        except (AssertionError, oracle.OracleError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {mutant} ({MUTANTS[mutant]}) passed every pin"
