"""The fp64 oracle against what the pages and the mathematics fix (CPU only).

Pins: exact-rational brute force and the unrolled closed form (acpost page,
section 9.1); identity at beta = 0, alpha = 1; pure decay; exact write at
beta = 1 (separates the decay-first reading from the literal bracket); the
outer-product associative memory; the affine composition law and its
non-commutativity (acpost page, section 1.3); column independence; resume from a
checkpoint equals the uninterrupted run; checkpoint = state after P tokens;
bf16 and fp32 inputs decode exactly (bitwise equal to numpy-widened fp64
inputs); a head subset equals the matching slices of the all-heads run.
The mutation test builds the oracle with each planted mistake and requires that
at least one pin fails for every one of them.
"""
import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    1: "decay dropped",
    2: "read before write",
    3: "sign of the delta-rule residual",
    4: "state read with k instead of q",
    5: "decay only inside the erase term (literal bracket)",
    6: "checkpoint one token early",
    7: "beta dropped from the write",
    8: "decay applied after the write",
    9: "bf16 input decoded with one mantissa bit flipped",
    10: "first selected head used for every selected head",
    11: "fp32 input truncated to 16 bits",
}


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(oracle_lib, pin):
    ok, detail = pin(None)
    assert ok, detail


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[m] for m in sorted(MUTANTS)])
def test_pins_catch_planted_mistake(oracle_lib, mutant):
    path = oracle.build(mutant=mutant)
    assert oracle.load(path).kda_oracle_mutant() == mutant
    failed = [p.__name__ for p in ALL_PINS if not p(path)[0]]
    assert failed, f"no pin caught mutant {mutant} ({MUTANTS[mutant]})"
