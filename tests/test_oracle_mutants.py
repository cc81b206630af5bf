"""Every planted mistake in the oracle trips at least one pin.

Each mutant is the oracle compiled with -DORACLE_MUTANT=n (see moe_oracle.c):
 1 ties broken toward the higher index      7 sign error in the sigmoid
 2 unstable order inside an expert segment  8 square root dropped from the score
 3 bias leaks into the weights              9 router weights read transposed
 4 scale applied before renormalising      10 down projection indexed transposed
 5 SwiGLU intermediate left unrounded      11 NaN keys ranked first
 6 shared expert dropped                  12 row top-k: k-th and (k+1)-th swapped
The pins are tried cheapest first and the search stops at the first one that
fails, so a mutant costs only the pins it survives.
"""
import pytest

import pins
from oracle import Oracle, build, load

CHEAP_FIRST = sorted(pins.ALL_PINS, key=lambda f: (f.__name__ in (
    "pin_score_correctly_rounded", "pin_topk_bruteforce", "pin_bf16_rounding",
    "pin_f16_decode_all_patterns", "pin_logits_fp64_accuracy"), f.__name__))


@pytest.mark.parametrize("n", range(1, 13))
def test_mutant_is_caught(n, tmp_path):
    orc = Oracle(load(build.build_mutant(n, str(tmp_path))))
    assert orc.mutant() == n
    for pin in CHEAP_FIRST:
        try:
            pin(orc)
        except AssertionError:
            return
    pytest.fail("planted mistake %d passed every pin" % n)
