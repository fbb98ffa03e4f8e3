"""Each planted mistake in the oracle (a build with -DORACLE_MUTANT=k) must
fail at least one pin, and the clean build must fail none."""
import pytest

import oracle
from oracle import build as obuild
import oracle_pins as P

MUTANTS = {
    1: "score drops the 64-wide rope term",
    2: "causal alignment off by one",
    3: "page index and slot swapped",
    4: "softmax scale not applied",
    5: "lse in log2 instead of ln",
    6: "output takes the wrong 512 columns",
    7: "fp8 dequantisation ignores k_scale",
    9: "split merge uses equal weights",
    10: "fp8 subnormals decoded 8x too large",
    11: "bf16 decoded with a wrong shift",
    12: "output not divided by the normaliser",
    13: "last visible token dropped",
}


def test_clean_build_passes_all_pins():
    assert P.all_pins(oracle.default()) == []


@pytest.mark.parametrize("k", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, k):
    lib = obuild.build(out=str(tmp_path / f"liboracle_m{k}.so"), mutant=k)
    orc = oracle.Oracle(lib)
    assert orc.lib.oracle_version() == 1 + 1000 * k
    fails = P.all_pins(orc)
    assert fails, f"planted mistake {k} ({MUTANTS[k]}) passed every pin"
