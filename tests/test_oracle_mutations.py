"""Each planted mistake in the oracle (compiled on the CPU with -DGDN_ORACLE_MUTATION=n)
must fail at least one pin; otherwise the pins would not see that class of mistake."""
import pytest

import oracle
import oracle_pins as P

MUTATIONS = {
    1: "incoming output gradient ignored",
    2: "final-state cotangent ignored",
    3: "dk read after the du update",
    4: "interleaved head map h / r",
    5: "decay dropped from the state gradient",
    6: "previous state used for dq",
    7: "dg from dM before the du update",
    8: "dbeta uses u instead of v - u",
    9: "sign of the prediction error flipped",
    10: "decay applied after the correction",
    11: "beta dropped from dv",
    12: "per-channel gate applied along rows",
}


@pytest.mark.parametrize("m", sorted(MUTATIONS))
def test_planted_mistake_is_caught(m, tmp_path_factory):
    d = str(tmp_path_factory.mktemp(f"mut{m}"))
    orc = oracle.Oracle(mutation=m, out_dir=d, threads=2)
    assert orc.lib.gdn_oracle_mutation() == m
    res = P.battery(orc)
    failed = [n for n, (ok, _) in res.items() if not ok]
    assert failed, f"mutation {m} ({MUTATIONS[m]}) passed every pin: {res}"
