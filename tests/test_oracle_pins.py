"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
import oracle_pins as P

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle(threads=4)


@pytest.mark.parametrize("case", range(3))
def test_finite_differences_all_six_gradients(orc, case):
    shape, x = P.standard_fd_cases()[case]
    ok, msg = P.pin_finite_differences(orc, shape, x)
    assert ok, msg


def test_euler_identities(orc):
    for seed, kw in ((201, dict(T=9, S_k=8, S_v=8, lens=[9, 6])),
                     (202, dict(kda=False, T=9, H_k=1, H_v=3, S_k=6, S_v=6))):
        shape, x = P.rand_problem(seed, **kw)
        ok, msg = P.pin_euler(orc, shape, x)
        assert ok, msg


def test_closed_forms(orc):
    ok, msg = P.pin_closed_forms(orc)
    assert ok, msg


def test_scalar_gate_equals_kda_with_equal_columns(orc):
    ok, msg = P.pin_scalar_equals_kda(orc)
    assert ok, msg


def test_gqa_equals_explicit_repeat(orc):
    ok, msg = P.pin_gqa_equals_repeat(orc)
    assert ok, msg


def test_row_additivity(orc):
    ok, msg = P.pin_row_additivity(orc)
    assert ok, msg


def test_checkpoint_interval_is_bit_invariant(orc):
    ok, msg = P.pin_checkpoint_invariance(orc)
    assert ok, msg


def test_thread_count_is_bit_invariant():
    shape, x = P.rand_problem(61, n_seqs=3, T=10, H_k=2, H_v=6, S_k=8, S_v=8, lens=[10, 3, 7])
    # order-sensitive magnitudes (mixing 1e6 with 1e-6) make any reordering visible
    x["v"][0, :, 0] *= 1e6
    x["v"][1, :, 2] *= 1e-6
    outs = []
    for th in (1, 3, 8):
        o = oracle.Oracle(threads=th)
        outs.append(o.bwd(shape, *(x[n] for n in P.INPUTS), x["gy"], x["dstate_out"]))
    for o in outs[1:]:
        for n in P.GRADS:
            assert np.array_equal(o[n], outs[0][n]), n


def test_padding_is_never_read_and_written_zero(orc):
    shape, x = P.rand_problem(71, n_seqs=3, T=8, lens=[8, 5, 0])
    ref_y, ref_so = orc.fwd(shape, *(x[n] for n in P.INPUTS))
    ref = orc.bwd(shape, *(x[n] for n in P.INPUTS), x["gy"], x["dstate_out"])
    xn = {k: v.copy() for k, v in x.items()}
    for s, L in enumerate(shape["seq_lens"]):
        for n in ("q", "k", "v", "g", "beta", "gy"):
            xn[n][s, L:] = np.nan
    y, so = orc.fwd(shape, *(xn[n] for n in P.INPUTS))
    d = orc.bwd(shape, *(xn[n] for n in P.INPUTS), xn["gy"], xn["dstate_out"])
    assert np.array_equal(y, ref_y) and np.array_equal(so, ref_so)
    for n in P.GRADS:
        assert np.array_equal(d[n], ref[n]), n
    for s, L in enumerate(shape["seq_lens"]):
        for n in ("dq", "dk", "dv", "dg", "dbeta"):
            assert not np.any(d[n][s, L:]), n
        assert not np.any(y[s, L:])
    # an empty sequence passes its state and its cotangent straight through
    assert np.array_equal(so[2], x["state0"][2])
    assert np.array_equal(d["dstate"][2], x["dstate_out"][2])


def test_workspace_formula_matches_pages():
    """Pins the checkpoint-interval reading C = ceil(sqrt(T)), n_ck = ceil(T / C) against the
    scratch size the pages print for S_v = 128 at a window of 8192 tokens and 48 heads."""
    with open(os.path.join(HERE, "golden", "workspace_formula.json")) as f:
        g = json.load(f)
    assert oracle.default_C(g["T"]) == g["C"]
    per_head = oracle.workspace_formula_bytes(g["S_v"], g["T"])
    assert per_head == g["bytes_per_head"]
    assert abs(per_head / 2**20 - g["printed_MiB_per_head"]) < 0.05
    assert round(per_head * g["heads"] / 2**20) == g["printed_MiB_per_op"]


@pytest.mark.parametrize("T,C", [(1, 1), (2, 2), (4, 2), (5, 3), (16, 4), (64, 8), (4096, 64),
                                 (65536, 256), (8192, 91), (8191, 91), (8281, 91), (8282, 92)])
def test_default_checkpoint_interval(T, C):
    assert oracle.default_C(T) == C
