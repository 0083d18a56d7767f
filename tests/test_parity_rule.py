"""The parity checker accepts the oracle's own answer and rejects planted
mistakes (planted in a copy of the oracle's result, on the CPU)."""
import numpy as np
import pytest

from full_catalog_ranking_amd import synth
from tests import parity


@pytest.fixture(scope="module")
def case(oracle_mod):
    d = synth.make_dense(6, 64, 2000, seed=13)
    K = 20
    ref = oracle_mod.full(d["H"], d["E"], K)
    g = (ref["idx"].astype(np.int32), ref["score"].astype(np.float32), ref["lse"].astype(np.float32))
    return ref, g


def copy(g):
    return tuple(x.copy() for x in g)


def test_accepts_oracle(case):
    ref, g = case
    parity.check_dense(g, ref)


def test_rejects_wrong_lse(case):
    ref, g = case
    g = copy(g)
    g[2][3] += 2e-3
    with pytest.raises(AssertionError):
        parity.check_dense(g, ref)


def test_rejects_far_swap(case):
    ref, g = case
    g = copy(g)
    g[0][1][[0, 10]] = g[0][1][[10, 0]]
    with pytest.raises(AssertionError):
        parity.check_dense(g, ref)


def test_rejects_foreign_item(case):
    ref, g = case
    g = copy(g)
    outside = int(ref["S"][2].argmin())
    g[0][2][0] = outside
    with pytest.raises(AssertionError):
        parity.check_dense(g, ref)


def test_rejects_score_error(case):
    ref, g = case
    g = copy(g)
    tau = 2e-3 * np.abs(ref["S"]).max()
    g[1][4][5] -= 3 * tau
    g[1][4][6:] = np.minimum(g[1][4][6:], g[1][4][5])
    with pytest.raises(AssertionError):
        parity.check_dense(g, ref)


def test_rejects_missing_padding(oracle_mod):
    d = synth.make_dense(2, 32, 5, seed=1)
    ref = oracle_mod.full(d["H"], d["E"], 8)
    g = (ref["idx"].astype(np.int32), ref["score"].astype(np.float32), ref["lse"].astype(np.float32))
    parity.check_dense(g, ref)
    g[0][0][6] = 3
    with pytest.raises(AssertionError):
        parity.check_dense(g, ref)
