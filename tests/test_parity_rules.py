"""CPU tests of the parity rules the GPU tests apply: the oracle's own
outputs pass; outputs moved past each tolerance fail."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle import parity


@pytest.fixture(scope="module")
def case():
    w = W.Workload("rules", 97, "chain", B=12, K=4, V=3000, dtype="bf16", T=1.0, recipe="peaked",
                   sigma=0.7)
    d = W.chain_inputs(w, 0)
    tok, acc, diag = oracle.verify_chain(d["target"], d["draft"], d["tokens"], d["u_accept"],
                                         d["u_sample"], d["T"], diag=True)
    return d, tok, acc, diag.astype(np.float32)


def test_oracle_outputs_pass(case):
    d, tok, acc, diag = case
    n = parity.check_chain(d, tok, acc, diag)
    assert n["exact"] == n["sequences"] == 12


def test_probability_past_relative_tolerance_fails(case):
    d, tok, acc, diag = case
    bad = diag.copy()
    bad[3, 0, 0] *= 1 + 3e-5
    with pytest.raises(AssertionError, match="P gpu"):
        parity.check_chain(d, tok, acc, bad)
    ok = diag.copy()
    ok[3, 0, 0] = np.float32(float(diag[3, 0, 0]) * (1 + 5e-6))
    parity.check_chain(d, tok, acc, ok)


def test_drawn_mass_within_and_past_its_bound(case):
    d, tok, acc, diag = case
    i = 5
    j = int(acc[i])
    S = float(diag[i, j, 3])
    M = parity._support_mass(d["target"][i, j], d["draft"][i, j] if j < 4 else None, 1.0)
    bound = parity.REL * S + parity.S_MASS_REL * M
    assert M > S > 0
    ok = diag.copy()
    ok[i, j, 3] = S + 0.5 * bound
    parity.check_chain(d, tok, acc, ok)
    bad = diag.copy()
    bad[i, j, 3] = S + 2.0 * bound
    with pytest.raises(AssertionError, match="S gpu"):
        parity.check_chain(d, tok, acc, bad)


def test_support_mass_closed_forms():
    """M is the p + q mass where p > q; for the bonus draw, the mass of p (1)."""
    t = np.log(np.array([0.5, 0.3, 0.2], np.float32))
    q = np.log(np.array([0.2, 0.3, 0.5], np.float32))
    assert parity._support_mass(t, q, 1.0) == pytest.approx(0.7, rel=1e-6)
    assert parity._support_mass(t, None, 1.0) == pytest.approx(1.0, rel=1e-12)


def test_wrong_tokens_and_lengths_fail(case):
    d, tok, acc, diag = case
    bad = tok.copy()
    i = int(np.argmax(acc > 0))
    bad[i, 0] = (bad[i, 0] + 1) % 3000
    with pytest.raises(AssertionError):
        parity.check_chain(d, bad, acc, diag)
    far = tok.copy()
    j = int(acc[2])
    far[2, j] = (int(far[2, j]) + 1500) % 3000
    with pytest.raises(AssertionError, match="drawn token"):
        parity.check_chain(d, far, acc, diag)
    ua = d["u_accept"]
    ratios = diag[:, :4, 2]
    # a sequence whose first tested u is far from its ratio: changing its length must fail
    cand = [b for b in range(12) if abs(float(ua[b, 0]) - float(ratios[b, 0])) > 1e-3]
    b = cand[0]
    la = acc.copy()
    la[b] = 0 if acc[b] != 0 else 1
    with pytest.raises(AssertionError, match="accepted"):
        parity.check_chain(d, tok, la, diag)
