"""The parity measures of tests/ttt_testutil.py on hand-made cases (CPU)."""
import numpy as np
import pytest

from ttt_testutil import errors, max_rel, parity


def test_errors_hand_made():
    ref = np.array([[[1.0, -4.0], [0.0, 2.0]], [[10.0, 0.0], [0.0, 0.0]]])   # two chains
    x = ref.copy()
    x[0, 0, 0] += 0.04           # chain 0: max|ref| = 4 -> max-norm 0.01, elementwise 0.04
    x[0, 1, 0] += 1e-5           # ref 0: elementwise floor 1e-6 * 4 -> 2.5
    x[1, 0, 0] -= 0.3            # chain 1: max-norm 0.03, elementwise 0.03
    e = errors(x, ref)
    assert e["max"] == pytest.approx(0.03)
    assert e["elem"] == pytest.approx(1e-5 / 4e-6)
    frob0 = np.sqrt(0.04 ** 2 + 1e-10) / np.sqrt(1 + 16 + 4)
    frob1 = 0.3 / 10.0
    assert e["frob"] == pytest.approx(max(frob0, frob1))
    assert max_rel(x, ref) == pytest.approx(0.03)


def test_errors_zero_reference_chain():
    ref = np.zeros((1, 3))
    x = np.array([[0.0, 1e-9, 0.0]])
    e = errors(x, ref)                   # an all-zero chain is compared in absolute terms
    assert e["max"] == pytest.approx(1e-9) and e["frob"] == pytest.approx(1e-9)


def test_parity_asserts_both_bounds():
    ref = np.ones((2, 4))
    parity("ok", [("a", ref * (1 + 1e-6), ref)], 2e-3, 5e-5)
    with pytest.raises(AssertionError, match="regression bound"):
        parity("regress", [("a", ref * (1 + 1e-4), ref)], 2e-3, 5e-5)
    with pytest.raises(AssertionError, match="contract"):
        parity("contract", [("a", ref * (1 + 1e-2), ref)], 2e-3, None)
