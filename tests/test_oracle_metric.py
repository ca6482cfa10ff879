"""Pins of the comparison metric, max-normwise relative error (oracle.max_norm_rel_err):
hand-worked values (tests/golden/max_norm_rel_err.json), its argument order (the
reference is the second argument and sets the denominator), the all-zero reference,
and properties that follow from the definition (scale invariance, bound by the
elementwise ratio, a planted error of known size)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "max_norm_rel_err.json")
CASES = json.load(open(GOLDEN))["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_worked(case):
    assert oracle.max_norm_rel_err(np.array(case["a"]), np.array(case["b"])) == case["err"]


def test_denominator_is_the_reference():
    a = np.array([1.0, 2.0])
    b = np.array([1.0, 4.0])
    # |a - b| = 2 either way; the reference's max is 4, the result's 2
    assert oracle.max_norm_rel_err(a, b) == 0.5
    assert oracle.max_norm_rel_err(b, a) == 1.0


def test_scale_invariant_and_planted_error():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((37, 53))
    big = np.abs(ref).max()
    got = ref.copy()
    got[11, 17] += 0.003 * big              # one element off by 0.3 % of the norm
    assert oracle.max_norm_rel_err(got, ref) == pytest.approx(0.003, rel=1e-12)
    for s in (1e-6, 3.0, 1e6):              # the same ratio at any scale
        assert oracle.max_norm_rel_err(got * s, ref * s) == pytest.approx(0.003, rel=1e-9)


def test_never_above_the_worst_elementwise_ratio():
    # max|a-b| / max|b| <= max over elements of |a-b| / |b| (where b != 0)
    rng = np.random.default_rng(9)
    for _ in range(20):
        b = rng.standard_normal(200) + 0.1
        a = b * (1 + 1e-3 * rng.standard_normal(200))
        elem = np.max(np.abs(a - b) / np.abs(b))
        assert oracle.max_norm_rel_err(a, b) <= elem + 1e-15


def test_accepts_float32_and_lists():
    assert oracle.max_norm_rel_err([[1.0, 2.0]], np.array([[1.0, 2.5]], dtype=np.float32)) == 0.2
