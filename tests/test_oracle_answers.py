"""Pins of the oracle's answer mapping (CoreML conversion metadata page of
clef-flash, "decision.response" and "decision.option_order").

The mapping is a plain definition, so each pin is a closed form or a library
routine independent of it: Python's built-in round() for the 4-decimal
rounding, exact binary ties, one-hot and uniform level distributions for the
score mean, the level-reversal symmetry, and the noul option order [true,
false].  A few plausible slips (levels counted from 1, the wrong noul option,
rounding half up, confidence taken from option 0) are planted and must be
caught by these pins."""
import random

import numpy as np
import pytest

from conftest import table_reader, tiny_spec
from oracle import answers as A
from oracle import head as O
from structured_decision_head_amd import synth

_values = A.answer_values


def _one(t, p, am=None):
    p = np.asarray(p, np.float64)
    am = int(np.argmax(p)) if am is None else am
    v, c = A.answer_values(p, np.array([am]), np.array([t]), np.array([0, len(p)]))
    return float(v[0]), float(c[0])


# -- rounding ----------------------------------------------------------------

def test_round4_matches_python_round():
    rng = random.Random(5)
    xs = [rng.random() for _ in range(20000)] + [rng.uniform(0, 40) for _ in range(5000)]
    xs += [k / 10000 for k in range(0, 10001, 7)] + [(2 * j + 1) / 32 for j in range(16)]
    for x in xs:
        assert A.round4(x) == round(x, 4), x


@pytest.mark.parametrize("x,want", [(1 / 32, 0.0312), (3 / 32, 0.0938), (5 / 32, 0.1562), (7 / 32, 0.2188),
                                    (0.5, 0.5), (1.0, 1.0), (0.0, 0.0), (15.5, 15.5)])
def test_round4_exact_binary_ties_go_to_even(x, want):
    # (2j+1)/32 has x * 10^4 = (2j+1) * 312.5: an exact tie at the 4th decimal
    assert A.round4(x) == want


def test_round4_of_fp32_values():
    # fp32 probabilities: x * 10^4 is exact in float64, so rint gives the same code
    rng = np.random.default_rng(3)
    x32 = rng.random(20000, dtype=np.float32)
    codes = np.rint(x32.astype(np.float64) * 10000.0)
    assert all(A.round4(float(x)) == float(k) / 10000.0 for x, k in zip(x32, codes))


# -- per-type values -----------------------------------------------------------

def test_noul_is_probability_of_true():
    assert _one(A.NOUL, [0.7, 0.3]) == (0.7, 0.7)
    assert _one(A.NOUL, [0.2, 0.8]) == (0.2, 0.8)


def test_choice_value_is_probability_of_argmax():
    p = [0.1, 0.25, 0.4, 0.25]
    assert _one(A.CHOICE, p) == (0.4, 0.4)


@pytest.mark.parametrize("n", [2, 3, 5, 8])
def test_score_one_hot_and_uniform(n):
    for j in range(n):
        p = np.zeros(n)
        p[j] = 1.0
        assert _one(A.SCORE, p) == (float(j), 1.0)
    v, c = _one(A.SCORE, np.full(n, 1.0 / n))
    assert abs(v - (n - 1) / 2) < 1e-12 and abs(c - 1.0 / n) < 1e-15


def test_score_level_reversal():
    rng = np.random.default_rng(11)
    for n in (3, 5, 9):
        p = rng.random(n)
        p /= p.sum()
        v, _ = _one(A.SCORE, p)
        vr, _ = _one(A.SCORE, p[::-1])
        assert abs(v + vr - (n - 1)) < 1e-12


def test_answers_on_oracle_outputs():
    """Over a whole tiny batch: every value is a probability (noul, choice) or a
    level mean inside [0, n-1] (score), every confidence is the largest
    probability and at least 1/n."""
    case = synth.make_case(tiny_spec(seed=31))
    b = case.batch
    lo, po, ao = O.forward(case.weights, case.head, b, table_reader(case))
    v, c = A.answer_values(po, ao, b.q_type, b.o_offsets)
    for q in range(b.NQ):
        p = po[b.o_offsets[q]:b.o_offsets[q + 1]]
        n = len(p)
        assert c[q] == p.max() and c[q] >= 1.0 / n - 1e-15
        if b.q_type[q] == A.SCORE:
            assert 0.0 <= v[q] <= n - 1
        else:
            assert 0.0 <= v[q] <= 1.0
        if b.q_type[q] == A.CHOICE:
            assert v[q] == c[q]


def test_response_shape():
    probs = np.array([0.6, 0.4, 0.2, 0.5, 0.3, 0.1, 0.2, 0.4, 0.2, 0.1])
    r = A.response(probs, np.array([0, 1, 2]), np.array([A.NOUL, A.CHOICE, A.SCORE]),
                   np.array([0, 2, 5, 10]), input_tokens=123, option_ids=[["true", "false"], ["a", "b", "c"],
                                                                            [0, 1, 2, 3, 4]])
    assert r["usage"] == {"input_tokens": 123, "output_tokens": 0}
    a = r["answers"]
    assert a[0] == {"type": "noul", "noul": 0.6}
    assert a[1]["choice"] == "b" and a[1]["confidence"] == 0.5 and a[1]["probabilities"] == {"a": 0.2, "b": 0.5,
                                                                                            "c": 0.3}
    assert a[2]["type"] == "score" and a[2]["score"] == 2.0   # 0.2 + 2*0.4 + 3*0.2 + 4*0.1
    assert a[2]["confidence"] == 0.4


# -- planted slips -------------------------------------------------------------

def _levels_from_one(probs, argmax, q_type, o_offsets):
    v, c = _values(probs, argmax, q_type, o_offsets)
    return np.where(np.asarray(q_type) == A.SCORE, v + 1.0, v), c


def _noul_false(probs, argmax, q_type, o_offsets):
    v, c = _values(probs, argmax, q_type, o_offsets)
    p1 = np.array([probs[int(o_offsets[q]) + 1] if len(probs) > int(o_offsets[q]) + 1 else 0.0
                   for q in range(len(q_type))])
    return np.where(np.asarray(q_type) == A.NOUL, p1, v), c


def _conf_first(probs, argmax, q_type, o_offsets):
    v, _ = _values(probs, argmax, q_type, o_offsets)
    return v, np.array([probs[int(o_offsets[q])] for q in range(len(q_type))])


@pytest.mark.parametrize("mutant", [_levels_from_one, _noul_false, _conf_first])
def test_value_mutants_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(A, "answer_values", mutant)
    caught = False
    for t in (test_noul_is_probability_of_true, test_choice_value_is_probability_of_argmax,
              lambda: test_score_one_hot_and_uniform(5)):
        try:
            t()
        except AssertionError:
            caught = True
    assert caught


def test_round_half_up_mutant_is_caught():
    from decimal import ROUND_HALF_UP, Decimal

    def half_up(x):
        return float(Decimal(float(x)).quantize(Decimal("0.0001"), rounding=ROUND_HALF_UP))

    assert half_up(1 / 32) != 0.0312       # the tie pin above rejects it
    assert any(half_up(x) != round(x, 4) for x in [(2 * j + 1) / 32 for j in range(16)])
