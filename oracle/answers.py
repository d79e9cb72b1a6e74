"""Answer mapping of the head's per-question softmax into the decision response.

TEST INFRASTRUCTURE ONLY.  Nothing in the library path imports, calls or links
this module: only tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library.

Source: the CoreML conversion metadata page of clef-flash, "decision.response"
(per question type: a noul question answers with the probability of "true"; a
choice question with the id of its most probable option, that option's
probability as confidence and every option's probability; a score question
with the probability-weighted mean level, the largest probability as
confidence and every level's probability; numbers carry 4 decimals; usage
counts the record's tokens as input and none as output) and
"decision.option_order" (noul options are [true, false]; score options are the
levels 0..n-1 in order).

Readings taken where the page leaves a step open:
  * "4 decimals" is round-half-to-even of the exact binary value of the number
    at the fourth decimal place (what Python's round(x, 4) does).
  * A noul answer has no confidence on the page; its confidence slot holds the
    largest probability of the two, like the other types.
  * A choice question's numeric value is the probability of its answer (the
    answer itself is the argmax index).
"""
from __future__ import annotations

from decimal import ROUND_HALF_EVEN, Decimal
from typing import Dict, List

import numpy as np

NOUL, CHOICE, SCORE = 0, 1, 2
_QUANTUM = Decimal("0.0001")


def round4(x: float) -> float:
    """Round half to even at the fourth decimal of the exact value of x."""
    return float(Decimal(float(x)).quantize(_QUANTUM, rounding=ROUND_HALF_EVEN))


def answer_values(probs: np.ndarray, argmax: np.ndarray, q_type: np.ndarray, o_offsets: np.ndarray):
    """Per question: (value, confidence), both float64 [NQ].

    noul  : value = p(true) (option 0), confidence = max p
    choice: value = confidence = p of the argmax option
    score : value = sum over levels i of i * p_i, confidence = max p
    """
    NQ = len(q_type)
    value = np.zeros(NQ)
    conf = np.zeros(NQ)
    for q in range(NQ):
        p = np.asarray(probs[int(o_offsets[q]):int(o_offsets[q + 1])], dtype=np.float64)
        conf[q] = p.max()
        t = int(q_type[q])
        if t == NOUL:
            value[q] = p[0]
        elif t == CHOICE:
            value[q] = p[int(argmax[q])]
        elif t == SCORE:
            value[q] = sum(i * p[i] for i in range(len(p)))
        else:
            raise ValueError(f"question type {t}")
    return value, conf


def response(probs, argmax, q_type, o_offsets, input_tokens: int, question_ids=None, option_ids=None) -> Dict:
    """The response object of one record, numbers rounded to 4 decimals.

    question_ids / option_ids name the questions and (per question) the options;
    by default they are the indices."""
    value, conf = answer_values(probs, argmax, q_type, o_offsets)
    answers = {}
    for q in range(len(q_type)):
        o0, o1 = int(o_offsets[q]), int(o_offsets[q + 1])
        qid = question_ids[q] if question_ids is not None else q
        ids: List = option_ids[q] if option_ids is not None else list(range(o1 - o0))
        pr = {ids[i]: round4(probs[o0 + i]) for i in range(o1 - o0)}
        t = int(q_type[q])
        if t == NOUL:
            answers[qid] = {"type": "noul", "noul": round4(value[q])}
        elif t == CHOICE:
            answers[qid] = {"type": "choice", "choice": ids[int(argmax[q])], "confidence": round4(conf[q]),
                            "probabilities": pr}
        else:
            answers[qid] = {"type": "score", "score": round4(value[q]), "confidence": round4(conf[q]),
                            "probabilities": pr}
    return {"answers": answers, "usage": {"input_tokens": int(input_tokens), "output_tokens": 0}}
