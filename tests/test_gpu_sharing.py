"""Heads that share one set of device weights (clef_head_create_sharing), with
batches in flight on two streams at once: every head returns exactly what a
single head returns for the same batch, and a sharing head keeps working
after the head it was made from is destroyed."""
import dataclasses

import numpy as np
import pytest
import torch

from parity import compare, local_offsets, oracle_outputs, say, select
from structured_decision_head_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from structured_decision_head_amd import clefhead
    clefhead.load()


def _same(a, b):
    return all(np.array_equal(x, y) for x, y in zip(a, b))


def test_two_heads_in_flight_match_one_head(gpu):
    from structured_decision_head_amd.runner import HeadRunner
    say("case 3 records H=4096, two sharing heads on two streams")
    spec = synth.CaseSpec("in-flight", 7201, synth.HeadConfig(hidden_size=4096, vocab_size=4096), 3, 1400,
                          ("uniform", 600, 1400), "counts", counts=(1, 2, 1), choice_opts=(2, 6))
    case = synth.make_case(spec)
    r1 = HeadRunner(case)
    r1.set_batch()
    r1.forward()
    ref = r1.outputs()
    # the second head runs another batch (same weights and table, different records)
    other = synth.make_case(dataclasses.replace(spec, seed=7202, B=4, lengths=("uniform", 300, 1400)),
                            with_table=False)
    case2 = dataclasses.replace(case, batch=other.batch)
    r2 = HeadRunner(case2, share=r1)
    r2.set_batch()
    r2.forward()
    ref2 = r2.outputs()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(6):
        r1.forward(s1)
        r2.forward(s2)
    torch.cuda.synchronize()
    assert _same(r1.outputs(), ref)
    assert _same(r2.outputs(), ref2)
    b = case2.batch
    recs = [r for r in range(b.B) if b.q_offsets[r + 1] > b.q_offsets[r]]
    compare("in-flight second head", select(b, recs, *ref2), oracle_outputs(case2, records=recs),
            local_offsets(b, recs))
    # the source head goes first; the sharing head still holds the weights
    r1.close()
    for _ in range(2):
        r2.forward(s2)
    torch.cuda.synchronize()
    assert _same(r2.outputs(), ref2)
    r2.close()
