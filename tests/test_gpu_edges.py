"""GPU parity on the degenerate and boundary cases of a batch.

* a question with 300 options (the per-question kernels loop over options in
  several waves) next to a single-option question (softmax 1, argmax 0);
* records without questions between records with questions (they take no
  rows, tiles or attention work, and must not shift anyone else's results);
* a batch with no questions at all (nothing to compute, the call succeeds);
* a record whose length is an exact multiple of the 256-row tile.
"""
import dataclasses

import numpy as np
import pytest

from parity import compare, local_offsets, oracle_outputs, say, select
from structured_decision_head_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from structured_decision_head_amd import clefhead
    clefhead.load()
    return torch


def _spec(name, seed, **kw):
    base = dict(name=name, seed=seed, head=synth.HeadConfig(hidden_size=4096, vocab_size=4096), B=2, L=None,
                lengths=("fixed", 1600, 1600), fields="ordered")
    base.update(kw)
    return synth.CaseSpec(**base)


def _run(case):
    from structured_decision_head_amd.runner import HeadRunner
    r = HeadRunner(case)
    r.set_batch()
    r.forward()
    out = r.outputs()
    r.close()
    return out


def _check_all(case, out, name):
    b = case.batch
    recs = [r for r in range(b.B) if int(b.q_offsets[r + 1]) > int(b.q_offsets[r])]
    ref = oracle_outputs(case, records=recs)
    compare(f"{name} ({len(recs)} records)", select(b, recs, *out), ref, local_offsets(b, recs))


def drop_questions(batch, r):
    """The same batch with record r's questions, options and option ids removed."""
    q0, q1 = int(batch.q_offsets[r]), int(batch.q_offsets[r + 1])
    o0, o1 = int(batch.o_offsets[q0]), int(batch.o_offsets[q1])
    ido = batch.o_id_offsets()
    i0, i1 = int(ido[o0]), int(ido[o1])
    nq, no = q1 - q0, o1 - o0
    q_off = np.concatenate([batch.q_offsets[:r + 1], batch.q_offsets[r + 1:] - nq]).astype(np.int32)
    o_off = np.concatenate([batch.o_offsets[:q0 + 1], batch.o_offsets[q1 + 1:] - no]).astype(np.int32)
    return dataclasses.replace(
        batch, q_offsets=q_off,
        q_type=np.delete(batch.q_type, np.s_[q0:q1]), q_span=np.delete(batch.q_span, np.s_[q0:q1], axis=0),
        o_offsets=o_off, o_span=np.delete(batch.o_span, np.s_[o0:o1], axis=0),
        o_ids=np.delete(batch.o_ids, np.s_[i0:i1]))


def test_many_options_and_single_option(torch_gpu):
    say("case 300-option choice + 1-option choice + noul + score")
    spec = _spec("wide-question", 7101, ordered=((synth.CHOICE, 300), (synth.CHOICE, 1), (synth.NOUL, 2),
                                                 (synth.SCORE, 5)), opt_len=(1, 2))
    case = synth.make_case(spec)
    b = case.batch
    assert int(np.diff(b.o_offsets).max()) == 300
    logits, probs, amax = _run(case)
    _check_all(case, (logits, probs, amax), "wide-question")
    single = [q for q in range(b.NQ) if int(b.o_offsets[q + 1]) - int(b.o_offsets[q]) == 1]
    assert single
    for q in single:
        k = int(b.o_offsets[q])
        assert probs[k] == 1.0 and amax[q] == 0


def test_records_without_questions(torch_gpu):
    say("case 5 records, records 1 and 3 without questions")
    spec = _spec("holes", 7102, B=5, lengths=("uniform", 700, 1300), L=1300, fields="counts", counts=(1, 2, 1))
    case = synth.make_case(spec)
    full = _run(case)
    holes = dataclasses.replace(case, batch=drop_questions(drop_questions(case.batch, 3), 1))
    assert int(holes.batch.q_offsets[2] - holes.batch.q_offsets[1]) == 0
    got = _run(holes)
    _check_all(holes, got, "holes")
    # the remaining records' outputs are those of the full batch
    b = case.batch
    keep = [0, 2, 4]
    ref = select(b, keep, *full)
    for a, c in zip(select(holes.batch, keep, *got), ref):
        assert np.allclose(a, c, rtol=0, atol=1e-3)


def test_batch_without_questions(torch_gpu):
    say("case 2 records, no questions")
    spec = _spec("empty", 7103, fields="counts", counts=(1, 1, 0), lengths=("fixed", 600, 600))
    case = synth.make_case(spec)
    b = drop_questions(drop_questions(case.batch, 1), 0)
    assert b.NQ == 0 and b.NO == 0
    logits, probs, amax = _run(dataclasses.replace(case, batch=b))
    assert logits.size == 0 and probs.size == 0 and amax.size == 0


def test_tile_multiple_lengths(torch_gpu):
    say("case records of exactly 512 and 768 rows")
    spec = _spec("tile-multiple", 7104, B=2, lengths=("fixed", 512, 512), fields="counts", counts=(1, 1, 1))
    case = synth.make_case(spec)
    lengths = case.batch.lengths.copy()
    lengths[1] = 768
    batch = dataclasses.replace(case.batch, lengths=lengths)
    if batch.hidden.shape[1] < 768:
        pad = np.zeros((batch.B, 768 - batch.hidden.shape[1], batch.hidden.shape[2]), np.uint16)
        g = np.random.default_rng(7104)
        pad[1] = synth.f32_to_bf16_bits(g.standard_normal(pad[1].shape, dtype=np.float32))
        batch = dataclasses.replace(batch, hidden=np.concatenate([batch.hidden, pad], axis=1))
    # record 1's schema sits at the end of its first 512 tokens; move it to the end of 768
    shift = 256
    q0, q1 = int(batch.q_offsets[1]), int(batch.q_offsets[2])
    o0, o1 = int(batch.o_offsets[q0]), int(batch.o_offsets[q1])
    q_span = batch.q_span.copy()
    o_span = batch.o_span.copy()
    q_span[q0:q1] += shift
    o_span[o0:o1] += shift
    batch = dataclasses.replace(batch, q_span=q_span, o_span=o_span)
    case = dataclasses.replace(case, batch=batch)
    _check_all(case, _run(case), "tile-multiple")


@pytest.mark.parametrize("B,L", [(1, 200), (1, 2048), (3, 1000), (2, 4096)])
def test_split_k_big_gemms(torch_gpu, B, L):
    """Batches of few 256-row tiles split the K of the memory and K/V GEMMs
    into slices (1 tile: 8 and 4 slices; 8 tiles: 8 and 1; 3 records of 4
    tiles: 4 and 1; 32 tiles: none) whose partial sums a reduction kernel
    adds in order before the epilogue; the result must match the oracle like
    the unsplit GEMMs do."""
    spec = _spec(f"split-{B}x{L}", 7200 + B * 10 + L // 100, B=B, L=L, lengths=("fixed", L, L), fields="counts",
                 counts=(2, 2, 1), choice_opts=(2, 5), instr_len=(2, 6), opt_len=(1, 4))
    say(f"case split-K big GEMMs: B={B} L={L}")
    case = synth.make_case(spec)
    out = _run(case)
    _check_all(case, out, f"split {B}x{L}")


@pytest.mark.parametrize("H", [512, 8192])
def test_smallest_and_largest_hidden_size(torch_gpu, H):
    """hidden_size 512 and 8192, the ends of the supported range (row kernels
    with 1 and 16 chunks per lane, memory GEMM depth 512 and 8192)."""
    spec = _spec(f"hidden-{H}", 7400 + H // 512, head=synth.HeadConfig(hidden_size=H, vocab_size=4096), B=2,
                 lengths=("uniform", 700, 1300), fields="counts", counts=(2, 2, 1), choice_opts=(2, 5))
    say(f"case hidden size {H}")
    case = synth.make_case(spec)
    _check_all(case, _run(case), f"H={H}")


def test_records_with_more_than_64_fields(torch_gpu):
    """Records of 70 fields: the field attention takes each record's fields in
    two 64-row query blocks, and its W_o share runs once per block."""
    spec = _spec("many-fields", 7601, B=2, lengths=("fixed", 1600, 1600), fields="counts", counts=(40, 20, 10),
                 choice_opts=(2, 3), opt_len=(1, 2), instr_len=(2, 4))
    say("case 2 records of 70 fields")
    case = synth.make_case(spec)
    assert int(np.diff(case.batch.q_offsets).min()) == 70
    _check_all(case, _run(case), "70 fields")


def test_question_with_the_most_options(torch_gpu):
    """A question with 1024 options, the most the per-question kernels hold."""
    spec = _spec("max-options", 7501, B=1, lengths=("fixed", 3400, 3400), fields="ordered",
                 ordered=((synth.CHOICE, 1024), (synth.NOUL, 2)), opt_len=(1, 1), instr_len=(2, 4))
    say("case question with 1024 options")
    case = synth.make_case(spec)
    assert int(np.diff(case.batch.o_offsets).max()) == 1024
    _check_all(case, _run(case), "1024 options")
