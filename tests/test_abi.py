"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, enumerates the expected weights, and validates batches on the
host (no GPU needed for any of these calls)."""
import copy
import os
import re
import subprocess

import numpy as np
import pytest

from structured_decision_head_amd import clefhead as C
from structured_decision_head_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "clef_head.h")


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"CLEF_API\s+[\w\s\*]*?\b(clef_head_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    C.load()
    names = declared()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (clef_head_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    assert set(names) == set(C.EXPORTS)
    for n in names:
        assert hasattr(C.load(), n)


def test_weight_list_matches_generator():
    head = synth.HeadConfig()
    specs = synth.weight_specs(head)
    assert C.clef_head_weight_count(head) == len(specs)
    for i, (name, shape, kind, _) in enumerate(specs):
        n, numel, dt = C.clef_head_weight_info(head, i)
        assert n == name and numel == int(np.prod(shape))
        assert dt == (C.CLEF_F32 if kind in ("gate", "scale") else C.CLEF_BF16)


def test_unsupported_config_is_rejected():
    with pytest.raises(C.ClefError) as e:
        C.clef_head_weight_count(synth.HeadConfig(width=512))
    head = synth.HeadConfig(hidden_size=4000)
    with pytest.raises(C.ClefError) as e:
        C.clef_head_weight_info(head, 0)
    assert e.value.code == C.CLEF_E_UNSUPPORTED


@pytest.fixture(scope="module")
def case1():
    spec = synth.config_spec(1, B=3, L=900, lengths=("uniform", 400, 900), head=synth.HeadConfig(vocab_size=512))
    return synth.make_case(spec, with_table=False)


def _args(batch, layout=C.CLEF_PADDED):
    return C.BatchArgs(batch, 0x1000, layout)


def test_check_batch_accepts_valid_padded_and_varlen(case1):
    b = case1.batch
    assert C.clef_head_check_batch(case1.head, _args(b)) == int(b.lengths.sum())
    assert C.clef_head_check_batch(case1.head, _args(b, C.CLEF_VARLEN)) == int(b.lengths.sum())


def test_span_rows_are_exact(case1):
    b = case1.batch
    cu = b.cu_seqlens()
    want = []
    for r in range(b.B):
        for q in range(b.q_offsets[r], b.q_offsets[r + 1]):
            want.append(b.q_span[q] + cu[r])
    for r in range(b.B):
        for q in range(b.q_offsets[r], b.q_offsets[r + 1]):
            for k in range(b.o_offsets[q], b.o_offsets[q + 1]):
                want.append(b.o_span[k] + cu[r])
    for r in range(b.B):
        want.append([cu[r + 1] - 1, cu[r + 1]])
    got = C.clef_head_span_rows(case1.head, _args(b), b.NQ + b.NO + b.B)
    np.testing.assert_array_equal(got, np.array(want, np.int32))
    got2 = C.clef_head_span_rows(case1.head, _args(b, C.CLEF_VARLEN), b.NQ + b.NO + b.B)
    np.testing.assert_array_equal(got, got2)


def _mutated(case1, fn):
    b = copy.deepcopy(case1.batch)
    fn(b)
    return b


@pytest.mark.parametrize("what,code", [
    ("span_empty", C.CLEF_E_SPAN), ("span_past_end", C.CLEF_E_SPAN), ("opt_span_neg", C.CLEF_E_SPAN),
    ("id_high", C.CLEF_E_ID), ("id_neg", C.CLEF_E_ID), ("type_bad", C.CLEF_E_SCHEMA),
    ("noul_three", C.CLEF_E_SCHEMA), ("no_options", C.CLEF_E_SCHEMA), ("mask_hole", C.CLEF_E_LENGTH),
    ("empty_record", C.CLEF_E_LENGTH), ("q_offsets_bad", C.CLEF_E_SCHEMA),
])
def test_validation_errors(case1, what, code):
    b = copy.deepcopy(case1.batch)
    mask = None
    if what == "span_empty":
        b.q_span[0, 1] = b.q_span[0, 0]
    elif what == "span_past_end":
        b.q_span[0, 1] = b.lengths[0] + 1
    elif what == "opt_span_neg":
        b.o_span[0, 0] = -1
    elif what == "id_high":
        b.o_ids[3] = case1.head.vocab_size
    elif what == "id_neg":
        b.o_ids[0] = -5
    elif what == "type_bad":
        b.q_type[1] = 3
    elif what == "noul_three":
        q = int(np.where(b.q_type == synth.NOUL)[0][0])
        b.q_type[q] = synth.NOUL
        # give the noul question a third option by stealing one from the next question
        nxt = q + 1
        if b.o_offsets[nxt + 1] - b.o_offsets[nxt] > 1:
            b.o_offsets[q + 1] += 1
        else:
            b.q_type[q] = synth.NOUL
            b.o_offsets[q + 1] -= 1
    elif what == "no_options":
        b.o_offsets[1] = b.o_offsets[0]
    elif what == "mask_hole":
        mask = b.key_mask()
        mask[0, 5] = 0
    elif what == "empty_record":
        mask = b.key_mask()
        mask[1, :] = 0
    elif what == "q_offsets_bad":
        b.q_offsets[-1] += 1
    a = _args(b)
    if mask is not None:
        a._keep.append(mask)
        a.struct.key_mask = mask.ctypes.data
    with pytest.raises(C.ClefError) as e:
        C.clef_head_check_batch(case1.head, a)
    assert e.value.code == code, str(e.value)


def test_null_arguments_are_errors(case1):
    a = _args(case1.batch)
    a.struct.q_offsets = None
    with pytest.raises(C.ClefError) as e:
        C.clef_head_check_batch(case1.head, a)
    assert e.value.code == C.CLEF_E_ARG
    a = _args(case1.batch)
    a.struct.hidden = None
    with pytest.raises(C.ClefError):
        C.clef_head_check_batch(case1.head, a)


def test_create_without_gpu_or_with_bad_weights_fails_cleanly():
    head = synth.HeadConfig(hidden_size=512, vocab_size=64, routing_layers=0, layers=0)
    w = synth.make_weights(head, 1)
    w.pop("mem.w")
    with pytest.raises(C.ClefError) as e:
        C.clef_head_create(head, w, 0x1000)
    # missing weight (or no device here): either way an error code, never a crash
    assert e.value.code in (C.CLEF_E_ARG, C.CLEF_E_HIP)


def test_create_sharing_rejects_null_source():
    with pytest.raises(C.ClefError) as e:
        C.clef_head_create_sharing(0)
    assert e.value.code == C.CLEF_E_ARG


def test_forward_answers_rejects_null_before_any_work(case1):
    """NULL answers (or a NULL handle) is refused on the host with CLEF_E_ARG."""
    args = C.BatchArgs(case1.batch, 0)
    L = C.load()
    rc = L.clef_head_forward_answers(None, C.ctypes.byref(args.struct), None, None, None, None, None)
    assert rc == C.CLEF_E_ARG
    ans = C.clef_head_answers()
    rc = L.clef_head_forward_answers(None, C.ctypes.byref(args.struct), None, None, None, C.ctypes.byref(ans), None)
    assert rc == C.CLEF_E_ARG


def test_weight_list_of_the_decoder_field_variant():
    head = synth.HeadConfig(field_cross_attention=1)
    specs = synth.weight_specs(head)
    assert C.clef_head_weight_count(head) == len(specs) == len(synth.weight_specs(synth.HeadConfig())) + 40
    for i, (name, shape, kind, _) in enumerate(specs):
        n, numel, dt = C.clef_head_weight_info(head, i)
        assert n == name and numel == int(np.prod(shape))
    with pytest.raises(C.ClefError) as e:
        C.clef_head_weight_count(synth.HeadConfig(field_cross_attention=2))
    assert e.value.code == C.CLEF_E_ARG


def test_question_with_too_many_options_is_refused():
    spec = synth.CaseSpec(name="too-many", seed=5, head=synth.HeadConfig(vocab_size=512), B=1, L=None,
                          lengths=("fixed", 3400, 3400), fields="ordered", ordered=((synth.CHOICE, 1025),),
                          opt_len=(1, 1), instr_len=(2, 4))
    case = synth.make_case(spec, with_table=False)
    args = C.BatchArgs(case.batch, 1)
    with pytest.raises(C.ClefError) as e:
        C.clef_head_check_batch(case.head, args)
    assert e.value.code == C.CLEF_E_UNSUPPORTED
