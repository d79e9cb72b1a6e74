"""GPU parity of the fp16-hidden variant (CLEF_HIDDEN_F16: the CoreML packaging
of clef-flash hands the head fp16 hidden states, CoreML conversion metadata
page "decision.head").  Row statistics, span pooling and the memory GEMM read
fp16 rows (fp16 MFMA with an fp16 copy of the folded memory weight); the rest
of the head is the bf16-storage / fp32-accumulation path.  Same tolerances as
the bf16 path: max |d logit| <= 2e-2, max |d prob| <= 2e-3, argmax per the
near-tie rule."""
import dataclasses

import numpy as np
import pytest

from oracle import head as O
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


def _run(case, layout=None):
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    r = HeadRunner(case)
    r.set_batch(None, C.CLEF_PADDED if layout is None else layout)
    r.forward()
    out = r.outputs()
    r.close()
    return out


def _check(case, out, name, recs=None):
    b = case.batch
    recs = [r for r in range(b.B) if int(b.q_offsets[r + 1]) > int(b.q_offsets[r])] if recs is None else recs
    ref = oracle_outputs(case, records=recs)
    compare(f"{name} ({len(recs)} records)", select(b, recs, *out), ref, local_offsets(b, recs))
    return ref


def test_f16_mini_ragged_and_same_values_as_bf16(torch_gpu):
    """A ragged 3-record batch in fp16; then hidden values that bf16 and fp16
    both hold exactly, run once per encoding: both match the same oracle
    outputs."""
    spec = synth.config_spec(1, B=3, L=1100, lengths=("uniform", 600, 1100), head=synth.HeadConfig(vocab_size=4096),
                             hidden_dtype="f16")
    case = synth.make_case(spec)
    say("case mini ragged, fp16 hidden")
    _check(case, _run(case), "mini fp16")

    cb = synth.make_case(dataclasses.replace(spec, hidden_dtype="bf16", seed=spec.seed + 1))
    b = cb.batch
    x = O.from_bf16(b.hidden)
    bits = np.where(np.abs(x) >= 2.0 ** -14, b.hidden, np.uint16(0)).astype(np.uint16)
    h = O.from_bf16(bits).astype(np.float16)
    assert np.array_equal(h.astype(np.float64), O.from_bf16(bits))
    case_b = dataclasses.replace(cb, batch=dataclasses.replace(b, hidden=bits))
    case_h = dataclasses.replace(cb, batch=dataclasses.replace(b, hidden=h.view(np.uint16), hidden_dtype="f16"))
    say("case same values, bf16 and fp16 encodings")
    ob, oh = _run(case_b), _run(case_h)
    ref = _check(case_b, ob, "same values bf16")
    recs = list(range(b.B))
    compare("same values fp16", select(b, recs, *oh), ref, local_offsets(b, recs))


def test_f16_online_serving_full_size(torch_gpu):
    case = synth.make_case(dataclasses.replace(synth.config_spec(1), hidden_dtype="f16"))
    b = case.batch
    say(f"case online-serving full size, fp16 hidden: B={b.B} T={int(b.lengths.sum())} NO={b.NO}")
    _check(case, _run(case), "online-serving fp16")


def test_f16_h5120_padded_vs_varlen_nan_padding(torch_gpu):
    """H=5120, NaN (fp16 0x7E00) padding rows: padded and varlen runs agree bit
    for bit and match the oracle."""
    from structured_decision_head_amd import clefhead as C
    spec = synth.config_spec(4, B=5, lengths=("loguniform", 300, 2500), hidden_dtype="f16", vocab_size=4096)
    case = synth.make_case(spec)
    b = case.batch
    assert b.hidden_dtype == "f16"
    say(f"case H=5120 fp16, NaN padding: B={b.B} L={b.L} lengths={b.lengths.tolist()}")
    op = _run(case, C.CLEF_PADDED)
    ov = _run(case, C.CLEF_VARLEN)
    for a, c in zip(op, ov):
        assert np.array_equal(a, c)
    _check(case, op, "H=5120 fp16")
