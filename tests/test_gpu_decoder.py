"""GPU parity of the decoder-layer field variant (field_cross_attention = 1:
each field layer also cross-attends, pre-LN, over its record's memory rows;
clef-4bit page §三 step 3 and the architecture page §3.2 call the field
layers transformer decoder layers).  The fields' K/V come from one more big
K/V GEMM over the memory rows, the cross-attention runs in the routing
attention kernels with the fields as queries.  Same tolerances as the rest of
the head; the streamed path must stay bit-identical to the whole-batch
forward."""
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


def _variant(spec):
    return dataclasses.replace(spec, head=dataclasses.replace(spec.head, field_cross_attention=1))


def _run(case, layout=None):
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    r = HeadRunner(case)
    r.set_batch(None, C.CLEF_PADDED if layout is None else layout)
    r.forward()
    out = r.outputs()
    r.close()
    return out


def _check(case, out, name):
    b = case.batch
    recs = [k for k in range(b.B) if int(b.q_offsets[k + 1]) > int(b.q_offsets[k])]
    ref = oracle_outputs(case, records=recs)
    compare(name, select(b, recs, *out), ref, local_offsets(b, recs))
    return ref


@pytest.mark.parametrize("cfg", [0, 1])
def test_decoder_variant_parity(torch_gpu, cfg):
    """Workload 0 (one 160-row record: the field K/V GEMM runs split) and
    workload 1 at full size."""
    spec = _variant(synth.config_spec(cfg))
    case = synth.make_case(spec)
    b = case.batch
    say(f"case decoder-layer fields, workload {cfg}: B={b.B} T={int(b.lengths.sum())} NQ={b.NQ}")
    out = _run(case)
    _check(case, out, f"decoder fields w{cfg}")
    extra = ("xln", "xq", "xk", "xv", "xo")
    plain = _run(dataclasses.replace(
        case, spec=dataclasses.replace(case.spec, head=dataclasses.replace(case.head, field_cross_attention=0)),
        weights={k: v for k, v in case.weights.items() if not any(f".{m}." in k for m in extra)}))
    assert np.abs(out[0] - plain[0]).max() > 1e-3   # the cross-attention is live


def test_decoder_variant_ragged_varlen_and_streamed(torch_gpu):
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    from test_gpu_stream import _stream
    spec = _variant(synth.config_spec(1, B=3, L=1100, lengths=("uniform", 600, 1100),
                                      head=synth.HeadConfig(vocab_size=4096)))
    case = synth.make_case(spec)
    say(f"case decoder-layer fields, ragged: lengths={case.batch.lengths.tolist()}")
    op = _run(case)
    r = HeadRunner(case)
    r.set_batch(None, C.CLEF_VARLEN)
    r.forward()
    ov = r.outputs()
    for a, c in zip(op, ov):
        assert np.array_equal(a, c)
    os_ = _stream(torch_gpu, r, 64)
    r.close()
    for a, c in zip(op, os_):
        assert np.array_equal(a, c)
    _check(case, op, "decoder fields ragged")


def test_decoder_variant_without_routing_layers_fp16(torch_gpu):
    """routing_layers = 0: the memory rows are still computed for the fields'
    cross-attention; with fp16 hidden rows."""
    spec = _variant(synth.config_spec(1, B=2, L=900, lengths=("uniform", 500, 900), routing_layers=0,
                                      vocab_size=4096, hidden_dtype="f16"))
    case = synth.make_case(spec)
    assert case.head.routing_layers == 0 and case.head.field_cross_attention == 1
    say(f"case decoder-layer fields, no routing layers, fp16: lengths={case.batch.lengths.tolist()}")
    _check(case, _run(case), "decoder fields, no routing, fp16")
