"""GPU parity of the fp32 precision mode (CLEF_PRECISION_F32): the head in
fp32 arithmetic, as the CoreML packaging of clef-flash runs it on fp16 hidden
states (CoreML conversion metadata page, decision.head, dtype_of_record).

Tolerance (derived from the arithmetic).  Every product of the mode is exact
(bf16 weights times activations split into three bf16 terms) or fp32 (the
attention's products) and only fp32 accumulation rounds, unit roundoff
u = 2^-24.  A length-K accumulation of O(1) terms then errs by about
sqrt(K) u relative (K <= 8192: <= 5.4e-6); a logit passes through about 26
dependent accumulations (option query, 2 routing layers of 4 products, 4
field layers of 4 products, the scoring layer), so its error stays below
26 x 5.4e-6 = 1.4e-4 even when those errors add up, and far below when they
are independent.  Hence max |d logit| <= 1e-4 against the fp64 oracle (at
logits of size O(1)) and, since a softmax probability moves by at most half
the largest logit change, max |d prob| <= 5e-5: 200 and 40 times tighter
than the bf16 mode's 2e-2 and 2e-3.  A float32 evaluation of the oracle's
own steps lands at |d logit| ~ 2e-6 on these inputs.  Argmax must equal the
oracle's."""
import dataclasses

import numpy as np
import pytest

from oracle import head as O
from parity import compare, local_offsets, oracle_outputs, say, select
from structured_decision_head_amd import synth

pytestmark = pytest.mark.gpu

TOL32_LOGIT = 1e-4
TOL32_PROB = 5e-5


@pytest.fixture(scope="module")
def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from structured_decision_head_amd import clefhead
    clefhead.load()
    return torch


def f32(spec):
    return dataclasses.replace(spec, head=dataclasses.replace(spec.head, precision=1))


def _run(case, layout=None, trace=False):
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    r = HeadRunner(case)
    r.set_trace(trace)
    r.set_batch(None, C.CLEF_PADDED if layout is None else layout)
    r.forward()
    return r, r.outputs()


def _check(case, out, name, recs=None):
    b = case.batch
    recs = [r for r in range(b.B) if int(b.q_offsets[r + 1]) > int(b.q_offsets[r])] if recs is None else recs
    ref = oracle_outputs(case, records=recs)
    compare(f"{name} ({len(recs)} records)", select(b, recs, *out), ref, local_offsets(b, recs),
            tol_logit=TOL32_LOGIT, tol_prob=TOL32_PROB)
    return ref


@pytest.mark.parametrize("hidden", ["f16", "bf16"])
def test_f32_single_record_stages(torch_gpu, hidden):
    """Every traced intermediate of the single record against the oracle's."""
    from structured_decision_head_amd import clefhead as C
    case = synth.make_case(f32(dataclasses.replace(synth.config_spec(0), hidden_dtype=hidden)))
    say(f"case single record, fp32 mode, {hidden} hidden")
    r, out = _run(case, trace=True)
    b = case.batch
    p = O.load_params(case.weights)
    tr = {}
    ido = b.o_id_offsets()
    n = int(b.lengths[0])
    O.forward_record(p, case.head, O.hidden_rows(b, 0, n), b.q_type, b.q_span, b.o_offsets, b.o_span,
                     [O.from_bf16(case.table[b.o_ids[ido[k]: ido[k + 1]]]) for k in range(b.NO)], trace=tr)
    H, D = case.head.hidden_size, case.head.width

    def rel(a, ref):
        return float(np.abs(a - ref).max() / max(np.abs(ref).max(), 1e-30))

    stages = {"memory": rel(r.trace(C.CLEF_TRACE_MEMORY, (256, D))[:n], tr["memory"])}
    for i in range(case.head.routing_layers + 1):
        stages[f"u{i}"] = rel(r.trace(C.CLEF_TRACE_U + i, (b.NO, D)), tr["u_layers"][i])
    stages["f0"] = rel(r.trace(C.CLEF_TRACE_F0, (b.NQ, D)), tr["f0"])
    stages["f"] = rel(r.trace(C.CLEF_TRACE_F, (b.NQ, D)), tr["f"])
    stages["jcos"] = rel(r.trace(C.CLEF_TRACE_JCOS, (b.NO,)), tr["joint_cos"])
    stages["mlp"] = rel(r.trace(C.CLEF_TRACE_MLP, (b.NO,)), tr["mlp"])
    say("  stage max relative error: " + ", ".join(f"{k}={v:.2e}" for k, v in stages.items()))
    for k, v in stages.items():
        assert v < 2e-5, (k, v)   # bf16 mode: memory rows alone carry ~4e-3
    r.close()
    compare("single record fp32", out, oracle_outputs(case), b.o_offsets, tol_logit=TOL32_LOGIT, tol_prob=TOL32_PROB)


def test_f32_online_serving_full_size_f16_hidden(torch_gpu):
    """The online-serving batch (B=8, L=4096) at full size, fp16 hidden rows."""
    case = synth.make_case(f32(dataclasses.replace(synth.config_spec(1), hidden_dtype="f16")))
    b = case.batch
    say(f"case online-serving full size, fp32 mode, fp16 hidden: B={b.B} T={int(b.lengths.sum())} NO={b.NO}")
    r, out = _run(case)
    r.close()
    _check(case, out, "online-serving fp32")


def test_f32_h5120_padded_vs_varlen_nan_padding(torch_gpu):
    """H=5120 with NaN padding rows: the normalised-row loader never reads
    them; padded and varlen runs agree bit for bit."""
    from structured_decision_head_amd import clefhead as C
    spec = f32(synth.config_spec(4, B=5, lengths=("loguniform", 300, 2500), hidden_dtype="f16", vocab_size=4096))
    case = synth.make_case(spec)
    b = case.batch
    say(f"case H=5120 fp32 mode, NaN padding: B={b.B} L={b.L} lengths={b.lengths.tolist()}")
    r, op = _run(case, C.CLEF_PADDED)
    r.set_batch(None, C.CLEF_VARLEN)
    r.forward()
    ov = r.outputs()
    r.close()
    for a, c in zip(op, ov):
        assert np.array_equal(a, c)
    _check(case, op, "H=5120 fp32")


def test_f32_decoder_fields_and_gate_closed(torch_gpu):
    """The decoder-layer field variant in fp32 mode on a ragged batch; and the
    gate closed, where the logits are the prior."""
    import math
    spec = f32(synth.config_spec(1, B=3, L=1100, lengths=("uniform", 600, 1100),
                                 head=synth.HeadConfig(vocab_size=4096, field_cross_attention=1)))
    case = synth.make_case(spec)
    say("case mini ragged, decoder-layer fields, fp32 mode")
    r, out = _run(case)
    r.close()
    _check(case, out, "decoder fp32")
    case = synth.make_case(dataclasses.replace(spec, gate_logit=-math.inf,
                                               head=dataclasses.replace(spec.head, field_cross_attention=0)))
    say("case mini ragged, gate closed, fp32 mode")
    r, out = _run(case)
    r.close()
    _check(case, out, "gate closed fp32")


def test_f32_big_gemm_path_memory_rows_and_decoder(torch_gpu):
    """A batch of more than 16 row tiles, where the memory and K/V products run
    as whole-K bf16 GEMMs over the three bf16 terms of each fp32 activation
    (the single-record and small-batch tests above take the split-K path):
    one record's memory rows against the oracle's, then every output, with
    the decoder-layer field variant so that the field K/V product runs too."""
    from structured_decision_head_amd import clefhead as C
    spec = f32(synth.config_spec(1, B=6, L=3000, lengths=("uniform", 2500, 3000),
                                 head=synth.HeadConfig(vocab_size=4096, field_cross_attention=1)))
    case = synth.make_case(spec)
    b = case.batch
    tiles = sum(-(-int(n) // 256) for n in b.lengths)
    say(f"case fp32 mode, {tiles} row tiles, decoder-layer fields: lengths={b.lengths.tolist()}")
    assert tiles > 16
    r, out = _run(case, trace=True)
    n0 = int(b.lengths[0])
    mem = r.trace(C.CLEF_TRACE_MEMORY, (tiles * 256, case.head.width))[:n0]
    r.close()
    p = O.load_params(case.weights)
    xh = O.layer_norm(O.hidden_rows(b, 0, n0), p["ln_in.w"], p["ln_in.b"], case.head.ln_eps)
    ref = O.linear(xh, p["mem.w"], p["mem.b"])
    rel = float(np.abs(mem - ref).max() / np.abs(ref).max())
    say(f"  memory rows of record 0: max relative error {rel:.2e}")
    assert rel < 2e-5
    _check(case, out, "fp32 big-GEMM path, decoder fields")


def test_f32_refuses_streamed_ingest(torch_gpu):
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    case = synth.make_case(f32(synth.config_spec(0)))
    r = HeadRunner(case)
    r.set_batch(None, C.CLEF_VARLEN)
    with pytest.raises(C.ClefError) as e:
        C.clef_head_stream_begin(r.handle, r.args)
    assert e.value.code == C.CLEF_E_UNSUPPORTED
    r.close()


def test_f32_records_with_more_than_64_fields(torch_gpu):
    """Records of 70 fields in the fp32 mode: two 64-row query blocks per record
    in the field attention, whose W_o share takes three bf16 terms per value."""
    spec = f32(synth.CaseSpec(name="many-fields", seed=7602, head=synth.HeadConfig(hidden_size=4096, vocab_size=4096),
                              B=2, L=None, lengths=("fixed", 1600, 1600), fields="counts", counts=(40, 20, 10),
                              choice_opts=(2, 3), opt_len=(1, 2), instr_len=(2, 4)))
    say("case 2 records of 70 fields, fp32 mode")
    case = synth.make_case(spec)
    assert int(np.diff(case.batch.q_offsets).min()) == 70
    _r, out = _run(case)
    _check(case, out, "70 fields, fp32")


@pytest.mark.parametrize("H", [512, 8192])
def test_f32_smallest_and_largest_hidden_size_big_gemm_path(torch_gpu, H):
    """hidden_size 512 and 8192 in the fp32 mode with 25 row tiles, so that the
    memory product runs whole-K over the raw bf16 rows read three times
    (depth 3 x 512 and 3 x 8192, the row read wrapping at H)."""
    spec = synth.config_spec(1, B=5, L=1100, lengths=("uniform", 1030, 1100), seed=4300 + H // 512,
                             head=synth.HeadConfig(hidden_size=H, vocab_size=4096, precision=1))
    say(f"case fp32 mode, hidden size {H}, 25 row tiles")
    case = synth.make_case(spec)
    _r, out = _run(case)
    _check(case, out, f"fp32 H={H}")
