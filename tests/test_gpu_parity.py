"""GPU parity: the HIP library, called through its C ABI, against the fp64
oracle on the same seeded inputs."""
import math

import numpy as np
import pytest

from parity import compare, local_offsets, oracle_outputs, say, select
from oracle import head as O
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


def _run(case, layout=None, trace=False, batch=None):
    from structured_decision_head_amd.runner import HeadRunner
    from structured_decision_head_amd import clefhead as C
    r = HeadRunner(case)
    r.set_trace(trace)
    r.set_batch(batch, C.CLEF_PADDED if layout is None else layout)
    r.forward()
    return r, r.outputs()


def mini_spec(**over):
    kw = dict(B=3, L=1100, lengths=("uniform", 600, 1100), head=synth.HeadConfig(vocab_size=4096))
    kw.update(over)
    return synth.config_spec(1, **kw)


def test_single_record_parity_and_stages(torch_gpu):
    say("case single record (B=1, L=160, H=4096)")
    case = synth.config_case(0)
    r, out = _run(case, trace=True)
    b = case.batch
    ref = oracle_outputs(case)
    # per-stage parity against the oracle's intermediates
    p = O.load_params(case.weights)
    tr = {}
    ido = b.o_id_offsets()
    n = int(b.lengths[0])
    O.forward_record(p, case.head, O.from_bf16(b.hidden[0, :n]), b.q_type, b.q_span, b.o_offsets, b.o_span,
                     [O.from_bf16(case.table[b.o_ids[ido[k]: ido[k + 1]]]) for k in range(b.NO)], trace=tr)
    from structured_decision_head_amd import clefhead as C
    H, D = case.head.hidden_size, case.head.width
    pooled = r.trace(C.CLEF_TRACE_POOLED, (b.NQ + b.NO + 1, H))

    def rel(a, ref):
        return float(np.abs(a - ref).max() / max(np.abs(ref).max(), 1e-30))

    stages = {
        "qbar": rel(pooled[: b.NQ], tr["qbar"]),
        "cbar": rel(pooled[b.NQ: b.NQ + b.NO], tr["cbar"]),
        "g": rel(pooled[-1], tr["g"]),
        "ebar": rel(r.trace(C.CLEF_TRACE_LEXICAL, (b.NO, H)), tr["ebar"]),
        "prior": rel(r.trace(C.CLEF_TRACE_PRIOR, (b.NO,)), tr["prior"]),
    }
    mem = r.trace(C.CLEF_TRACE_MEMORY, (256, D), np.uint16)[:n]
    stages["memory"] = rel(synth.bf16_bits_to_f32(mem).astype(np.float64), tr["memory"])
    for i in range(case.head.routing_layers + 1):
        stages[f"u{i}"] = rel(r.trace(C.CLEF_TRACE_U + i, (b.NO, D)), tr["u_layers"][i])
    stages["f0"] = rel(r.trace(C.CLEF_TRACE_F0, (b.NQ, D)), tr["f0"])
    stages["f"] = rel(r.trace(C.CLEF_TRACE_F, (b.NQ, D)), tr["f"])
    stages["jcos"] = rel(r.trace(C.CLEF_TRACE_JCOS, (b.NO,)), tr["joint_cos"])
    stages["mlp"] = rel(r.trace(C.CLEF_TRACE_MLP, (b.NO,)), tr["mlp"])
    say("  stage max relative error: " + ", ".join(f"{k}={v:.2e}" for k, v in stages.items()))
    for k in ("qbar", "cbar", "g", "ebar", "prior"):
        assert stages[k] < 1e-4, (k, stages[k])
    assert stages["memory"] < 1e-2
    r.close()
    compare(case.spec.name, out, ref, b.o_offsets)


def test_mini_ragged_parity(torch_gpu):
    say("case mini (B=3, L=1100 ragged, H=4096, V=4096)")
    case = synth.make_case(mini_spec())
    r, out = _run(case)
    r.close()
    compare("mini", out, oracle_outputs(case), case.batch.o_offsets)


def test_gate_closed_gives_prior(torch_gpu):
    say("case mini, gate_logit = -inf")
    case = synth.make_case(mini_spec(gate_logit=-math.inf, ln_random=True))
    r, out = _run(case)
    r.close()
    lo, po, ao = oracle_outputs(case)
    lg, pr, am = out
    say(f"  max |logit - prior| = {np.abs(lg - lo).max():.3e}")
    assert np.abs(lg - lo).max() <= 1e-5
    compare("gate-closed", out, (lo, po, ao), case.batch.o_offsets)


def test_ln_random_parity(torch_gpu):
    say("case mini, random LayerNorm affine")
    case = synth.make_case(mini_spec(seed=77, ln_random=True))
    r, out = _run(case)
    r.close()
    compare("mini-ln", out, oracle_outputs(case), case.batch.o_offsets)


def test_padded_vs_varlen_bit_identical_h5120(torch_gpu):
    from structured_decision_head_amd import clefhead as C
    say("case mini4 (H=5120, B=5, log-uniform lengths, NaN padding), padded vs varlen")
    spec = synth.config_spec(4, B=5, lengths=("loguniform", 300, 1500),
                             head=synth.HeadConfig(hidden_size=5120, vocab_size=4096))
    case = synth.make_case(spec)
    r, out_p = _run(case, layout=C.CLEF_PADDED)
    r.set_batch(None, C.CLEF_VARLEN)
    r.forward()
    out_v = r.outputs()
    r.close()
    for a, b in zip(out_p, out_v):
        assert np.array_equal(a, b)
    compare("mini4", out_p, oracle_outputs(case), case.batch.o_offsets)


def test_determinism_and_batch_composition(torch_gpu):
    say("case mini, repeat and record-by-record")
    case = synth.make_case(mini_spec(seed=91))
    from structured_decision_head_amd.runner import HeadRunner
    r = HeadRunner(case)
    r.set_batch()
    r.forward()
    a = r.outputs()
    r.forward()
    b = r.outputs()
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # a record alone: the split-K partition of the small GEMMs depends on the
    # batch's row count, so only fp32 summation order may differ
    ref = oracle_outputs(case)
    for rec in range(case.batch.B):
        sub = case.batch.record(rec)
        r.set_batch(sub)
        r.forward()
        alone = r.outputs()
        l2, p2, a2 = select(case.batch, [rec], *a)
        say(f"  record {rec}: alone vs in batch max|dlogit|={np.abs(alone[0] - l2).max():.2e}")
        assert np.abs(alone[0] - l2).max() < 1e-3 and np.abs(alone[1] - p2).max() < 2e-4
        compare(f"record {rec} alone", alone, select(case.batch, [rec], *ref), sub.o_offsets)
    r.close()
