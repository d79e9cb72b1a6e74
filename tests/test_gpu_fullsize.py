"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (padded layout, one clef_head_forward over the whole batch;
for the online-serving batch also two heads sharing weights with batches in
flight on two streams, as the benchmark runs them).

Records are independent, so the fp64 oracle checks the batch record by
record (every record with questions).  Config 4 is also run as a varlen batch
and must match the padded run bit for bit."""
import numpy as np
import pytest

from parity import compare, local_offsets, oracle_outputs, say, select
from structured_decision_head_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from structured_decision_head_amd import clefhead
    clefhead.load()
    return torch


def _check(case, out, name):
    b = case.batch
    recs = [r for r in range(b.B) if int(b.q_offsets[r + 1]) > int(b.q_offsets[r])]
    ref = oracle_outputs(case, records=recs)
    got = select(b, recs, *out)
    compare(f"{name} ({len(recs)} records)", got, ref, local_offsets(b, recs))


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_full_size_parity(torch_gpu, cfg):
    from structured_decision_head_amd.runner import HeadRunner
    case = synth.config_case(cfg)
    say(f"case {case.spec.name} full size")
    b = case.batch
    say(f"  B={b.B} L={b.L} T={int(b.lengths.sum())} NQ={b.NQ} NO={b.NO}")
    r = HeadRunner(case)
    r.set_batch()
    r.forward()
    out = r.outputs()
    r.close()
    _check(case, out, case.spec.name)


def test_full_size_h5120_padded_and_varlen(torch_gpu):
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    say("case heterogeneous H=5120 full size (B=32, NaN padding), padded and varlen")
    case = synth.config_case(4)
    b = case.batch
    say(f"  B={b.B} L={b.L} T={int(b.lengths.sum())} NQ={b.NQ} NO={b.NO}")
    r = HeadRunner(case)
    r.set_batch(None, C.CLEF_PADDED)
    r.forward()
    out_p = r.outputs()
    r.set_batch(None, C.CLEF_VARLEN)
    r.forward()
    out_v = r.outputs()
    r.close()
    for a, c in zip(out_p, out_v):
        assert np.array_equal(a, c)
    _check(case, out_p, case.spec.name)


def test_full_size_two_in_flight(torch_gpu):
    """Two heads over one weight blob, forwards alternating on two streams
    (the benchmark's timed loop): every head returns exactly what one head
    returns alone, and two records are checked against the oracle."""
    from structured_decision_head_amd.runner import HeadRunner
    case = synth.config_case(1)
    say(f"case {case.spec.name} full size, two batches in flight")
    r1 = HeadRunner(case)
    r1.set_batch()
    r1.forward()
    ref = r1.outputs()
    r2 = HeadRunner(case, share=r1)
    r2.set_batch()
    streams = [torch_gpu.cuda.Stream(), torch_gpu.cuda.Stream()]
    for i in range(8):
        (r1, r2)[i % 2].forward(streams[i % 2])
    torch_gpu.cuda.synchronize()
    for r in (r1, r2):
        assert all(np.array_equal(a, b) for a, b in zip(r.outputs(), ref))
    b = case.batch
    recs = [0, b.B - 1]
    compare("two in flight (records 0 and last)", select(b, recs, *r2.outputs()),
            oracle_outputs(case, records=recs), local_offsets(b, recs))
    r2.close()
    r1.close()
