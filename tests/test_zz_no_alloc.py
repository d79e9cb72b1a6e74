"""The allocation-free entry point (clef_head_forward_noalloc) against
clef_head_forward, through the C ABI: two calls in a row, the second with a
smaller batch, each bit-identical to the allocating entry point's outputs on
the same batch (same kernels, same plan) and within the parity tolerances of
the fp64 oracle; a batch larger than the static scratch is refused before
anything runs."""
import numpy as np
import pytest

from parity import compare, oracle_outputs, say
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


def _both(torch, case, r):
    """Outputs of clef_head_forward, then of clef_head_forward_noalloc, on the runner's batch."""
    r.forward()
    ref = r.outputs()
    for t in (r.logits, r.probs):
        t.fill_(float("nan"))
    r.argmax.fill_(-1)
    r.forward_noalloc()
    return ref, r.outputs()


def test_noalloc_two_calls_match_forward(torch_gpu):
    from structured_decision_head_amd.runner import HeadRunner
    big = synth.make_case(synth.config_spec(1, B=3, L=1100, lengths=("uniform", 600, 1100),
                                            head=synth.HeadConfig(vocab_size=4096)))
    say(f"case noalloc call 1: B={big.batch.B} T={int(big.batch.lengths.sum())} NO={big.batch.NO}")
    r = HeadRunner(big)
    r.set_batch()
    ref, got = _both(torch_gpu, big, r)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    compare("noalloc call 1", got, oracle_outputs(big), big.batch.o_offsets)
    r.close()

    small = synth.config_case(0)
    say(f"case noalloc call 2 (smaller): B=1 T={int(small.batch.lengths.sum())} NO={small.batch.NO}")
    r2 = HeadRunner(small)
    r2.set_batch()
    ref2, got2 = _both(torch_gpu, small, r2)
    for a, b in zip(ref2, got2):
        assert np.array_equal(a, b)
    compare("noalloc call 2", got2, oracle_outputs(small), small.batch.o_offsets)
    r2.close()


def test_noalloc_fp32_mode_two_calls_match_forward(torch_gpu):
    """The same in the fp32 precision mode: a batch of 25 row tiles (whole-K
    memory and K/V products, the fp32 K/V planes in the static scratch), then
    the single record (split-K products)."""
    import dataclasses
    from structured_decision_head_amd.runner import HeadRunner
    tol = {"tol_logit": 1e-4, "tol_prob": 5e-5}
    head = synth.HeadConfig(vocab_size=4096, precision=1)
    big = synth.make_case(synth.config_spec(1, B=5, L=1100, lengths=("uniform", 1030, 1100), head=head))
    say(f"case noalloc fp32 call 1: B={big.batch.B} T={int(big.batch.lengths.sum())} NO={big.batch.NO}")
    r = HeadRunner(big)
    r.set_batch()
    ref, got = _both(torch_gpu, big, r)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    compare("noalloc fp32 call 1", got, oracle_outputs(big), big.batch.o_offsets, **tol)
    r.close()

    spec0 = synth.config_spec(0)
    small = synth.make_case(dataclasses.replace(spec0, head=dataclasses.replace(spec0.head, precision=1)))
    say(f"case noalloc fp32 call 2 (smaller): B=1 T={int(small.batch.lengths.sum())} NO={small.batch.NO}")
    r2 = HeadRunner(small)
    r2.set_batch()
    ref2, got2 = _both(torch_gpu, small, r2)
    for a, b in zip(ref2, got2):
        assert np.array_equal(a, b)
    compare("noalloc fp32 call 2", got2, oracle_outputs(small), small.batch.o_offsets, **tol)
    r2.close()


def test_noalloc_refuses_a_batch_beyond_the_scratch(torch_gpu):
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    # two records of 16384 rows: memory and K/V rows alone need over 256 MiB
    spec = synth.config_spec(2, B=2, L=16384, lengths=("uniform", 16384, 16384),
                             head=synth.HeadConfig(vocab_size=1024))
    case = synth.make_case(spec)
    say("case noalloc oversize: B=2, L=16384")
    r = HeadRunner(case)
    r.set_batch()
    r.logits.fill_(7.0)
    with pytest.raises(C.ClefError) as e:
        r.forward_noalloc()
    assert e.value.code == C.CLEF_E_UNSUPPORTED and "allocation-free" in str(e.value)
    torch_gpu.cuda.synchronize()
    assert bool((r.logits == 7.0).all())
    r.close()
