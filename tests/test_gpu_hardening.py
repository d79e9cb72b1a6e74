"""Hardening checks through the C ABI on the GPU:

* the span tables the kernels read, copied back from the device, equal bit
  for bit the tables derived here from the batch (CoreML conversion metadata
  page, decision.spans: half-open spans over each record's own positions);
* working memory poisoned with NaN patterns at allocation changes no output
  bit (no kernel reads memory it did not write first);
* a capped allocation fails with CLEF_E_NOMEM before anything runs and
  leaves the outputs untouched, and the handle works again once uncapped;
* hidden rows with large per-row offsets and outlier channels (the kind a
  backbone's final norm hands over) stay within the parity tolerances, in the
  bf16 mode, whose memory projection folds the LayerNorm into the product,
  and in the fp32 mode;
* one handle driven on two streams back to back: the second forward waits
  for the first (they share the workspace)."""
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


def mini4():
    return synth.config_spec(4, B=6, lengths=("loguniform", 300, 1500),
                             head=synth.HeadConfig(hidden_size=5120, vocab_size=4096))


def expected_tables(b, varlen):
    """Pooling entries, lexical entries and id table as the kernels must see them."""
    cu = np.concatenate([[0], np.cumsum(b.lengths)])
    act = [r for r in range(b.B) if b.q_offsets[r + 1] > b.q_offsets[r]]
    kvb, base = {}, 0
    for r in act:
        kvb[r] = base
        base += -(-int(b.lengths[r]) // 256) * 256
    src = {r: int(cu[r]) if varlen else r * b.L for r in act}
    qs, os_, gl, lex = [], [], [], []
    idoff = 0
    for a, r in enumerate(act):
        for q in range(b.q_offsets[r], b.q_offsets[r + 1]):
            s, e = b.q_span[q]
            qs.append((src[r] + s, e - s, kvb[r] + s, q))
            for k in range(b.o_offsets[q], b.o_offsets[q + 1]):
                s2, e2 = b.o_span[k]
                os_.append((src[r] + s2, e2 - s2, kvb[r] + s2, b.NQ + k))
                lex.append((idoff, e2 - s2, q, b.NQ + b.NO + a))
                idoff += e2 - s2
        n = int(b.lengths[r])
        gl.append((src[r] + n - 1, 1, kvb[r] + n - 1, b.NQ + b.NO + a))
    return (np.array(qs + os_ + gl, np.int32), np.array(lex, np.int32), np.asarray(b.o_ids, np.int32), len(act))


@pytest.mark.parametrize("layout", ["padded", "varlen"])
def test_uploaded_span_tables_bit_exact(torch_gpu, layout):
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    case = synth.make_case(mini4())
    b = case.batch
    r = HeadRunner(case)
    r.set_trace(True)
    r.set_batch(None, C.CLEF_VARLEN if layout == "varlen" else C.CLEF_PADDED)
    r.forward()
    pool, lex, ids, nact = expected_tables(b, layout == "varlen")
    say(f"case span tables ({layout}): {len(pool)} pooling entries, {len(lex)} options, {len(ids)} ids")
    got_pool = r.trace(C.CLEF_TRACE_POOL_TABLE, (b.NQ + b.NO + nact, 4), np.int32)
    got_lex = r.trace(C.CLEF_TRACE_LEX_TABLE, (b.NO, 4), np.int32)
    got_ids = r.trace(C.CLEF_TRACE_IDS, (len(ids),), np.int32)
    r.close()
    assert np.array_equal(got_pool, pool)
    assert np.array_equal(got_lex, lex)
    assert np.array_equal(got_ids, ids)


def _fresh_outputs(case, layout, noalloc=False, streamed=False):
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    r = HeadRunner(case)
    r.set_batch(None, layout)
    if streamed:
        b = case.batch
        cu = b.cu_seqlens()
        H = case.head.hidden_size
        C.clef_head_stream_begin(r.handle, r.args)
        for k in range(b.B):
            for p0 in range(0, int(b.lengths[k]), 64):
                n = int(min(64, b.lengths[k] - p0))
                C.clef_head_stream_rows(r.handle, k, p0, n, r.hidden.data_ptr() + (int(cu[k]) + p0) * H * 2)
        C.clef_head_stream_end(r.handle, r.args, r.logits.data_ptr(), r.probs.data_ptr(), r.argmax.data_ptr())
    elif noalloc:
        r.forward_noalloc()
    else:
        r.forward()
    out = r.outputs()
    r.close()
    return out


def test_poisoned_working_memory_changes_nothing(torch_gpu):
    from structured_decision_head_amd import clefhead as C
    mini = synth.config_spec(1, B=3, L=1100, lengths=("uniform", 600, 1100), head=synth.HeadConfig(vocab_size=4096))
    cases = {
        "mini padded": (synth.make_case(mini), C.CLEF_PADDED, {}),
        "mini varlen": (synth.make_case(mini), C.CLEF_VARLEN, {}),
        "mini streamed": (synth.make_case(mini), C.CLEF_VARLEN, {"streamed": True}),
        "mini no-alloc": (synth.make_case(mini), C.CLEF_PADDED, {"noalloc": True}),
        "decoder fields": (synth.make_case(dataclasses.replace(
            mini, head=dataclasses.replace(mini.head, field_cross_attention=1))), C.CLEF_PADDED, {}),
        "fp32 mode": (synth.make_case(dataclasses.replace(
            mini, head=dataclasses.replace(mini.head, precision=1))), C.CLEF_PADDED, {}),
        # 25 row tiles: the fp32 products run as whole-K GEMMs over three-term rows
        "fp32 mode, whole-K GEMMs": (synth.make_case(dataclasses.replace(
            mini, B=5, lengths=("uniform", 1030, 1100), head=dataclasses.replace(mini.head, precision=1))),
            C.CLEF_PADDED, {}),
        "single record": (synth.config_case(0), C.CLEF_PADDED, {}),
        "H=5120 NaN padding": (synth.make_case(mini4()), C.CLEF_PADDED, {}),
    }
    try:
        for name, (case, layout, kw) in cases.items():
            C.clef_head_debug_set(C.CLEF_DEBUG_POISON, 0)
            clean = _fresh_outputs(case, layout, **kw)
            C.clef_head_debug_set(C.CLEF_DEBUG_POISON, 1)
            poisoned = _fresh_outputs(case, layout, **kw)
            say(f"case poisoned working memory: {name}")
            for a, c in zip(clean, poisoned):
                assert np.array_equal(a, c), name
            assert np.isfinite(poisoned[0]).all() and np.isfinite(poisoned[1]).all()
    finally:
        C.clef_head_debug_set(C.CLEF_DEBUG_POISON, 0)


def test_allocation_failure_gives_nomem(torch_gpu):
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    case = synth.make_case(synth.config_spec(1, B=3, L=1100, lengths=("uniform", 600, 1100),
                                             head=synth.HeadConfig(vocab_size=4096)))
    try:
        C.clef_head_debug_set(C.CLEF_DEBUG_ALLOC_LIMIT, 1 << 20)
        with pytest.raises(C.ClefError) as e:
            HeadRunner(case)
        assert e.value.code == C.CLEF_E_NOMEM
        say("case capped allocation: create refused with CLEF_E_NOMEM")
        C.clef_head_debug_set(C.CLEF_DEBUG_ALLOC_LIMIT, 0)
        r = HeadRunner(case)
        r.set_batch()
        r.logits.fill_(5.0)
        C.clef_head_debug_set(C.CLEF_DEBUG_ALLOC_LIMIT, 1 << 20)
        with pytest.raises(C.ClefError) as e:
            r.forward()
        assert e.value.code == C.CLEF_E_NOMEM and "workspace" in str(e.value)
        torch_gpu.cuda.synchronize()
        assert bool((r.logits == 5.0).all())
        say("case capped allocation: forward refused with CLEF_E_NOMEM, outputs untouched")
        C.clef_head_debug_set(C.CLEF_DEBUG_ALLOC_LIMIT, 0)
        r.forward()
        compare("after the cap is lifted", r.outputs(), oracle_outputs(case), case.batch.o_offsets)
        r.close()
    finally:
        C.clef_head_debug_set(C.CLEF_DEBUG_ALLOC_LIMIT, 0)


def _offset_outlier_case(precision):
    """Hidden rows x = offset_row + scale_row * z with offsets up to +-8, scales
    0.5..4 and four channels carrying values near +-200 (bf16-rounded).  25 row
    tiles, so that the memory projection runs whole-K with the LayerNorm folded
    into its epilogue (in the fp32 mode over the raw bf16 rows against the
    three-term fp32 weight), where the offsets cancel."""
    spec = synth.config_spec(1, B=5, L=1100, lengths=("uniform", 1030, 1100), seed=4242,
                             head=synth.HeadConfig(vocab_size=4096, precision=precision))
    case = synth.make_case(spec)
    b = case.batch
    rng = np.random.default_rng(99)
    z = synth.bf16_bits_to_f32(b.hidden).astype(np.float32)
    off = rng.uniform(-8, 8, (b.B, b.L, 1)).astype(np.float32)
    scl = rng.uniform(0.5, 4, (b.B, b.L, 1)).astype(np.float32)
    x = off + scl * z
    for ch in (7, 1234, 2900, 4001):
        x[:, :, ch] = rng.choice([-1.0, 1.0], (b.B, b.L)) * rng.uniform(150, 250, (b.B, b.L))
    bits = synth.f32_to_bf16_bits(x)
    return dataclasses.replace(case, batch=dataclasses.replace(b, hidden=bits))


@pytest.mark.parametrize("precision", [0, 1])
def test_offset_and_outlier_rows(torch_gpu, precision):
    from structured_decision_head_amd.runner import HeadRunner
    case = _offset_outlier_case(precision)
    say(f"case offset/outlier hidden rows, precision {'fp32' if precision else 'bf16'}")
    r = HeadRunner(case)
    r.set_batch()
    r.forward()
    out = r.outputs()
    r.close()
    kw = {} if precision == 0 else {"tol_logit": 1e-4, "tol_prob": 5e-5}
    compare("offset/outlier rows", out, oracle_outputs(case), case.batch.o_offsets, **kw)


def test_one_handle_two_streams_back_to_back(torch_gpu):
    """Two forwards of one handle issued on two streams with no host wait
    between them (different batches, different output buffers): the second
    waits for the first, and both match their own single runs."""
    from structured_decision_head_amd import clefhead as C
    from structured_decision_head_amd.runner import HeadRunner
    torch = torch_gpu
    c1 = synth.make_case(synth.config_spec(1, B=3, L=1100, lengths=("uniform", 600, 1100),
                                           head=synth.HeadConfig(vocab_size=4096)))
    other = synth.make_case(dataclasses.replace(synth.config_spec(1, B=2, L=900, lengths=("uniform", 500, 900),
                                                                  head=synth.HeadConfig(vocab_size=4096)), seed=555))
    c2 = dataclasses.replace(c1, batch=other.batch)   # the same head and table, another batch
    r = HeadRunner(c1)
    r.set_batch()
    r.forward()
    ref1 = r.outputs()
    a1 = r.args
    h1 = r.hidden
    r2 = HeadRunner(c2, table=r.table)
    r2.set_batch()
    r2.forward()
    ref2 = r2.outputs()
    r2.close()
    # second batch through the first handle, on another stream, right after the first batch
    a2 = C.BatchArgs(c2.batch, r2.hidden.data_ptr())
    outs = [torch.empty(max(c2.batch.NO, 1), dtype=torch.float32, device="cuda"),
            torch.empty(max(c2.batch.NO, 1), dtype=torch.float32, device="cuda"),
            torch.empty(max(c2.batch.NQ, 1), dtype=torch.int32, device="cuda")]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        C.clef_head_forward(r.handle, a1, r.logits.data_ptr(), r.probs.data_ptr(), r.argmax.data_ptr(),
                            s1.cuda_stream)
        C.clef_head_forward(r.handle, a2, *[t.data_ptr() for t in outs], s2.cuda_stream)
    torch.cuda.synchronize()
    got1 = r.outputs()
    got2 = (outs[0][:c2.batch.NO].cpu().numpy().astype(np.float64), outs[1][:c2.batch.NO].cpu().numpy().astype(
        np.float64), outs[2][:c2.batch.NQ].cpu().numpy().astype(np.int64))
    r.close()
    del h1
    for a, c in zip(got1, ref1):
        assert np.array_equal(a, c)
    for a, c in zip(got2, ref2):
        assert np.array_equal(a, c)
    say("case one handle, two streams: both batches bit-identical to their single runs")
