"""Pins of the oracle's fp16-hidden input (the CoreML packaging of clef-flash
feeds the head fp16 hidden states: CoreML conversion metadata page,
"decision.head", dtype of record).

The head's definition does not change with the input encoding; only the
decoding of the hidden bits does.  So: the decoder matches torch's float16
conversion on every bit pattern, and hidden values that both bf16 and fp16
represent exactly give bit-identical oracle outputs under either encoding.
The generator rounds the same fp32 draws to fp16 that it rounds to bf16."""
import dataclasses

import numpy as np
import torch

from conftest import table_reader, tiny_spec
from oracle import head as O
from structured_decision_head_amd import synth


def test_f16_decode_matches_torch_on_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.from_f16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert np.array_equal(ours[~nan], ref[~nan])


def _bf16_to_f16_bits(bits16: np.ndarray) -> np.ndarray:
    x = O.from_bf16(bits16)
    h = x.astype(np.float16)
    assert np.array_equal(h.astype(np.float64), x), "value not representable in fp16"
    return h.view(np.uint16)


def test_same_values_same_outputs_under_either_encoding():
    case = synth.make_case(tiny_spec(seed=41, ln_random=True))
    b = case.batch
    # keep values fp16 represents exactly: |x| >= 2^-14 (normal range) or 0
    x = O.from_bf16(b.hidden)
    keep = (np.abs(x) >= 2.0 ** -14) | ~np.isfinite(x)
    bits = np.where(keep, b.hidden, np.uint16(0)).astype(np.uint16)
    bf = dataclasses.replace(b, hidden=bits)
    valid = np.zeros(bits.shape[:2], bool)
    for r in range(b.B):
        valid[r, :b.lengths[r]] = True
    f16 = bits.copy()
    f16[valid] = _bf16_to_f16_bits(bits[valid])
    f16[~valid] = np.uint16(0x7E00)
    hb = dataclasses.replace(b, hidden=f16, hidden_dtype="f16")
    lo1, po1, ao1 = O.forward(case.weights, case.head, bf, table_reader(case))
    lo2, po2, ao2 = O.forward(case.weights, case.head, hb, table_reader(case))
    assert np.array_equal(lo1, lo2) and np.array_equal(po1, po2) and np.array_equal(ao1, ao2)


def test_generator_rounds_the_same_draws():
    spec = tiny_spec(seed=43)
    cb = synth.make_case(spec)
    ch = synth.make_case(dataclasses.replace(spec, hidden_dtype="f16"))
    assert ch.batch.hidden_dtype == "f16" and cb.batch.hidden_dtype == "bf16"
    for r in range(cb.batch.B):
        n = int(cb.batch.lengths[r])
        xb = O.from_bf16(cb.batch.hidden[r, :n])
        xh = O.from_f16(ch.batch.hidden[r, :n])
        # both round one fp32 draw: they differ by at most half a bf16 ulp plus half an fp16 ulp
        assert np.all(np.abs(xb - xh) <= np.abs(xh) * (2.0 ** -8 + 2.0 ** -11) + 2.0 ** -24)
        assert not np.array_equal(xb, xh)
    # the span tables do not depend on the encoding
    assert np.array_equal(cb.batch.o_ids, ch.batch.o_ids) and np.array_equal(cb.batch.q_span, ch.batch.q_span)
