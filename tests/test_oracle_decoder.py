"""Pins of the decoder-layer reading of the field stack (field layers that
also cross-attend over the record's memory rows: the clef-4bit page §三 step
3 and the architecture page §3.2 call them transformer decoder layers).

The layer is pinned to torch.nn.TransformerDecoderLayer(norm_first=True)
with extra masked memory rows, and the whole head with the variant to the
pure-Python scalar evaluator.  Invariants: the variant changes the outputs
(the cross-attention is live), padding and batch composition still do not."""
import dataclasses
import math

import numpy as np
import torch

from conftest import table_reader, tiny_spec
from oracle import head as O
from structured_decision_head_amd import synth
from test_oracle_pins import _attn_params, _brute, _rng


def test_decoder_field_layer_matches_torch_decoder_layer():
    D, F, heads, eps = 64, 128, 4, 1e-5
    r = _rng(77)
    p = _attn_params(r, D, F, "field.0")
    for m in ("xq", "xk", "xv", "xo"):
        p[f"field.0.{m}.w"] = r.standard_normal((D, D)) / math.sqrt(D)
        p[f"field.0.{m}.b"] = r.standard_normal(D) / math.sqrt(D)
    p["field.0.xln.w"] = 1 + 0.1 * r.standard_normal(D)
    p["field.0.xln.b"] = 0.1 * r.standard_normal(D)
    f = r.standard_normal((5, D)) * 2
    mem = r.standard_normal((13, D))
    got = O.field_layer(f, p, "field.0", heads, eps, memory=mem)
    layer = torch.nn.TransformerDecoderLayer(D, heads, F, dropout=0.0, activation="gelu", layer_norm_eps=eps,
                                             batch_first=True, norm_first=True).double()
    layer.train()   # dropout is 0; keeps the plain (non fused) path
    with torch.no_grad():
        for att, names in ((layer.self_attn, "qkvo"), (layer.multihead_attn, ("xq", "xk", "xv", "xo"))):
            att.in_proj_weight.copy_(torch.tensor(np.concatenate([p[f"field.0.{x}.w"] for x in names[:3]])))
            att.in_proj_bias.copy_(torch.tensor(np.concatenate([p[f"field.0.{x}.b"] for x in names[:3]])))
            att.out_proj.weight.copy_(torch.tensor(p[f"field.0.{names[3]}.w"]))
            att.out_proj.bias.copy_(torch.tensor(p[f"field.0.{names[3]}.b"]))
        layer.linear1.weight.copy_(torch.tensor(p["field.0.ffn1.w"]))
        layer.linear1.bias.copy_(torch.tensor(p["field.0.ffn1.b"]))
        layer.linear2.weight.copy_(torch.tensor(p["field.0.ffn2.w"]))
        layer.linear2.bias.copy_(torch.tensor(p["field.0.ffn2.b"]))
        for i, nm in ((1, "ln1"), (2, "xln"), (3, "ln2")):
            ln = getattr(layer, f"norm{i}")
            ln.weight.copy_(torch.tensor(p[f"field.0.{nm}.w"]))
            ln.bias.copy_(torch.tensor(p[f"field.0.{nm}.b"]))
        # three extra memory rows, masked out
        mem_pad = np.concatenate([mem, 50 * r.standard_normal((3, D))])
        mask = torch.tensor([[False] * 13 + [True] * 3])
        ref = layer(torch.tensor(f)[None], torch.tensor(mem_pad)[None], memory_key_padding_mask=mask)[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def _case(seed, **over):
    spec = tiny_spec(seed=seed, ln_random=True, **over)
    spec = dataclasses.replace(spec, head=dataclasses.replace(spec.head, field_cross_attention=1))
    return synth.make_case(spec)


def test_decoder_head_matches_brute_force():
    case = _case(61)
    lo, po, ao = O.forward(case.weights, case.head, case.batch, table_reader(case))
    lb, pb, ab = _brute(case)
    np.testing.assert_allclose(lo, lb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(po, pb, rtol=1e-12, atol=1e-12)
    assert np.array_equal(ao, ab)


def test_decoder_variant_is_live_and_keeps_the_other_weights():
    case = _case(62)
    plain = dataclasses.replace(case.head, field_cross_attention=0)
    lo1, _, _ = O.forward(case.weights, case.head, case.batch, table_reader(case))
    lo0, _, _ = O.forward(case.weights, plain, case.batch, table_reader(case))
    assert np.abs(lo1 - lo0).max() > 1e-3
    # the variant's tensors come after all others, which keep their values
    base = synth.make_case(dataclasses.replace(case.spec, head=plain)).weights
    assert set(case.weights) - set(base) == {f"field.{l}.{m}.{x}" for l in range(plain.layers)
                                              for m in ("xln", "xq", "xk", "xv", "xo") for x in "wb"}
    for k, v in base.items():
        assert np.array_equal(case.weights[k], v), k


def test_decoder_padding_and_batch_composition():
    case = _case(63)
    b = case.batch
    lo, po, ao = O.forward(case.weights, case.head, b, table_reader(case))
    hid = b.hidden.copy()
    for r in range(b.B):
        hid[r, b.lengths[r]:] = np.uint16(0x7FC0)
    lp, pp, ap = O.forward(case.weights, case.head, dataclasses.replace(b, hidden=hid), table_reader(case))
    assert np.array_equal(lo, lp) and np.array_equal(po, pp)
    off = 0
    for r in range(b.B):
        sub = b.record(r)
        l1, p1, a1 = O.forward(case.weights, case.head, sub, table_reader(case))
        assert np.array_equal(l1, lo[off:off + len(l1)])
        off += len(l1)
