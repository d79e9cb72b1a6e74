"""Input generator: determinism, layout validity, and agreement with the facts
the pages fix (tests/golden/page_facts.json)."""
import json
import os

import numpy as np

from structured_decision_head_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_page_constants():
    assert (synth.NOUL, synth.CHOICE, synth.SCORE) == tuple(GOLD["question_types"][k] for k in ("noul", "choice", "score"))
    assert synth.PREFIX_TOKENS == GOLD["prefix_tokens"] and synth.SUFFIX_TOKENS == GOLD["suffix_tokens"]
    h = synth.HeadConfig()
    for k, v in GOLD["head"].items():
        assert getattr(h, k) == v
    assert h.vocab_size == GOLD["vocab_size"]
    assert synth.config_spec(4).head.hidden_size == GOLD["hidden_size_27b"]


def test_bf16_round_trip_and_rne():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38, 1e-40], np.float32)
    b = synth.f32_to_bf16_bits(x)
    y = synth.bf16_bits_to_f32(b)
    assert y[0] == 1.0 and y[1] == 1.0           # tie to even
    assert y[2] == 1.015625                        # tie rounds up to even
    assert y[3] == -2.5


def _check_layout(b: synth.Batch, spec):
    assert b.q_offsets[0] == 0 and b.q_offsets[-1] == b.NQ
    assert b.o_offsets[0] == 0 and b.o_offsets[-1] == b.NO
    assert len(b.o_ids) == int((b.o_span[:, 1] - b.o_span[:, 0]).sum())
    assert (b.o_ids >= 0).all() and (b.o_ids < spec.head.vocab_size).all()
    for r in range(b.B):
        n = int(b.lengths[r])
        spans = []
        for q in range(b.q_offsets[r], b.q_offsets[r + 1]):
            spans.append(tuple(b.q_span[q]))
            nopt = b.o_offsets[q + 1] - b.o_offsets[q]
            t = b.q_type[q]
            if t == synth.NOUL:
                assert nopt == 2
            if t == synth.SCORE:
                assert nopt == spec.score_levels
            for k in range(b.o_offsets[q], b.o_offsets[q + 1]):
                spans.append(tuple(b.o_span[k]))
        spans.sort()
        for s, e in spans:
            assert spec.prefix <= s < e <= n - spec.suffix
        for (s0, e0), (s1, e1) in zip(spans, spans[1:]):
            assert e0 <= s1                        # disjoint


def test_configs_layout_and_determinism():
    for i, over in [(0, {}), (1, dict(B=3, L=None, lengths=("uniform", 400, 900), head=synth.HeadConfig(vocab_size=512))),
                    (3, dict(B=1, L=None, lengths=("fixed", 6000, 6000), head=synth.HeadConfig(vocab_size=512))),
                    (4, dict(B=4, lengths=("loguniform", 512, 2048), head=synth.HeadConfig(hidden_size=5120, vocab_size=512)))]:
        spec = synth.config_spec(i, **over)
        b1 = synth.make_batch(spec)
        b2 = synth.make_batch(spec)
        _check_layout(b1, spec)
        for f in ("hidden", "lengths", "q_offsets", "q_type", "q_span", "o_offsets", "o_span", "o_ids"):
            assert np.array_equal(getattr(b1, f), getattr(b2, f), equal_nan=False) or f == "hidden"
        assert b1.hidden.tobytes() == b2.hidden.tobytes()


def test_config0_explicit_layout():
    b = synth.make_batch(synth.config_spec(0))
    assert b.B == 1 and b.L == 160 and int(b.lengths[0]) == 160
    assert list(b.q_type) == [synth.NOUL, synth.CHOICE]
    assert tuple(b.q_span[0]) == (97, 107) and tuple(b.q_span[1]) == (114, 124)
    assert tuple(b.o_span[0]) == (107, 110) and tuple(b.o_span[1]) == (110, 113)
    assert b.o_span[2, 0] == 124 and b.o_span[4, 1] <= 150
    for k in (2, 3, 4):
        assert 4 <= b.o_span[k, 1] - b.o_span[k, 0] <= 8


def test_config4_nan_padding_and_varlen():
    spec = synth.config_spec(4, B=5, lengths=("loguniform", 512, 2048), head=synth.HeadConfig(hidden_size=5120, vocab_size=512))
    b = synth.make_batch(spec)
    for r in range(b.B):
        n = int(b.lengths[r])
        assert not np.isnan(synth.bf16_bits_to_f32(b.hidden[r, :n])).any()
        assert np.isnan(synth.bf16_bits_to_f32(b.hidden[r, n:])).all()
    v = b.varlen_hidden()
    cu = b.cu_seqlens()
    assert v.shape[0] == cu[-1]
    for r in range(b.B):
        assert np.array_equal(v[cu[r]: cu[r + 1]], b.hidden[r, : b.lengths[r]])


def test_weights_shapes_and_init():
    c = synth.HeadConfig(hidden_size=256, width=64, heads=4, feedforward=128, vocab_size=100)
    w = synth.make_weights(c, 3)
    specs = synth.weight_specs(c)
    assert list(w) == [s[0] for s in specs]
    for name, shape, kind, fan in specs:
        assert w[name].shape == shape
        if kind == "lin" and np.prod(shape) > 1000:
            x = synth.bf16_bits_to_f32(w[name]).astype(np.float64)
            assert abs(x.std() * np.sqrt(fan) - 1) < 0.1
    assert w["gate_logit"].dtype == np.float32 and w["gate_logit"][0] == 0.0
    assert w["joint_scale"][0] == 1.0


def test_top2_margin_helper():
    """The test helper that logs each question's top-2 logit gap, against a
    partition-based form."""
    from parity import top2_margin
    rng = np.random.default_rng(5)
    offs = np.array([0, 1, 4, 9, 11])
    x = rng.standard_normal(11)
    got = top2_margin(x, offs)
    assert np.isinf(got[0])
    for i in range(1, 4):
        seg = x[offs[i]: offs[i + 1]]
        part = np.partition(seg, len(seg) - 2)
        assert got[i] == part[-1] - part[-2]
    x[5] = x[6] = x[4:9].max() + 1.0
    assert top2_margin(x, offs)[2] == 0.0
