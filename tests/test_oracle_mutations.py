"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
check that the brute-force pin notices each one.  Guards against pins that
are too weak to catch a dropped term, a wrong index or a transposed operand."""
import math

import numpy as np
import pytest

from conftest import table_reader, tiny_spec
from oracle import head as O
from structured_decision_head_amd import synth
from test_oracle_pins import _brute

_orig = {k: getattr(O, k) for k in ("layer_norm", "gelu", "cosine", "softmax", "attention", "span_mean",
                                     "linear", "ffn", "sigmoid")}


def _m_attention_scale(q_in, kv_in, p, prefix, heads):
    q = O.linear(q_in, p[prefix + ".q.w"], p[prefix + ".q.b"])
    k = O.linear(kv_in, p[prefix + ".k.w"], p[prefix + ".k.b"])
    v = O.linear(kv_in, p[prefix + ".v.w"], p[prefix + ".v.b"])
    d = q.shape[-1] // heads
    outs = [O.softmax(q[:, j * d:(j + 1) * d] @ k[:, j * d:(j + 1) * d].T / d) @ v[:, j * d:(j + 1) * d]
            for j in range(heads)]
    return O.linear(np.concatenate(outs, 1), p[prefix + ".o.w"], p[prefix + ".o.b"])


def _m_attention_nohead(q_in, kv_in, p, prefix, heads):
    return _orig["attention"](q_in, kv_in, p, prefix, 1)


MUTANTS = {
    "ln_no_beta": ("layer_norm", lambda x, w, b, eps: _orig["layer_norm"](x, w, 0 * b, eps)),
    "ln_unbiased_var": ("layer_norm", lambda x, w, b, eps: (x - x.mean(-1, keepdims=True)) /
                        np.sqrt(x.var(-1, ddof=1, keepdims=True) + eps) * w + b),
    "gelu_tanh": ("gelu", lambda x: 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))),
    "cos_unnormalised": ("cosine", lambda a, b: (a * b).sum(-1)),
    "softmax_no_norm": ("softmax", lambda s: np.exp(s - s.max(-1, keepdims=True))),
    "attn_scale": ("attention", _m_attention_scale),
    "attn_one_head": ("attention", _m_attention_nohead),
    "span_inclusive": ("span_mean", lambda x, sp: x[int(sp[0]): int(sp[1]) + 1].mean(0)),
    "span_shift": ("span_mean", lambda x, sp: x[int(sp[0]) + 1: int(sp[1]) + 1].mean(0)),
    "linear_no_bias": ("linear", lambda x, w, b: x @ w.T),
    "ffn_no_gelu": ("ffn", lambda x, p, pre: O.linear(O.linear(x, p[pre + ".ffn1.w"], p[pre + ".ffn1.b"]),
                                                      p[pre + ".ffn2.w"], p[pre + ".ffn2.b"])),
    "gate_sign": ("sigmoid", lambda x: _orig["sigmoid"](-x)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    case = synth.make_case(tiny_spec(seed=21, ln_random=True, gate_logit=0.7))
    lb, pb, ab = _brute(case)
    fn, impl = MUTANTS[name]
    monkeypatch.setattr(O, fn, impl)
    lo, po, ao = O.forward(case.weights, case.head, case.batch, table_reader(case))
    assert not np.allclose(lo, lb, rtol=1e-8, atol=1e-10), f"mutant {name} slipped through"
