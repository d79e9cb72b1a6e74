"""fp64 CPU oracle of the JointSchemaHead forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the library path imports, calls or links
this module: only tests, the smoke check and the benchmark's CPU-baseline leg do.
It is a plain, slow, one-op-at-a-time definition of what the head computes,
record by record, touching only valid rows, in float64.  It shares no code with
the HIP library.

Sources (page titles as they appear in the collected pages):
  [P2] "Cloudflare 发布 9B 多模态决策模型 Clef-Flash 完整解析", §三 (the head in three
       steps: pool spans, 2 routing layers, joint scoring) and §四 (per-question
       softmax over the returned logits).
  [P3] "拆解 Clef-Flash 架构 ...", §3.2 (head config table: width 1024, 16 heads,
       routing_layers 2, layers 4, feedforward 4096; cosine prior with the output
       embedding; learnable gate).
  [P4] "clef-4bit ... JointSchemaHead 内部结构拆解", §三 steps 1-4 (span pooling,
       lexical vector, option query = three projections summed, evidence routing =
       cross-attention + FFN with residual, field vector = base + option-weighted
       summary + global vector + type embedding, 4 transformer layers across
       fields, logit = prior + gate * (joint_scale * cosine + residual MLP over
       [f, o, f*o, |f-o|])).
  [P5] CoreML conversion metadata of clef-flash, "decision.head" (LayerNorm over
       the hidden width into memory; global vector = last token; question and
       option vectors = mean of LayerNorm-ed rows over each span; lexical vector =
       mean of lm_head rows over the option span ids), "softmax" (per question,
       fp32, temperature 1), "option_order", "question_types".

Readings taken where the pages leave a step open (each is listed with its reason
in the design notes of this repository):
  * LayerNorm is affine with biased variance and eps = 1e-5 (input norm and every
    pre-norm); no norm after the memory projection or after either stack.
  * The global vector is the LayerNorm-ed row at the last valid position.
  * The lexical vector is the raw mean of table rows (no norm).
  * The prior is cos(e_k, q_q + g) in hidden space, with no scale.
  * The option query is W_c c + W_l e + W_qo q, three Linear maps with biases.
  * Routing layers are pre-LN cross-attention (16 heads of width/16, scale
    1/sqrt(head_dim), Q/K/V/O Linear with biases, keys = all valid rows of the
    record's memory) then a pre-LN GELU FFN, both residual; no self-attention
    among options.
  * The option-weighted summary is softmax over the question's options of
    (w_s . u_k + b_s) applied to the routed option vectors.
  * The global term of the field vector is its own Linear map of g.
  * Field layers are pre-LN self-attention across the record's fields (no mask,
    no positions) plus a pre-LN GELU FFN, both residual.
  * The residual MLP is Linear(4D -> D), exact-erf GELU, Linear(D -> 1).
  * cos(a, b) = a.b / (max(|a|, 1e-8) * max(|b|, 1e-8)).
  * argmax is the first index of the maximal logit.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Sequence, Tuple

import numpy as np
from scipy.special import erf

COS_EPS = 1e-8


# ----------------------------------------------------------------------------
# representation
# ----------------------------------------------------------------------------
def from_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def from_f16(bits: np.ndarray) -> np.ndarray:
    """IEEE half-precision bit patterns (uint16) -> float64, exactly."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def hidden_rows(batch, b: int, n: int) -> np.ndarray:
    """The first n hidden rows of record b as float64.  The backbone hands the
    head bf16 rows, or fp16 rows in the CoreML packaging (CoreML conversion
    metadata page, "decision.head": the head reads fp16 hidden in fp32)."""
    bits = batch.hidden[b, :n]
    return from_f16(bits) if getattr(batch, "hidden_dtype", "bf16") == "f16" else from_bf16(bits)


def load_params(weights: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """Convert named head tensors to float64 (bf16 tensors exactly; fp32 scalars as is)."""
    out = {}
    for k, v in weights.items():
        v = np.asarray(v)
        out[k] = from_bf16(v) if v.dtype == np.uint16 else v.astype(np.float64)
    return out


# ----------------------------------------------------------------------------
# elementary operations
# ----------------------------------------------------------------------------
def layer_norm(x: np.ndarray, w: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """Affine LayerNorm over the last axis, biased variance ([P5] decision.head)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * w + b


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """PyTorch-layout Linear: x @ w.T + b."""
    return x @ w.T + b


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def cosine(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Cosine similarity along the last axis with norms clamped below at 1e-8."""
    na = np.maximum(np.sqrt((a * a).sum(-1)), COS_EPS)
    nb = np.maximum(np.sqrt((b * b).sum(-1)), COS_EPS)
    return (a * b).sum(-1) / (na * nb)


def softmax(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis (max-subtracted)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def sigmoid(x: float) -> float:
    """Logistic function of the gate logit ([P4] step 4: the gate is the
    sigmoid of a learned scalar).  For x < 0 it is evaluated as
    e^x / (1 + e^x), so that no exponent of a positive argument is ever taken
    and every finite x (and -inf) gives a finite result."""
    if x >= 0.0:
        return 1.0 / (1.0 + math.exp(-x))
    z = math.exp(x)
    return z / (1.0 + z)


def attention(q_in: np.ndarray, kv_in: np.ndarray, p: Dict[str, np.ndarray], prefix: str,
              heads: int, names=("q", "k", "v", "o")) -> np.ndarray:
    """Multi-head attention of the rows of ``q_in`` over the rows of ``kv_in``:
    Q/K/V projections with biases, per-head softmax(Q K^T / sqrt(d)), V mix,
    concatenation over heads, output projection with bias.  ``names`` are the
    four projections' weight names under ``prefix``."""
    nq_, nk_, nv_, no_ = (prefix + "." + n for n in names)
    q = linear(q_in, p[nq_ + ".w"], p[nq_ + ".b"])
    k = linear(kv_in, p[nk_ + ".w"], p[nk_ + ".b"])
    v = linear(kv_in, p[nv_ + ".w"], p[nv_ + ".b"])
    D = q.shape[-1]
    d = D // heads
    outs = []
    for j in range(heads):
        sl = slice(j * d, (j + 1) * d)
        a = softmax(q[:, sl] @ k[:, sl].T / math.sqrt(d))
        outs.append(a @ v[:, sl])
    return linear(np.concatenate(outs, axis=1), p[no_ + ".w"], p[no_ + ".b"])


def ffn(x: np.ndarray, p: Dict[str, np.ndarray], prefix: str) -> np.ndarray:
    return linear(gelu(linear(x, p[prefix + ".ffn1.w"], p[prefix + ".ffn1.b"])),
                  p[prefix + ".ffn2.w"], p[prefix + ".ffn2.b"])


# ----------------------------------------------------------------------------
# the head's steps ([P4] §三 steps 1-4)
# ----------------------------------------------------------------------------
def routing_layer(u: np.ndarray, memory: np.ndarray, p: Dict[str, np.ndarray], prefix: str,
                  heads: int, eps: float) -> np.ndarray:
    """Evidence routing ([P4] step 2; [P2] §三): every option query attends over
    the whole memory of its record, then an FFN; both residual, pre-LN."""
    a = layer_norm(u, p[prefix + ".ln1.w"], p[prefix + ".ln1.b"], eps)
    u = u + attention(a, memory, p, prefix, heads)
    a = layer_norm(u, p[prefix + ".ln2.w"], p[prefix + ".ln2.b"], eps)
    return u + ffn(a, p, prefix)


def field_layer(f: np.ndarray, p: Dict[str, np.ndarray], prefix: str, heads: int,
                eps: float, memory: np.ndarray = None) -> np.ndarray:
    """Field transformer layer ([P4] step 3): fields of one record see each other.

    With ``memory`` (the decoder-layer reading of the field stack: [P4] §三
    step 3 and [P3] §3.2 call the field layers transformer decoder layers) a
    pre-LN cross-attention of the fields over the record's memory rows sits
    between the self-attention and the FFN, as in a standard decoder layer;
    its weights are ``xln`` (norm) and ``xq, xk, xv, xo`` (projections)."""
    a = layer_norm(f, p[prefix + ".ln1.w"], p[prefix + ".ln1.b"], eps)
    f = f + attention(a, a, p, prefix, heads)
    if memory is not None:
        a = layer_norm(f, p[prefix + ".xln.w"], p[prefix + ".xln.b"], eps)
        f = f + attention(a, memory, p, prefix, heads, names=("xq", "xk", "xv", "xo"))
    a = layer_norm(f, p[prefix + ".ln2.w"], p[prefix + ".ln2.b"], eps)
    return f + ffn(a, p, prefix)


def span_mean(x: np.ndarray, span: Sequence[int]) -> np.ndarray:
    """Mean of rows [start, end) ([P4] step 1; [P5] decision.head)."""
    s, e = int(span[0]), int(span[1])
    return x[s:e].mean(axis=0)


def forward_record(p: Dict[str, np.ndarray], head, hidden: np.ndarray,
                   q_type: np.ndarray, q_span: np.ndarray, o_offsets: np.ndarray,
                   o_span: np.ndarray, o_rows: List[np.ndarray], trace: Dict = None):
    """One record.

    hidden: float64 [n, H], valid rows only.  q_type/q_span: the record's
    questions; o_offsets: [nq+1] record-local CSR questions -> options;
    o_span: [no, 2]; o_rows[k]: float64 [len_k, H] lexical-table rows of option
    k's span ids.  Returns (logits [no], probs [no], argmax [nq])."""
    eps, heads = head.ln_eps, head.heads
    nq = len(q_type)
    no = len(o_span)
    opt_q = np.repeat(np.arange(nq), np.diff(o_offsets))

    # step 1: LayerNorm over the hidden width, memory, pooled vectors
    xh = layer_norm(hidden, p["ln_in.w"], p["ln_in.b"], eps)
    memory = linear(xh, p["mem.w"], p["mem.b"])
    qbar = np.stack([span_mean(xh, q_span[i]) for i in range(nq)])
    cbar = np.stack([span_mean(xh, o_span[k]) for k in range(no)])
    g = xh[hidden.shape[0] - 1]
    ebar = np.stack([o_rows[k].mean(axis=0) for k in range(no)])

    # lexical prior: cosine of the lexical vector with the question + global anchor
    prior = cosine(ebar, qbar[opt_q] + g[None, :])

    # option queries: context + lexical + question projections
    u = (linear(cbar, p["opt_ctx.w"], p["opt_ctx.b"]) + linear(ebar, p["opt_lex.w"], p["opt_lex.b"])
         + linear(qbar[opt_q], p["q_opt.w"], p["q_opt.b"]))

    # step 2: evidence routing
    u_layers = [u]
    for r in range(head.routing_layers):
        u = routing_layer(u, memory, p, f"route.{r}", heads, eps)
        u_layers.append(u)

    # step 3: field vectors, then the field transformer
    qv = linear(qbar, p["q_base.w"], p["q_base.b"])
    gp = linear(g, p["glob.w"], p["glob.b"])
    s = u @ p["summary.w"] + p["summary.b"][0]
    f = np.empty((nq, u.shape[1]))
    for i in range(nq):
        o0, o1 = int(o_offsets[i]), int(o_offsets[i + 1])
        beta = softmax(s[o0:o1])
        f[i] = qv[i] + beta @ u[o0:o1] + gp + p["type_emb"][int(q_type[i])]
    f0 = f.copy()
    cross = memory if getattr(head, "field_cross_attention", 0) else None
    for l in range(head.layers):
        f = field_layer(f, p, f"field.{l}", heads, eps, cross)

    # step 4: scoring
    fo = f[opt_q]
    joint_cos = cosine(u, fo)
    z = np.concatenate([fo, u, fo * u, np.abs(fo - u)], axis=1)
    mlp = gelu(linear(z, p["score.w1"], p["score.b1"])) @ p["score.w2"] + p["score.b2"][0]
    gate = sigmoid(float(p["gate_logit"][0]))
    logits = prior + gate * (float(p["joint_scale"][0]) * joint_cos + mlp)

    probs = np.empty(no)
    amax = np.empty(nq, np.int64)
    for i in range(nq):
        o0, o1 = int(o_offsets[i]), int(o_offsets[i + 1])
        probs[o0:o1] = softmax(logits[o0:o1])
        amax[i] = int(np.argmax(logits[o0:o1]))
    if trace is not None:
        trace.update(xh=xh, memory=memory, qbar=qbar, cbar=cbar, g=g, ebar=ebar, prior=prior,
                     u=u, u_layers=u_layers, f0=f0, f=f, joint_cos=joint_cos, mlp=mlp)
    return logits, probs, amax


def forward(weights: Dict[str, np.ndarray], head, batch, table_rows: Callable[[np.ndarray], np.ndarray],
            records: Sequence[int] = None, params: Dict[str, np.ndarray] = None):
    """Whole batch: records are independent, outputs are concatenated in
    question / option order.

    weights: named tensors (bf16 bit patterns or fp32); batch: a padded batch
    (hidden [B, L, H] bf16 or fp16 bits + lengths + span tables); table_rows(ids) returns
    the bf16 bit patterns of those lexical-table rows.  ``records`` restricts the
    evaluation to a subset (outputs for those records only)."""
    p = params if params is not None else load_params(weights)
    B = len(batch.lengths)
    recs = range(B) if records is None else records
    id_off = np.concatenate([[0], np.cumsum(batch.o_span[:, 1] - batch.o_span[:, 0])])
    L_all, P_all, A_all = [], [], []
    for b in recs:
        n = int(batch.lengths[b])
        q0, q1 = int(batch.q_offsets[b]), int(batch.q_offsets[b + 1])
        o0, o1 = int(batch.o_offsets[q0]), int(batch.o_offsets[q1])
        hid = hidden_rows(batch, b, n)
        o_rows = [from_bf16(table_rows(batch.o_ids[id_off[k]: id_off[k + 1]])) for k in range(o0, o1)]
        lg, pr, am = forward_record(p, head, hid, batch.q_type[q0:q1], batch.q_span[q0:q1],
                                    batch.o_offsets[q0: q1 + 1] - o0, batch.o_span[o0:o1], o_rows)
        L_all.append(lg)
        P_all.append(pr)
        A_all.append(am)
    return np.concatenate(L_all), np.concatenate(P_all), np.concatenate(A_all)

