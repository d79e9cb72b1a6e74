"""Seeded synthetic inputs for the JointSchemaHead forward pass.

This module only draws random numbers and lays them out; it holds none of the
head's arithmetic.  Tests, the benchmark and the smoke check use it to feed the
same inputs to the fp64 oracle and to the HIP library.

Shapes and structure follow the decision model's prompt layout (CoreML
conversion metadata page, "decision.prompt": a 36-token prefix, the state, the
schema block, an 18-token suffix whose last token is the global row) and the
span semantics of the same page ("decision.spans": half-open [start, end) token
spans; "option_order"; "question_types" noul=0, choice=1, score=2).  The
schema rendering (FIELD / ID / TYPE / INSTRUCTION / ALLOWED OPTIONS / OPTION j /
END FIELD) is represented by filler tokens around the spans, since the
tokenizer is not available.

bf16 tensors are numpy ``uint16`` arrays holding bf16 bit patterns; fp32 draws
are rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

NOUL, CHOICE, SCORE = 0, 1, 2
PREFIX_TOKENS = 36
SUFFIX_TOKENS = 18


# ----------------------------------------------------------------------------
# bf16 encoding (representation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    nan = np.isnan(x)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_bf16(ss: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.Philox(ss))
    x = g.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x).reshape(shape)


# ----------------------------------------------------------------------------
# head configuration and weights
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class HeadConfig:
    """Head hyper-parameters (joint_head_config.json keys as the pages list them)."""
    hidden_size: int = 4096
    width: int = 1024
    heads: int = 16
    routing_layers: int = 2
    layers: int = 4
    feedforward: int = 4096
    vocab_size: int = 248320
    num_types: int = 3
    ln_eps: float = 1e-5
    field_cross_attention: int = 0   # 1: field layers also cross-attend over the record's memory rows
    precision: int = 0               # arithmetic of the library (0 bf16, 1 fp32); the generated values do not depend on it


def weight_specs(c: HeadConfig) -> List[Tuple[str, Tuple[int, ...], str, int]]:
    """(name, shape, init kind, fan_in) for every named head tensor, in order.

    Linear weights use PyTorch's [out, in] layout.
    """
    H, D, F, T = c.hidden_size, c.width, c.feedforward, c.num_types
    s: List[Tuple[str, Tuple[int, ...], str, int]] = [
        ("ln_in.w", (H,), "ln_w", H), ("ln_in.b", (H,), "ln_b", H)]
    for n in ("mem", "q_base", "q_opt", "opt_ctx", "opt_lex", "glob"):
        s += [(n + ".w", (D, H), "lin", H), (n + ".b", (D,), "lin", H)]
    s += [("type_emb", (T, D), "lin", T), ("summary.w", (D,), "lin", D), ("summary.b", (1,), "lin", D)]
    stacks = [f"route.{r}" for r in range(c.routing_layers)] + [f"field.{l}" for l in range(c.layers)]
    for p in stacks:
        s += [(p + ".ln1.w", (D,), "ln_w", D), (p + ".ln1.b", (D,), "ln_b", D)]
        for m in ("q", "k", "v", "o"):
            s += [(f"{p}.{m}.w", (D, D), "lin", D), (f"{p}.{m}.b", (D,), "lin", D)]
        s += [(p + ".ln2.w", (D,), "ln_w", D), (p + ".ln2.b", (D,), "ln_b", D),
              (p + ".ffn1.w", (F, D), "lin", D), (p + ".ffn1.b", (F,), "lin", D),
              (p + ".ffn2.w", (D, F), "lin", F), (p + ".ffn2.b", (D,), "lin", F)]
    s += [("score.w1", (D, 4 * D), "lin", 4 * D), ("score.b1", (D,), "lin", 4 * D),
          ("score.w2", (D,), "lin", D), ("score.b2", (1,), "lin", D),
          ("gate_logit", (1,), "gate", 1), ("joint_scale", (1,), "scale", 1)]
    if c.field_cross_attention:   # appended, so every other tensor keeps its seed
        for l in range(c.layers):
            p = f"field.{l}"
            s += [(p + ".xln.w", (D,), "ln_w", D), (p + ".xln.b", (D,), "ln_b", D)]
            for m in ("xq", "xk", "xv", "xo"):
                s += [(f"{p}.{m}.w", (D, D), "lin", D), (f"{p}.{m}.b", (D,), "lin", D)]
    return s


def make_weights(c: HeadConfig, seed: int, ln_random: bool = False,
                 gate_logit: float = 0.0, joint_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Random-init head weights: N(0, 1/fan_in) for every Linear weight and bias,
    LayerNorm gamma=1 / beta=0 (or N(1, 0.1^2) / N(0, 0.1^2) with ``ln_random``),
    ``gate_logit`` and ``joint_scale`` as given (fp32).  All other tensors bf16."""
    specs = weight_specs(c)
    kids = np.random.SeedSequence(seed).spawn(len(specs))

    def one(i):
        name, shape, kind, fan_in = specs[i]
        if kind == "lin":
            return name, _normal_bf16(kids[i], shape, 1.0 / math.sqrt(fan_in))
        if kind == "ln_w":
            if ln_random:
                g = np.random.Generator(np.random.Philox(kids[i]))
                return name, f32_to_bf16_bits(1.0 + 0.1 * g.standard_normal(shape, dtype=np.float32))
            return name, f32_to_bf16_bits(np.ones(shape, np.float32))
        if kind == "ln_b":
            if ln_random:
                g = np.random.Generator(np.random.Philox(kids[i]))
                return name, f32_to_bf16_bits(0.1 * g.standard_normal(shape, dtype=np.float32))
            return name, f32_to_bf16_bits(np.zeros(shape, np.float32))
        if kind == "gate":
            return name, np.array([gate_logit], np.float32)
        if kind == "scale":
            return name, np.array([joint_scale], np.float32)
        raise ValueError(kind)

    with ThreadPoolExecutor(_threads()) as ex:
        return dict(ex.map(one, range(len(specs))))


def make_table(V: int, H: int, seed: int, std: float = 0.02) -> np.ndarray:
    """Lexical table [V, H] bf16, N(0, std^2), 64 row chunks each with its own stream."""
    out = np.empty((V, H), np.uint16)
    nch = 64
    kids = np.random.SeedSequence(seed).spawn(nch)
    bounds = [(V * i) // nch for i in range(nch + 1)]

    def one(i):
        a, b = bounds[i], bounds[i + 1]
        if b > a:
            out[a:b] = _normal_bf16(kids[i], (b - a, H), std)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(nch)))
    return out


# ----------------------------------------------------------------------------
# batches
# ----------------------------------------------------------------------------
@dataclass
class Batch:
    """One padded batch plus its span tables (record-relative positions)."""
    hidden: np.ndarray           # uint16 [B, L, H] (bf16), rows >= lengths[b] are padding
    lengths: np.ndarray          # int32 [B]
    q_offsets: np.ndarray        # int32 [B+1]  records -> questions
    q_type: np.ndarray           # int32 [NQ]
    q_span: np.ndarray           # int32 [NQ, 2]
    o_offsets: np.ndarray        # int32 [NQ+1] questions -> options
    o_span: np.ndarray           # int32 [NO, 2]
    o_ids: np.ndarray            # int32 [sum of option span lengths]
    hidden_dtype: str = "bf16"   # element type of the hidden bits: "bf16" | "f16"

    @property
    def B(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def L(self) -> int:
        return int(self.hidden.shape[1])

    @property
    def H(self) -> int:
        return int(self.hidden.shape[2])

    @property
    def NQ(self) -> int:
        return int(self.q_type.shape[0])

    @property
    def NO(self) -> int:
        return int(self.o_span.shape[0])

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)

    def varlen_hidden(self) -> np.ndarray:
        """Valid rows of every record packed back to back: [T, H]."""
        return np.ascontiguousarray(np.concatenate(
            [self.hidden[b, : self.lengths[b]] for b in range(self.B)], axis=0))

    def key_mask(self) -> np.ndarray:
        return (np.arange(self.L)[None, :] < self.lengths[:, None]).astype(np.uint8)

    def o_id_offsets(self) -> np.ndarray:
        ln = self.o_span[:, 1] - self.o_span[:, 0]
        return np.concatenate([[0], np.cumsum(ln)]).astype(np.int64)

    def record(self, b: int) -> "Batch":
        """Batch holding record ``b`` alone (unpadded)."""
        q0, q1 = int(self.q_offsets[b]), int(self.q_offsets[b + 1])
        o0, o1 = int(self.o_offsets[q0]), int(self.o_offsets[q1])
        ido = self.o_id_offsets()
        n = int(self.lengths[b])
        return Batch(hidden=np.ascontiguousarray(self.hidden[b: b + 1, :n]),
                     lengths=self.lengths[b: b + 1].copy(),
                     q_offsets=np.array([0, q1 - q0], np.int32),
                     q_type=self.q_type[q0:q1].copy(),
                     q_span=self.q_span[q0:q1].copy(),
                     o_offsets=(self.o_offsets[q0: q1 + 1] - o0).astype(np.int32),
                     o_span=self.o_span[o0:o1].copy(),
                     o_ids=self.o_ids[ido[o0]: ido[o1]].copy(),
                     hidden_dtype=self.hidden_dtype)


@dataclass
class CaseSpec:
    """Recipe for one synthetic workload."""
    name: str
    seed: int
    head: HeadConfig
    B: int
    L: Optional[int]                     # padded length; None = longest record
    lengths: Tuple[str, float, float]    # ("fixed", n, n) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    fields: str                          # "single" | "counts" | "ordered" | "random"
    counts: Tuple[int, int, int] = (0, 0, 0)      # noul, choice, score (fields == "counts")
    ordered: Tuple[Tuple[int, int], ...] = ()     # (type, options) in order (fields == "ordered")
    field_range: Tuple[int, int] = (1, 16)        # fields == "random"
    choice_opts: Tuple[int, int] = (2, 6)
    score_levels: int = 5
    instr_len: Tuple[int, int] = (8, 32)
    opt_len: Tuple[int, int] = (3, 16)
    pad_fill: str = "normal"             # "normal" | "nan"
    ln_random: bool = False
    gate_logit: float = 0.0
    joint_scale: float = 1.0
    prefix: int = PREFIX_TOKENS
    suffix: int = SUFFIX_TOKENS
    filler: Tuple[int, int, int, int, int] = (6, 4, 2, 2, 1)   # block, field header, options header, per option, end
    hidden_dtype: str = "bf16"           # "bf16" | "f16": rounding of the hidden draws


@dataclass
class Case:
    spec: CaseSpec
    weights: Dict[str, np.ndarray]
    table: np.ndarray
    batch: Batch

    @property
    def head(self) -> HeadConfig:
        return self.spec.head


def _draw_opts(rng, t, spec: CaseSpec) -> int:
    if t == NOUL:
        return 2
    if t == SCORE:
        return spec.score_levels
    return int(rng.integers(spec.choice_opts[0], spec.choice_opts[1] + 1))


def _draw_fields(rng, spec: CaseSpec) -> List[Tuple[int, int]]:
    if spec.fields == "counts":
        types = [NOUL] * spec.counts[0] + [CHOICE] * spec.counts[1] + [SCORE] * spec.counts[2]
        types = [types[i] for i in rng.permutation(len(types))]
        return [(t, _draw_opts(rng, t, spec)) for t in types]
    if spec.fields == "ordered":
        return list(spec.ordered)
    if spec.fields == "random":
        nf = int(rng.integers(spec.field_range[0], spec.field_range[1] + 1))
        out = []
        for _ in range(nf):
            t = int(rng.integers(0, 3))
            out.append((t, _draw_opts(rng, t, spec)))
        return out
    raise ValueError(spec.fields)


def _schema_block(rng, fields, spec: CaseSpec):
    """Lay out one schema block relative to its start.

    Returns (length, [(type, instr_span, [option_spans])]).  Filler counts stand
    in for the rendered header text (defaults): 6 before the first field; per
    field 4 (FIELD/ID/TYPE/INSTRUCTION) + instruction + 2 (ALLOWED OPTIONS) + per
    option 2 (OPTION j:) + option span, then 1 (END FIELD)."""
    f_block, f_head, f_opts, f_opt, f_end = spec.filler
    pos = f_block
    out = []
    for t, nopt in fields:
        pos += f_head
        il = int(rng.integers(spec.instr_len[0], spec.instr_len[1] + 1))
        ispan = (pos, pos + il)
        pos += il + f_opts
        ospans = []
        for _ in range(nopt):
            pos += f_opt
            ol = int(rng.integers(spec.opt_len[0], spec.opt_len[1] + 1))
            ospans.append((pos, pos + ol))
            pos += ol
        pos += f_end
        out.append((t, ispan, ospans))
    return pos, out


def _single_record_schema(rng):
    """The explicit single-record layout: prefix 0-35, state 36-95, schema 96-150,
    suffix 151-159; noul field (instruction [97,107), options [107,110) and
    [110,113)); choice field (instruction [114,124), three options of 4-8 tokens
    placed back to back from 124)."""
    f1 = (NOUL, (97, 107), [(107, 110), (110, 113)])
    pos = 124
    ospans = []
    for _ in range(3):
        ol = int(rng.integers(4, 9))
        ospans.append((pos, pos + ol))
        pos += ol
    f2 = (CHOICE, (114, 124), ospans)
    return [f1, f2]


def make_batch(spec: CaseSpec) -> Batch:
    root = np.random.SeedSequence(spec.seed)
    ss_w, ss_t, ss_s, ss_l, ss_i, ss_h = root.spawn(6)
    H, V = spec.head.hidden_size, spec.head.vocab_size
    rs = np.random.Generator(np.random.Philox(ss_s))
    rl = np.random.Generator(np.random.Philox(ss_l))
    ri = np.random.Generator(np.random.Philox(ss_i))

    kind, lo, hi = spec.lengths
    lengths = []
    for _ in range(spec.B):
        if kind == "fixed":
            lengths.append(int(lo))
        elif kind == "uniform":
            lengths.append(int(rl.integers(int(lo), int(hi) + 1)))
        elif kind == "loguniform":
            lengths.append(int(round(math.exp(rl.uniform(math.log(lo), math.log(hi))))))
        else:
            raise ValueError(kind)

    q_types, q_spans, o_counts, o_spans = [], [], [], []
    q_off = [0]
    for b in range(spec.B):
        n = lengths[b]
        if spec.fields == "single":
            fl = _single_record_schema(rs)
        else:
            for _attempt in range(10000):
                fields = _draw_fields(rs, spec)
                slen, fl = _schema_block(rs, fields, spec)
                if spec.prefix + 1 + slen + spec.suffix <= n:
                    break
            else:
                raise ValueError(f"schema does not fit a record of {n} tokens")
            start = n - spec.suffix - slen
            fl = [(t, (i0 + start, i1 + start), [(a + start, c + start) for a, c in os_])
                  for t, (i0, i1), os_ in fl]
        for t, isp, osp in fl:
            q_types.append(t)
            q_spans.append(isp)
            o_counts.append(len(osp))
            o_spans.extend(osp)
        q_off.append(len(q_types))

    o_span = np.array(o_spans, np.int32).reshape(-1, 2)
    nid = int((o_span[:, 1] - o_span[:, 0]).sum())
    o_ids = ri.integers(0, V, size=nid, dtype=np.int64).astype(np.int32)

    L = spec.L if spec.L is not None else max(lengths)
    if L < max(lengths):
        raise ValueError("padded length shorter than a record")
    hidden = np.empty((spec.B, L, H), np.uint16)
    kids = ss_h.spawn(spec.B)

    def fill(b):
        n = lengths[b]
        g = np.random.Generator(np.random.Philox(kids[b]))
        rows = L if spec.pad_fill == "normal" else n
        x = g.standard_normal(rows * H, dtype=np.float32).reshape(rows, H)
        if spec.hidden_dtype == "f16":
            hidden[b, :rows] = x.astype(np.float16).view(np.uint16)   # round to nearest even
        else:
            hidden[b, :rows] = f32_to_bf16_bits(x)
        if rows < L:
            hidden[b, rows:] = np.uint16(0x7E00 if spec.hidden_dtype == "f16" else 0x7FC0)   # quiet NaN

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(spec.B)))

    return Batch(hidden=hidden, lengths=np.array(lengths, np.int32),
                 q_offsets=np.array(q_off, np.int32), q_type=np.array(q_types, np.int32),
                 q_span=np.array(q_spans, np.int32).reshape(-1, 2),
                 o_offsets=np.concatenate([[0], np.cumsum(o_counts)]).astype(np.int32),
                 o_span=o_span, o_ids=o_ids, hidden_dtype=spec.hidden_dtype)


def make_case(spec: CaseSpec, with_table: bool = True) -> Case:
    root = np.random.SeedSequence(spec.seed)
    ss_w, ss_t = root.spawn(2)
    c = spec.head
    w = make_weights(c, int(ss_w.generate_state(1)[0]), ln_random=spec.ln_random,
                     gate_logit=spec.gate_logit, joint_scale=spec.joint_scale)
    table = make_table(c.vocab_size, c.hidden_size, int(ss_t.generate_state(1)[0])) if with_table else None
    return Case(spec=spec, weights=w, table=table, batch=make_batch(spec))


# ----------------------------------------------------------------------------
# the five workloads, and reduced variants for quick parity runs
# ----------------------------------------------------------------------------
def config_spec(i: int, **over) -> CaseSpec:
    """Workload ``i`` (0..4) with optional field overrides.

    0: single record, L=160, V=8192, a noul and a choice field (explicit layout).
    1: online-serving batch, B=8, L=4096, valid U{2048..4096}, 8 fields (3:3:2).
    2: long state, B=1, L=16384, fields noul, choice(4), choice(4), score(5).
    3: wide schema, B=4, L=8192, 32 fields (8 noul, 16 choice of 4-16, 8 score).
    4: H=5120, B=32, valid log-uniform [512, 16384], 1-16 random fields.
    """
    base = {
        0: CaseSpec("single-record", 1000, HeadConfig(vocab_size=8192), 1, 160, ("fixed", 160, 160), "single",
                    suffix=9),
        1: CaseSpec("online-serving", 1001, HeadConfig(), 8, 4096, ("uniform", 2048, 4096), "counts",
                    counts=(3, 3, 2), choice_opts=(2, 6)),
        2: CaseSpec("long-state", 1002, HeadConfig(), 1, 16384, ("fixed", 16384, 16384), "ordered",
                    ordered=((NOUL, 2), (CHOICE, 4), (CHOICE, 4), (SCORE, 5))),
        3: CaseSpec("wide-schema", 1003, HeadConfig(), 4, 8192, ("fixed", 8192, 8192), "counts",
                    counts=(8, 16, 8), choice_opts=(4, 16)),
        4: CaseSpec("heterogeneous-h5120", 1004, HeadConfig(hidden_size=5120), 32, None, ("loguniform", 512, 16384),
                    "random", field_range=(1, 16), choice_opts=(2, 8), pad_fill="nan"),
    }[i]
    head_over = {k: over.pop(k) for k in list(over) if k in HeadConfig.__dataclass_fields__}
    if head_over:
        over["head"] = replace(base.head, **head_over)
    return replace(base, **over)


def config_case(i: int, with_table: bool = True, **over) -> Case:
    return make_case(config_spec(i, **over), with_table=with_table)
